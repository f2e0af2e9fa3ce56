// dense_dq.hip -- dQ of the dense (causal / sliding-window / full) backward.
//
// On the TileOPs PR #2281 page the KV-block-owned kernel also forms each step's dQ partial and
// settles it with an f32 add into a global accumulator that a landing pass later scales and
// casts ("TileFoundry Description", the Tiled program).  On MI355X that reduction is the
// bottleneck: f32 global atomics retire at about 1.36 TB/s of payload whatever their scope
// (measured), so the ~570 MB of dQ partials of the 2x2048x32x128 causal call alone would take
// ~420 us.  This kernel therefore owns dQ instead: one workgroup per (batch, head, 256 query
// rows) walks the key blocks its rows can see, recomputes S and dP for them, and writes dQ
// once, scaled and cast -- no atomics, no f32 workspace, no landing pass, deterministic.  The
// price is recomputing two of the five products (S and dP): 14*D instead of 10*D MFMA flops
// per (query, key) pair over the two kernels.
//
// CDNA4 layout: 4 wave64s, each owns 64 query rows whose Q and dO live in registers as MFMA
// B operands; K and V tiles of 32 keys are double-buffered in LDS and shared by the 4 waves.
// Per key tile a wave forms S^T = K Q^T and dP^T = V dO^T (keys x queries: each lane then owns
// one query column, so lse and delta are one register per lane), P^T and dS^T with exp2 on the
// f32 accumulators, and dQ += dS K with dS taken straight from the accumulator registers and K
// read transposed from LDS (ds_read_tr16_b64).  Tiles entirely outside a wave's mask are skipped
// by that wave; tiles entirely inside it skip the per-element mask.  Workgroups are dispatched
// longest-first (the last query blocks see the most keys under a causal mask).
#include "common.h"
#include "kernels.h"

namespace attn {

template <int D>
struct DqCfg {
  static constexpr int BK = 32;               // keys per step
  static constexpr int BQ = 256;              // query rows per workgroup (64 per wave)
  static constexpr int KK = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int PITCH = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BK * CPR / 256;  // 16-byte chunks per thread per K (or V) tile
  static_assert((BK * CPR) % 256 == 0, "tile must split evenly over 256 threads");
};

template <class TT, int D>
__global__ __launch_bounds__(256, 1) void dense_dq_kernel(const Params p) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) short k_s[2][C::BK * C::PITCH];
  __shared__ __attribute__((aligned(16))) short v_s[2][C::BK * C::PITCH];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int BH = p.B * p.Hq;
  const int bh = blockIdx.x % BH, qbr = blockIdx.x / BH;
  const int nqb = (p.Sq + C::BQ - 1) / C::BQ;
  const int q0 = (nqb - 1 - qbr) * C::BQ;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
  const int qw0 = q0 + 64 * w;
  const int off = p.Skv - p.Sq;

  // This wave's Q and dO rows as B operands B[k=d][n=query]; lse and delta of the lane's query.
  s8v qf[2][C::KK], dof[2][C::KK];
  float lr[2], dr[2];
#pragma unroll
  for (int nq = 0; nq < 2; nq++) {
    const int qi = qw0 + 32 * nq + lo;
    const bool ok = qi < p.Sq;
    const int64_t o64 = ((int64_t)(b * p.Sq + (ok ? qi : 0)) * p.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {
      qf[nq][kk] = ok ? *(const s8v *)(p.q + o64 + 16 * kk) : s8v{};
      dof[nq][kk] = ok ? *(const s8v *)(p.dout + o64 + 16 * kk) : s8v{};
    }
    const int64_t li = ((int64_t)b * p.Hq + h) * p.Sq + (ok ? qi : 0);
    lr[nq] = ok ? lse_fix(p.lse[li]) : __builtin_inff();
    dr[nq] = ok ? p.delta[li] : 0.f;
  }

  f16v acc[2][C::ND];
#pragma unroll
  for (int nq = 0; nq < 2; nq++)
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++) acc[nq][dn] = f16v{};

  // Keys any row of this workgroup can see.
  const int qlast = min(q0 + C::BQ, p.Sq) - 1;
  int k_lo = 0, k_hi = p.Skv;
  if (p.window > 0) k_lo = max(0, q0 + off - p.window + 1);
  if (p.causal) k_hi = min(p.Skv, qlast + off + 1);
  const int kb_lo = k_lo / C::BK;
  const int kb_hi = k_hi > k_lo ? (k_hi + C::BK - 1) / C::BK : kb_lo;
  const int nsteps = kb_hi - kb_lo;
  const int wlast = min(qw0 + 64, p.Sq) - 1;  // last valid query row of this wave

  s8v rk[C::CPT], rv[C::CPT];
  auto fetch = [&](int t) {
    const int k0 = (kb_lo + t) * C::BK;
#pragma unroll
    for (int u = 0; u < C::CPT; u++) {
      const int c = tid + 256 * u, row = c / C::CPR, ch = c % C::CPR;
      const int kj = k0 + row;
      if (kj < p.Skv) {
        const int64_t o64 = ((int64_t)(b * p.Skv + kj) * p.Hkv + g) * D + 8 * ch;
        rk[u] = *(const s8v *)(p.k + o64);
        rv[u] = *(const s8v *)(p.v + o64);
      } else {
        rk[u] = s8v{};
        rv[u] = s8v{};
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::CPT; u++) {
      const int c = tid + 256 * u, row = c / C::CPR, ch = c % C::CPR;
      *(s8v *)&k_s[buf][row * C::PITCH + 8 * ch] = rk[u];
      *(s8v *)&v_s[buf][row * C::PITCH + 8 * ch] = rv[u];
    }
  };

  if (nsteps > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; t++) {
    const int buf = t & 1;
    const int k0 = (kb_lo + t) * C::BK;
    if (t + 1 < nsteps) fetch(t + 1);
    const bool active = qw0 < p.Sq && (!p.causal || k0 <= wlast + off) &&
                        (p.window <= 0 || k0 + C::BK - 1 > qw0 + off - p.window);
    if (active) {
      const bool full = (!p.causal || k0 + C::BK - 1 <= qw0 + off) &&
                        (p.window <= 0 || k0 > qw0 + 63 + off - p.window) && (k0 + C::BK <= p.Skv) &&
                        (qw0 + 64 <= p.Sq);
      const short *ks = k_s[buf];
      const short *vs = v_s[buf];
      // S^T = K Q^T and dP^T = V dO^T: M = 32 keys, N = 2 x 32 queries.
      f16v s[2] = {f16v{}, f16v{}}, dp[2] = {f16v{}, f16v{}};
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) {
        const s8v ak = *(const s8v *)&ks[lo * C::PITCH + 16 * kk + 8 * hi];
        const s8v av = *(const s8v *)&vs[lo * C::PITCH + 16 * kk + 8 * hi];
#pragma unroll
        for (int nq = 0; nq < 2; nq++) {
          s[nq] = TT::mfma(ak, qf[nq][kk], s[nq]);
          dp[nq] = TT::mfma(av, dof[nq][kk], dp[nq]);
        }
      }
      // dS^T = P^T (dP^T - delta); each lane owns one query column.
      s8v da[2][2];  // dS as MFMA A operand A[m=query][k=key], [query block][16-key step]
      s8v dl[2][2];  // low half of dS when TT::SPLIT
#pragma unroll
      for (int nq = 0; nq < 2; nq++) {
        const int qi = qw0 + 32 * nq + lo;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          float x = exp2f_hw(s[nq][r] * p.c - lr[nq]);
          if (!full) {
            const int kj = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = kj < p.Skv && qi < p.Sq && (!p.causal || kj <= qi + off) &&
                            (p.window <= 0 || kj > qi + off - p.window);
            x = ok ? x : 0.f;
          }
          const float ds = x * (dp[nq][r] - dr[nq]);
          const short dh = TT::cvt(ds);
          da[nq][r >> 3][r & 7] = dh;
          dl[nq][r >> 3][r & 7] = TT::SPLIT ? TT::cvt(ds - TT::tof(dh)) : (short)0;
        }
      }
      // dQ += dS K: B = K[k=key][n=d] read transposed from LDS.
#pragma unroll
      for (int kstep = 0; kstep < 2; kstep++) {
#pragma unroll
        for (int dn = 0; dn < C::ND; dn++) {
          const short *bp = &ks[(16 * kstep + 4 * hi + (i16 >> 2)) * C::PITCH + 32 * dn + 16 * (g16 & 1) + 4 * (i16 & 3)];
          const s8v bb = cat8(lds_tr4(bp), lds_tr4(bp + 8 * C::PITCH));
          acc[0][dn] = TT::mfma(da[0][kstep], bb, acc[0][dn]);
          acc[1][dn] = TT::mfma(da[1][kstep], bb, acc[1][dn]);
          if (TT::SPLIT) {
            acc[0][dn] = TT::mfma(dl[0][kstep], bb, acc[0][dn]);
            acc[1][dn] = TT::mfma(dl[1][kstep], bb, acc[1][dn]);
          }
        }
      }
    }
    if (t + 1 < nsteps) stash(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: dq = scale * acc, cast once.
#pragma unroll
  for (int nq = 0; nq < 2; nq++)
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int qi = qw0 + 32 * nq + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qi < p.Sq) p.dq[((int64_t)(b * p.Sq + qi) * p.Hq + h) * D + 32 * dn + lo] = TT::cvt(acc[nq][dn][r] * p.scale);
      }
}

template <class TT, int D>
static hipError_t launch_dq_t(const Params &p, hipStream_t st) {
  const int nqb = (p.Sq + DqCfg<D>::BQ - 1) / DqCfg<D>::BQ;
  const int64_t blocks = (int64_t)nqb * p.B * p.Hq;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((dense_dq_kernel<TT, D>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_dense_dq(const Params &p, bool bf16, hipStream_t st) {
  if (p.Dqk == 128) return bf16 ? launch_dq_t<BF16, 128>(p, st) : launch_dq_t<F16, 128>(p, st);
  if (p.Dqk == 64) return bf16 ? launch_dq_t<BF16, 64>(p, st) : launch_dq_t<F16, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
