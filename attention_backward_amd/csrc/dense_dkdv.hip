// dense_dkdv.hip -- dK and dV of the dense (causal / sliding-window / full) backward.
//
// Ownership follows the Tiled program of the TileOPs PR #2281 page ("TileFoundry Description"):
// one workgroup owns a block of keys of one (batch, KV head), keeps it resident, walks the query
// blocks that can see it and accumulates dK and dV in registers; dK and dV leave the workgroup
// once, cast to the input dtype, with the softmax scale applied to dK at the end.  For GQA the
// workgroup walks all G query heads of its KV head for every query block, so dK/dV are written
// directly at Hkv heads with no Hq-shaped intermediate and no atomics (flash-linear-attention
// issue #8, the KV-head-owned kernel it proposes).
//
// CDNA4 layout of one workgroup (256 threads = 4 wave64s, 128 keys):
//   waves 0,1 ("P role")  own keys [k0, k0+64) and [k0+64, k0+128): hold those K rows in
//                         registers, form S = Q K^T on MFMA, P = exp2(S*c - lse) (masked), send P
//                         to the partner wave through LDS, and accumulate dV += P^T dO;
//   waves 2,3 ("dS role") own the same two key halves: hold V rows, form dP = dO V^T, read P,
//                         form dS = P (dP - delta) and accumulate dK += dS^T Q.
// Splitting the four products between two waves halves each wave's register footprint (one
// resident operand, one accumulator) so each wave can own 64 keys; every Q/dO byte read from
// LDS then feeds 64 rows of MFMA work.  P crosses to the partner wave in f32, so dS is formed
// from unrounded P and rounded once (for bf16, P and dS each enter their product as hi + lo).  Per step (one
// query block of BN rows, one head) each wave issues 2*BN*D/256 MFMAs of 32x32x16 (more with
// the bf16 split) in two phases separated by one barrier.
// Q and dO tiles are double-buffered in LDS; the next tile's global loads are issued at the
// top of a step and land in the other buffer at its end.  Causal / window tiles entirely
// outside the mask are never visited; tiles fully inside it skip the per-element mask.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int D, int BN>
struct DkdvCfg {
  static constexpr int BM = 128;               // keys per workgroup
  static constexpr int KK = D / 16;            // MFMA k-steps over the head dim
  static constexpr int ND = D / 32;            // 32-wide blocks of the head dim
  static constexpr int MB = BN / 32;           // 32-row query blocks per step
  static constexpr int KS = BN / 16;           // 16-query k-steps per step
  static constexpr int PITCH = D + 8;          // LDS row pitch (elements)
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int CPT = BN * CPR / 256;   // chunks per thread per tile
  static_assert((BN * CPR) % 256 == 0, "tile must split evenly over 256 threads");
};

template <class TT, int D, int BN>
__global__ __launch_bounds__(256, 1) void dense_dkdv_kernel(const Params p) {
  using C = DkdvCfg<D, BN>;
  __shared__ __attribute__((aligned(16))) short q_s[2][BN * C::PITCH];
  __shared__ __attribute__((aligned(16))) short do_s[2][BN * C::PITCH];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BN];
  __shared__ __attribute__((aligned(16))) float dl_s[2][BN];
  __shared__ f4v p_s[2][C::MB][2][4][64];  // f32 P: [key half][query block][key block][reg quarter][lane]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int role = w >> 1, kh = w & 1;
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int BH = p.B * p.Hkv;
  const int bg = blockIdx.x % BH, kb = blockIdx.x / BH;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int k0 = kb * C::BM;
  const int kbase = k0 + 64 * kh;
  const int off = p.Skv - p.Sq;

  // This wave's 64 K rows (P role) or V rows (dS role) as MFMA B operands: B[k=d][n=key].
  s8v kv[2][C::KK];
  {
    const short *src = role == 0 ? p.k : p.v;
#pragma unroll
    for (int nb = 0; nb < 2; nb++) {
      const int key = kbase + 32 * nb + lo;
      const bool ok = key < p.Skv;
      const short *row = src + ((int64_t)(b * p.Skv + (ok ? key : 0)) * p.Hkv + g) * D + 8 * hi;
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) kv[nb][kk] = ok ? *(const s8v *)(row + 16 * kk) : s8v{};
    }
  }

  f16v acc[2][C::ND];  // P role: dV, dS role: dK; [32-key block][32-wide d block]
#pragma unroll
  for (int nb = 0; nb < 2; nb++)
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++) acc[nb][dn] = f16v{};

  // Query rows that can see some key of this block.
  int q_lo = 0, q_hi = p.Sq;
  if (p.causal) q_lo = max(0, k0 - off);
  if (p.window > 0) q_hi = min(p.Sq, k0 + C::BM - 1 - off + p.window);
  const int qb_lo = q_lo / BN;
  const int qb_hi = q_hi > q_lo ? (q_hi + BN - 1) / BN : qb_lo;
  const int nsteps = (qb_hi - qb_lo) * p.G;

  s8v rq[C::CPT], rdo[C::CPT];
  float rl = 0.f, rd = 0.f;
  auto fetch = [&](int t) {
    const int q0 = (qb_lo + t / p.G) * BN;
    const int h = g * p.G + t % p.G;
#pragma unroll
    for (int u = 0; u < C::CPT; u++) {
      const int c = tid + 256 * u, row = c / C::CPR, ch = c % C::CPR;
      const int qi = q0 + row;
      if (qi < p.Sq) {
        const int64_t o64 = ((int64_t)(b * p.Sq + qi) * p.Hq + h) * D + 8 * ch;
        rq[u] = *(const s8v *)(p.q + o64);
        rdo[u] = *(const s8v *)(p.dout + o64);
      } else {
        rq[u] = s8v{};
        rdo[u] = s8v{};
      }
    }
    if (tid < BN) {
      const int qi = q0 + tid;
      if (qi < p.Sq) {
        const int64_t li = ((int64_t)b * p.Hq + h) * p.Sq + qi;
        rl = lse_fix(p.lse[li]);
        rd = p.delta[li];
      } else {
        rl = __builtin_inff();
        rd = 0.f;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::CPT; u++) {
      const int c = tid + 256 * u, row = c / C::CPR, ch = c % C::CPR;
      *(s8v *)&q_s[buf][row * C::PITCH + 8 * ch] = rq[u];
      *(s8v *)&do_s[buf][row * C::PITCH + 8 * ch] = rdo[u];
    }
    if (tid < BN) {
      lse_s[buf][tid] = rl;
      dl_s[buf][tid] = rd;
    }
  };

  if (nsteps > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; t++) {
    const int buf = t & 1;
    const int q0 = (qb_lo + t / p.G) * BN;
    if (t + 1 < nsteps) fetch(t + 1);
    const bool full = (!p.causal || k0 + C::BM - 1 <= q0 + off) && (p.window <= 0 || k0 > q0 + BN - 1 + off - p.window) &&
                      (q0 + BN <= p.Sq) && (k0 + C::BM <= p.Skv);
    const short *qs = q_s[buf];
    const short *dos = do_s[buf];

    // Phase 1: S = Q K^T (P role) or dP = dO V^T (dS role); M = queries, N = keys.
    f16v s[C::MB][2];
#pragma unroll
    for (int mb = 0; mb < C::MB; mb++) s[mb][0] = s[mb][1] = f16v{};
    {
      const short *asrc = role == 0 ? qs : dos;
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) {
#pragma unroll
        for (int mb = 0; mb < C::MB; mb++) {
          const s8v a = *(const s8v *)&asrc[(32 * mb + lo) * C::PITCH + 16 * kk + 8 * hi];
          s[mb][0] = TT::mfma(a, kv[0][kk], s[mb][0]);
          s[mb][1] = TT::mfma(a, kv[1][kk], s[mb][1]);
        }
      }
    }

    s8v pa[2][C::KS];  // P^T (P role) or dS^T (dS role) as MFMA A operands: A[m=key][k=query]
    s8v pl[2][C::KS];  // their low halves when TT::SPLIT
    if (role == 0) {
#pragma unroll
      for (int mb = 0; mb < C::MB; mb++) {
        f4v l4[4];
#pragma unroll
        for (int j = 0; j < 4; j++) l4[j] = *(const f4v *)&lse_s[buf][32 * mb + 8 * j + 4 * hi];
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
          s8v h0, h1, l0, l1;
          f4v pq[4];
#pragma unroll
          for (int r = 0; r < 16; r++) {
            float x = exp2f_hw(s[mb][nb][r] * p.c - l4[r >> 2][r & 3]);
            if (!full) {
              const int qi = q0 + 32 * mb + 8 * (r >> 2) + 4 * hi + (r & 3);
              const int kj = kbase + 32 * nb + lo;
              const bool ok = kj < p.Skv && qi < p.Sq && (!p.causal || kj <= qi + off) &&
                              (p.window <= 0 || kj > qi + off - p.window);
              x = ok ? x : 0.f;
            }
            pq[r >> 2][r & 3] = x;
            const short ph = TT::cvt(x);
            const short pl_ = TT::SPLIT ? TT::cvt(x - TT::tof(ph)) : (short)0;
            if (r < 8) {
              h0[r] = ph;
              l0[r] = pl_;
            } else {
              h1[r - 8] = ph;
              l1[r - 8] = pl_;
            }
          }
          pa[nb][2 * mb] = h0;
          pa[nb][2 * mb + 1] = h1;
          pl[nb][2 * mb] = l0;
          pl[nb][2 * mb + 1] = l1;
#pragma unroll
          for (int qq = 0; qq < 4; qq++) p_s[kh][mb][nb][qq][lane] = pq[qq];
        }
      }
    }
    __syncthreads();  // P visible to the dS-role waves

    // Phase 2: dV += P^T dO (P role) or dS = P (dP - delta), dK += dS^T Q (dS role).
    if (role == 1) {
#pragma unroll
      for (int mb = 0; mb < C::MB; mb++) {
        f4v d4[4];
#pragma unroll
        for (int j = 0; j < 4; j++) d4[j] = *(const f4v *)&dl_s[buf][32 * mb + 8 * j + 4 * hi];
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
          f4v pq[4];
#pragma unroll
          for (int qq = 0; qq < 4; qq++) pq[qq] = p_s[kh][mb][nb][qq][lane];
          s8v o0, o1, l0, l1;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const float ds = pq[r >> 2][r & 3] * (s[mb][nb][r] - d4[r >> 2][r & 3]);
            const short dh = TT::cvt(ds);
            const short dl = TT::SPLIT ? TT::cvt(ds - TT::tof(dh)) : (short)0;
            if (r < 8) {
              o0[r] = dh;
              l0[r] = dl;
            } else {
              o1[r - 8] = dh;
              l1[r - 8] = dl;
            }
          }
          pa[nb][2 * mb] = o0;
          pa[nb][2 * mb + 1] = o1;
          pl[nb][2 * mb] = l0;
          pl[nb][2 * mb + 1] = l1;
        }
      }
    }
    {
      // B operand: dO (P role) or Q (dS role) as B[k=query][n=d], read transposed from LDS.
      const short *bsrc = role == 0 ? dos : qs;
#pragma unroll
      for (int ks = 0; ks < C::KS; ks++) {
#pragma unroll
        for (int dn = 0; dn < C::ND; dn++) {
          const short *bp = &bsrc[(16 * ks + 4 * hi + (i16 >> 2)) * C::PITCH + 32 * dn + 16 * (g16 & 1) + 4 * (i16 & 3)];
          const s8v bb = cat8(lds_tr4(bp), lds_tr4(bp + 8 * C::PITCH));
          acc[0][dn] = TT::mfma(pa[0][ks], bb, acc[0][dn]);
          acc[1][dn] = TT::mfma(pa[1][ks], bb, acc[1][dn]);
          if (TT::SPLIT) {
            acc[0][dn] = TT::mfma(pl[0][ks], bb, acc[0][dn]);
            acc[1][dn] = TT::mfma(pl[1][ks], bb, acc[1][dn]);
          }
        }
      }
    }
    if (t + 1 < nsteps) stash(buf ^ 1);
    __syncthreads();  // next tile visible; P and this tile consumed
  }

  // Epilogue: dV (P role) or scale * dK (dS role), cast once, BSHD at the KV head.
  short *dst = role == 0 ? p.dv : p.dk;
  const float sc = role == 0 ? 1.f : p.scale;
#pragma unroll
  for (int nb = 0; nb < 2; nb++)
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int key = kbase + 32 * nb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key < p.Skv) dst[((int64_t)(b * p.Skv + key) * p.Hkv + g) * D + 32 * dn + lo] = TT::cvt(acc[nb][dn][r] * sc);
      }
}

template <class TT, int D, int BN>
static hipError_t launch_dkdv_t(const Params &p, hipStream_t st) {
  const int nkb = (p.Skv + DkdvCfg<D, BN>::BM - 1) / DkdvCfg<D, BN>::BM;
  const int64_t blocks = (int64_t)nkb * p.B * p.Hkv;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((dense_dkdv_kernel<TT, D, BN>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_dense_dkdv(const Params &p, bool bf16, hipStream_t st) {
  // bf16 carries dS as two halves (hi + lo), which needs more registers: it steps 32 query rows.
  if (p.Dqk == 128) return bf16 ? launch_dkdv_t<BF16, 128, 32>(p, st) : launch_dkdv_t<F16, 128, 64>(p, st);
  if (p.Dqk == 64) return bf16 ? launch_dkdv_t<BF16, 64, 32>(p, st) : launch_dkdv_t<F16, 64, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
