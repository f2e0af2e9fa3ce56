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
// CDNA4 layout: 8 wave64s (or 4, with two workgroups per CU: two waves per SIMD either way),
// each owning 32 query rows whose Q and dO live in registers as MFMA B operands; everything fits
// in 256 VGPRs, so there is no AGPR traffic.  K and V tiles of BK keys are double-buffered in
// LDS, shared by the workgroup's waves and filled by direct global->LDS loads into unpadded,
// XOR-swizzled rows.  Per key tile a wave forms
// S^T = K Q^T and dP^T = V dO^T (keys x queries: each lane then owns one query column, so lse
// and delta are one register per lane), P^T and dS^T with exp2 on the f32 accumulators, and
// dQ += dS K with dS taken straight from the accumulator registers and K read transposed
// from LDS (ds_read_tr16_b64).  Tiles entirely outside a wave's mask are skipped by that wave;
// tiles entirely inside it skip the per-element mask.  Workgroups are dispatched
// longest-first (the last query blocks see the most keys under a causal mask).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

#ifndef ATTN_LDS_PREFETCH
#define ATTN_LDS_PREFETCH 3
#endif

template <int D, int BK, int SB_ = 1, int NW_ = 8>
struct DqCfg {
  static constexpr int SB = SB_;           // sub-blocks a tile is taken in
  static constexpr int NW = NW_;           // waves per workgroup (two waves per SIMD either way)
  static constexpr int BQ = 32 * NW;       // query rows per workgroup
  static constexpr int KB = BK / 32;       // 32-key blocks per step
  static constexpr int KST = BK / 16;      // 16-key MFMA k-steps of the dQ product
  static constexpr int KK = D / 16;        // MFMA k-steps over the head dim
  static constexpr int ND = D / 32;        // 32-wide blocks of the head dim
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int WIW = BK * CPR / (64 * NW);  // 16-byte global->LDS loads per wave per tile
  static_assert(BK * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(KB % SB == 0, "sub-blocks of whole 32-key blocks");
};

template <class TT, int D, int BK, int SB, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void dense_dq_kernel(const Params p) {
  using C = DqCfg<D, BK, SB, NW>;
  // [buffer][K, V][tile]: one array, so that a V read is the matching K read plus a constant.
  __shared__ __attribute__((aligned(16))) short kv_s[2][2][BK * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int BH = (p.cu ? p.nseq : p.B) * p.Hq;
  const int qbr = blockIdx.x / BH;
  // Packed sequences without a window: rotate the (sequence, head) index by the query block so
  // that one long sequence's blocks spread over the 8 XCDs (workgroups go round-robin over them).
  const int bh = (blockIdx.x % BH + (p.cu && p.window == 0 ? qbr : 0)) % BH;
  const int nqb = ((p.cu ? p.max_seqlen : p.Sq) + C::BQ - 1) / C::BQ;
  const int q0 = (nqb - 1 - qbr) * C::BQ;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
  const SeqView sv = seq_view(p.cu, b, p.Sq, p.Skv, p.Hq, p.max_seqlen);
  const int Sq = sv.Sq, Skv = sv.Skv;
  if (q0 >= Sq) return;  // a packed sequence shorter than the longest (whole workgroup)
  const int qw0 = q0 + 32 * w;
  const int off = Skv - Sq;

  // This wave's Q and dO rows as B operands B[k=d][n=query]; lse, delta and the allowed key
  // range [klo, khi] of the lane's query column.
  s8v qf[C::KK], dof[C::KK];
  const int qi = qw0 + lo;
  const bool qok = qi < Sq;
  {
    const int64_t o64 = ((sv.q0 + (qok ? qi : 0)) * p.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {
      qf[kk] = qok ? *(const s8v *)(p.q + o64 + 16 * kk) : s8v{};
      dof[kk] = qok ? *(const s8v *)(p.dout + o64 + 16 * kk) : s8v{};
    }
  }
  // The preprocess runs here, in the prologue: delta = rowsum(O * dO) of the lane's query row
  // (split over the two lane halves like the dO operand; one cross-half add completes it) and lse
  // with -inf mapped to +inf.  Both also go to the workspace (delta negated) for the dK/dV
  // kernel, which runs after this one.
  const int64_t li = sv.l0 + (int64_t)h * p.Sq + (qok ? qi : 0);
  float dsum = 0.f;
  if (qok) {
    const short *orow = p.o + ((sv.q0 + qi) * p.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {
      const s8v ov = *(const s8v *)(orow + 16 * kk);
#pragma unroll
      for (int e = 0; e < 8; e++) dsum += TT::tof(ov[e]) * TT::tof(dof[kk][e]);
    }
  }
  dsum += __shfl_xor(dsum, 32);
  const float lr = qok ? lse_fix(p.lse_in[li]) : __builtin_inff();
  const float ndr = -dsum;  // minus delta
  if (qok && hi == 0) {
    p.ndelta[li] = ndr;
    p.lse_ws[li] = lr;
  }
  // Starting value of every dP accumulator: minus delta of the lane's query column.
  f16v ndr16;
#pragma unroll
  for (int r = 0; r < 16; r++) ndr16[r] = ndr;
  const int klo = p.window > 0 ? qi + off - p.window + 1 : 0;
  const int khi = !qok ? klo - 1 : p.causal ? min(qi + off, Skv - 1) : Skv - 1;

  const Factors fac = factors(p);
  f16v acc[C::ND];  // dQ rows of this wave's 32 queries, [32-wide d block]
#pragma unroll
  for (int dn = 0; dn < C::ND; dn++) acc[dn] = f16v{};

  // Keys any row of this workgroup can see.
  const int qlast = min(q0 + C::BQ, Sq) - 1;
  int k_lo = 0, k_hi = Skv;
  if (p.window > 0) k_lo = max(0, q0 + off - p.window + 1);
  if (p.causal) k_hi = min(Skv, qlast + off + 1);
  const int kb_lo = k_lo / BK;
  const int kb_hi = k_hi > k_lo ? (k_hi + BK - 1) / BK : kb_lo;
  const int nsteps = kb_hi - kb_lo;
  const int wlast = min(qw0 + 32, Sq) - 1;  // last valid query row of this wave

  // Direct global->LDS tile loads: slot s of a tile is physical chunk s % CPR of row s / CPR and
  // holds logical chunk (s % CPR) ^ swz<D>(row).  The loads go through buffer resources that start
  // at the step's first key and end with the sequence, so key rows past the end read as zero
  // (their scores are masked); the lanes' byte offsets within a tile are computed once.
  uint32_t ld_off[C::WIW];
#pragma unroll
  for (int u = 0; u < C::WIW; u++) {
    const int s = (w * C::WIW + u) * 64 + lane, row = s / C::CPR, ch = (s % C::CPR) ^ swz<D>(row);
    ld_off[u] = (uint32_t)((row * p.Hkv * D + 8 * ch) * 2);
  }
  const uint32_t kv_lds = lds_addr(&kv_s[0][0][0]);
  auto issue = [&](int t, int buf) {
    const int k0 = (kb_lo + t) * BK;
    const int64_t e0 = ((sv.k0 + k0) * p.Hkv + g) * D;  // element (key k0, KV head g)
    const uint64_t nbytes = ((uint64_t)(Skv - k0) * p.Hkv - g) * D * 2;
    const i4v rk = buf_rsrc(p.k + e0, nbytes), rv = buf_rsrc(p.v + e0, nbytes);
#pragma unroll
    for (int u = 0; u < C::WIW; u++) {
      const uint32_t slot_b = 16 * (w * C::WIW + u) * 64;
      b2lds16_at(rk, ld_off[u], kv_lds + 2 * (2 * buf + 0) * BK * D + slot_b);
      b2lds16_at(rv, ld_off[u], kv_lds + 2 * (2 * buf + 1) * BK * D + slot_b);
    }
  };

  // Per-lane LDS offsets (elements): natural read of key row 32*kb + lo, logical chunk
  // 2*kk + hi; transposed read of rows 16*kst + 8*half + 4*hi + i16/4, columns 32*dn +
  // 16*(g16&1) + 4*(i16&3).  The swizzle has period 16 in the row, so rows lo and 32*kb + lo
  // share it while the two halves of a transposed read need their own.
  const int sw_lo = swz<D>(lo);
  const int tr_row = 4 * hi + (i16 >> 2);
  const int sw_tr0 = swz<D>(tr_row), sw_tr1 = swz<D>(tr_row + 8);
  auto nat_off = [&](int kb, int kk) { return (32 * kb + lo) * D + 8 * ((2 * kk + hi) ^ sw_lo); };
  auto tr_off = [&](int kst, int dn, int half) {
    const int ch = (4 * dn + 2 * (g16 & 1) + ((i16 & 3) >> 1)) ^ (half ? sw_tr1 : sw_tr0);
    return (16 * kst + 8 * half + tr_row) * D + 8 * ch + 4 * (i16 & 1);
  };

  // Per-lane byte offsets of both reads within a tile; each step adds its tile base once per
  // offset (one add the compiler cannot hoist as a sum per read out of the loop) and the
  // row-block offsets fold into the read instructions.
  uint32_t nat_lane[C::KK], tr_lane[C::ND][2];
#pragma unroll
  for (int kk = 0; kk < C::KK; kk++) nat_lane[kk] = 2 * nat_off(0, kk);
#pragma unroll
  for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
    for (int half = 0; half < 2; half++) tr_lane[dn][half] = 2 * tr_off(0, dn, half);

  if (nsteps > 0) issue(0, 0);
  wait_vm0();
  __syncthreads();

  for (int t = 0; t < nsteps; t++) {
    const int buf = t & 1;
    const int k0 = (kb_lo + t) * BK;
    const bool active = qw0 < Sq && (!p.causal || k0 <= wlast + off) &&
                        (p.window <= 0 || k0 + BK - 1 > qw0 + off - p.window);
    if (t + 1 < nsteps) issue(t + 1, buf ^ 1);
    if (active) {
      const bool full = (!p.causal || k0 + BK - 1 <= qw0 + off) && (p.window <= 0 || k0 > qw0 + 31 + off - p.window) &&
                        (k0 + BK <= Skv) && (qw0 + 32 <= Sq);
      const short *ks = kv_s[buf][0];
      // Read bases of this step's tile for the natural K/V reads; the sub-block and row-block
      // offsets fold into the reads' offset fields.
      uint32_t abk[C::KK];
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) abk[kk] = lds_base_add(lds_addr(ks), nat_lane[kk]);
      // The tile is taken as SB sub-blocks of KS = BK / SB keys, one after the other: each forms
      // S^T = K Q^T and dP^T = V dO^T (M = keys in 32-row blocks, N = this wave's 32 queries), the
      // softmax gradient, and dQ += dS K.  Fewer keys at a time hold fewer accumulators live.
#pragma unroll
      for (int sb = 0; sb < C::SB; sb++) {
        constexpr int KBS = C::KB / C::SB, KSTS = C::KST / C::SB;
        f16v s[KBS], dp[KBS];
#pragma unroll
        for (int kb = 0; kb < KBS; kb++) {
          s[kb] = f16v{};
          dp[kb] = ndr16;  // the products leave dP - delta
        }
        mfma_prio_hi();
        {
          // K and V rows are read PF k-steps ahead through a ring of registers (the read
          // latency hides behind the matrix core); the fences keep that order.
          constexpr int N = C::KK * KBS, PF = ATTN_LDS_PREFETCH;
          auto ldk = [&](int n) { return lds_rd16_at(abk[n / KBS] + (sb * KBS + n % KBS) * 64 * D); };
          auto ldv = [&](int n) { return lds_rd16_at(abk[n / KBS] + (sb * KBS + n % KBS) * 64 * D + BK * D * 2); };
          s8v rk[PF + 1], rv[PF + 1];
#pragma unroll
          for (int n = 0; n < PF; n++) {
            rk[n] = ldk(n);
            rv[n] = ldv(n);
          }
#pragma unroll
          for (int n = 0; n < N; n++) {
            if (n + PF < N) {
              rk[(n + PF) % (PF + 1)] = ldk(n + PF);
              rv[(n + PF) % (PF + 1)] = ldv(n + PF);
            }
            sched_fence();
            const int kk = n / KBS, kb = n % KBS;
            s[kb] = TT::mfma(rk[n % (PF + 1)], qf[kk], s[kb]);
            dp[kb] = TT::mfma(rv[n % (PF + 1)], dof[kk], dp[kb]);
          }
        }
        mfma_prio_lo();
        s8v da[KSTS], dl[KSTS];
        auto softmax_grad = [&](auto masked) {
#pragma unroll
          for (int kb = 0; kb < KBS; kb++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
              f4v ds;
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const int r = 4 * j + i;
                float x = exp2f_hw(s[kb][r] * fac.c - lr);
                if (decltype(masked)::value) {
                  const int kj = k0 + 32 * (sb * KBS + kb) + 8 * j + 4 * hi + i;
                  x = ((kj >= klo) & (kj <= khi)) ? x : 0.f;
                }
                ds[i] = ds_of<TT>(x, dp[kb][r], fac);
              }
              put4<TT>(da[2 * kb + (j >> 1)], dl[2 * kb + (j >> 1)], 4 * (j & 1), ds);
            }
        };
        if (full)
          softmax_grad(std::false_type{});
        else
          softmax_grad(std::true_type{});
        // dQ += dS K: B = K[k=key][n=d] read transposed from LDS, PF products ahead.
        mfma_prio_hi();
        {
          constexpr int N = KSTS * C::ND, PF = ATTN_LDS_PREFETCH;
          uint32_t ab[C::ND][2];
#pragma unroll
          for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
            for (int half = 0; half < 2; half++) ab[dn][half] = lds_base_add(lds_addr(ks), tr_lane[dn][half]);
          auto ld = [&](int n) {
            const int kg = sb * KSTS + n / C::ND, dn = n % C::ND;
            return cat8(lds_tr4_at(ab[dn][0] + kg * 32 * D), lds_tr4_at(ab[dn][1] + kg * 32 * D));
          };
          s8v ring[PF + 1];
#pragma unroll
          for (int n = 0; n < PF; n++) ring[n] = ld(n);
#pragma unroll
          for (int n = 0; n < N; n++) {
            if (n + PF < N) ring[(n + PF) % (PF + 1)] = ld(n + PF);
            sched_fence();
            const int kst = n / C::ND, dn = n % C::ND;
            acc[dn] = TT::mfma(da[kst], ring[n % (PF + 1)], acc[dn]);
            if (TT::SPLIT) acc[dn] = TT::mfma(dl[kst], ring[n % (PF + 1)], acc[dn]);
          }
        }
        mfma_prio_lo();
      }
    }
    wait_vm0();
    __syncthreads();  // next tile landed; this tile consumed
  }

  // Epilogue: dq = scale * acc, cast once.  Row m of the accumulator is query qw0 + m.
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int qr = qw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (qr < Sq) {
      short *row = p.dq + ((sv.q0 + qr) * p.Hq + h) * D + lo;
#pragma unroll
      for (int dn = 0; dn < C::ND; dn++) row[32 * dn] = TT::cvt_out(acc[dn][r] * fac.dq);
    }
  }
}

template <class TT, int D, int BK, int SB, int NW>
static hipError_t launch_dq_t(const Params &p, hipStream_t st) {
  using C = DqCfg<D, BK, SB, NW>;
  const int nqb = ((p.cu ? p.max_seqlen : p.Sq) + C::BQ - 1) / C::BQ;
  const int64_t blocks = (int64_t)nqb * (p.cu ? p.nseq : p.B) * p.Hq;
  if (blocks < 1) return hipSuccess;
  launch((dense_dq_kernel<TT, D, BK, SB, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

#ifndef ATTN_DQ128_BK
#define ATTN_DQ128_BK 64
#endif
#ifndef ATTN_DQ128_SB
#define ATTN_DQ128_SB 2
#endif

template <int D, int BK, int SB, int NW>
static hipError_t launch_dq_arith(const Params &p, int arith, hipStream_t st) {
  return arith == ARITH_BF16 ? launch_dq_t<BF16, D, BK, SB, NW>(p, st)
         : arith == ARITH_F16B ? launch_dq_t<F16B, D, BK, SB, NW>(p, st)
                               : launch_dq_t<F16, D, BK, SB, NW>(p, st);
}

hipError_t launch_dense_dq(const Params &p, int arith, hipStream_t st) {
  // At D = 128, 64-key tiles are taken as two 32-key sub-blocks, so that the S/dP accumulators of
  // one sub-block (and, for bf16, dS as hi + lo halves) fit in 256 VGPRs without spilling.
  // Waves per workgroup: 8 (256 query rows, one workgroup per CU) or 4 (128 rows, two workgroups
  // per CU, so that the two waves of a SIMD belong to different workgroups and do not meet at the
  // same barriers).  Measured: at D = 64 (twice the vector work per product) 4 waves take the
  // 2 x 8192 window-1024 dQ from 150 to 126 us; at D = 128 8 waves are 3.6% faster on the
  // 2 x 2048 causal call and even on 16K GQA, and 4 waves 3% faster on packed sequences.
  constexpr int BK = ATTN_DQ128_BK, SB = ATTN_DQ128_SB;
  if (p.Dqk == 128)
    return p.cu ? launch_dq_arith<128, BK, SB, 4>(p, arith, st) : launch_dq_arith<128, BK, SB, 8>(p, arith, st);
  if (p.Dqk == 64) return launch_dq_arith<64, 64, 1, 4>(p, arith, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
