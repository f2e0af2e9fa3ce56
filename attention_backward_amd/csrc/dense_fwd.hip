// dense_fwd.hip -- the forward pass that produces the O and base-2 lse the backward consumes.
//
// The step before the backward.  The TileOPs PR #2281 page's programs take O and lse from a
// forward, and its Reference program defines lse in base 2 over scores scaled by
// c = scale * log2(e).  For each query row i and head h, over the keys j that row may see:
//   lse_i = log2 sum_j 2^(s_ij c),  o_i = sum_j 2^(s_ij c - lse_i) v_j,  s_ij = q_i . k_j;
// a row with no allowed key gets o = 0 and lse = -inf.  The mask conventions (bottom-right
// causal alignment, a window of `window` keys ending at the diagonal, GQA head h reading KV head
// h / G) are the backward's.
//
// CDNA4 layout, as in the dQ kernel: one workgroup of 8 wave64s (two per SIMD) per (batch, head,
// 256 query rows); each wave owns 32 query rows whose Q lives in registers as MFMA B operands.
// K and V tiles of BK keys are double-buffered in LDS, shared by the 8 waves and filled by direct
// global->LDS loads into unpadded, XOR-swizzled rows.  Per tile a wave forms S^T = K Q^T (keys x
// queries, so each lane owns one query column and the running max and sum are one register per
// lane), P^T = exp2(S^T c - m) with the online-softmax rescale, and O^T += V^T P^T with P^T taken
// straight from the accumulator registers and V read transposed (ds_read_tr16_b64).  O^T then
// also has one query per lane, so the rescale is a per-lane multiply.  The running max moves only
// when a tile's max exceeds it by more than 8 (so P stays <= 2^8), which lets most tiles skip the
// rescale; the result is exact either way, O = O^T / l at the end.  Tiles outside a wave's mask
// are skipped by that wave; tiles fully inside it skip the per-element mask.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

#ifndef ATTN_FWD_PF
#define ATTN_FWD_PF 3  // LDS operand reads issued ahead of their products
#endif

template <int D, int BK>
struct FwdCfg {
  static constexpr int NW = 8;             // waves per workgroup
  static constexpr int BQ = 32 * NW;       // query rows per workgroup
  static constexpr int KB = BK / 32;       // 32-key blocks per tile
  static constexpr int KST = BK / 16;      // 16-key MFMA k-steps of the O product
  static constexpr int KK = D / 16;        // MFMA k-steps over the head dim
  static constexpr int ND = D / 32;        // 32-wide blocks of the head dim
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int WIW = BK * CPR / (64 * NW);  // 16-byte global->LDS loads per wave per tile
  static_assert(BK * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
};

template <class TT, int D, int BK>
__global__ __launch_bounds__(512, 1) void dense_fwd_kernel(const FwdParams p) {
  using C = FwdCfg<D, BK>;
  constexpr float NEG = -3.0e38f;  // "no key yet": finite, so differences of it stay finite
  __shared__ __attribute__((aligned(16))) short kv_s[2][2][BK * D];  // [buffer][K, V][tile]

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
  const int q0 = (nqb - 1 - qbr) * C::BQ;  // longest first under a causal mask
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
  const SeqView sv = seq_view(p.cu, b, p.Sq, p.Skv, p.Hq, p.max_seqlen);
  const int Sq = sv.Sq, Skv = sv.Skv;
  if (q0 >= Sq) return;  // a packed sequence shorter than the longest (whole workgroup)
  const int qw0 = q0 + 32 * w;
  const int off = Skv - Sq;

  // This wave's Q rows as B operands B[k=d][n=query] and the allowed key range [klo, khi] of the
  // lane's query column.
  s8v qf[C::KK];
  const int qi = qw0 + lo;
  const bool qok = qi < Sq;
  {
    const int64_t o64 = ((sv.q0 + (qok ? qi : 0)) * p.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) qf[kk] = qok ? *(const s8v *)(p.q + o64 + 16 * kk) : s8v{};
  }
  const int klo = p.window > 0 ? qi + off - p.window + 1 : 0;
  const int khi = !qok ? klo - 1 : p.causal ? min(qi + off, Skv - 1) : Skv - 1;

  // O^T accumulators: block dn, register r is d = 32 dn + 8 (r/4) + 4 hi + r%4, lane lo the query.
  f16v acc[C::ND];
#pragma unroll
  for (int dn = 0; dn < C::ND; dn++) acc[dn] = f16v{};
  float m_run = NEG;  // running max of s c over the row (both lane halves agree)
  float l_run = 0.f;  // sum of 2^(s c - m_run) over this lane half's keys

  // Keys any row of this workgroup can see.
  const int qlast = min(q0 + C::BQ, Sq) - 1;
  int k_lo = 0, k_hi = Skv;
  if (p.window > 0) k_lo = max(0, q0 + off - p.window + 1);
  if (p.causal) k_hi = min(Skv, qlast + off + 1);
  const int kb_lo = k_lo / BK;
  const int kb_hi = k_hi > k_lo ? (k_hi + BK - 1) / BK : kb_lo;
  const int nsteps = kb_hi - kb_lo;
  const int wlast = min(qw0 + 32, Sq) - 1;

  // Direct global->LDS tile loads: slot s of a tile is physical chunk s % CPR of row s / CPR and
  // holds logical chunk (s % CPR) ^ swz<D>(row).  Rows past the end are clamped to the last key
  // (their scores are masked).
  auto issue = [&](int t, int buf) {
    const int k0 = (kb_lo + t) * BK;
#pragma unroll
    for (int u = 0; u < C::WIW; u++) {
      const int slot0 = (w * C::WIW + u) * 64;
      const int s = slot0 + lane, row = s / C::CPR, ch = (s % C::CPR) ^ swz<D>(row);
      const int kj = min(k0 + row, Skv - 1);
      const int64_t o64 = ((sv.k0 + kj) * p.Hkv + g) * D + 8 * ch;
      g2lds16(p.k + o64, &kv_s[buf][0][slot0 * 8]);
      g2lds16(p.v + o64, &kv_s[buf][1][slot0 * 8]);
    }
  };

  // Per-lane LDS offsets (bytes): natural read of key row lo, logical chunk 2*kk + hi; transposed
  // read of rows 16*kst + 8*half + 4*hi + i16/4, columns 32*dn + 16*(g16&1) + 4*(i16&3).
  const int sw_lo = swz<D>(lo);
  const int tr_row = 4 * hi + (i16 >> 2);
  const int sw_tr0 = swz<D>(tr_row), sw_tr1 = swz<D>(tr_row + 8);
  uint32_t nat_lane[C::KK], tr_lane[C::ND][2];
#pragma unroll
  for (int kk = 0; kk < C::KK; kk++) nat_lane[kk] = 2 * (lo * D + 8 * ((2 * kk + hi) ^ sw_lo));
#pragma unroll
  for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int ch = (4 * dn + 2 * (g16 & 1) + ((i16 & 3) >> 1)) ^ (half ? sw_tr1 : sw_tr0);
      tr_lane[dn][half] = 2 * ((8 * half + tr_row) * D + 8 * ch + 4 * (i16 & 1));
    }

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
      uint32_t abk[C::KK];
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) abk[kk] = lds_base_add(lds_addr(kv_s[buf][0]), nat_lane[kk]);
      // The tile is taken as KB sub-blocks of 32 keys, one after the other, each a step of the
      // online softmax: fewer scores and P operands live at once.
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++) {
        // S^T = K Q^T: M = the sub-block's 32 keys, N = this wave's 32 queries; K rows read PF
        // k-steps ahead through a ring of registers.
        f16v s = f16v{};
        mfma_prio_hi();
        ring_pipeline<C::KK, ATTN_FWD_PF>([&](int kk) { return lds_rd16_at(abk[kk] + kb * 64 * D); },
                                [&](int kk, s8v kr) { s = TT::mfma(kr, qf[kk], s); });
        mfma_prio_lo();
        // Online softmax; register r is key k0 + 32 kb + 8 (r/4) + 4 hi + r%4.  P^T is packed as
        // the B operand of the O product: element e of pb[ks] is key 32 kb + 16 ks + 4 hi +
        // (e < 4 ? e : e + 4), the order the transposed V reads supply.
        s8v pb[2];
        auto softmax = [&](auto masked) {
          float tmax = NEG;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            float x = s[r];
            if (decltype(masked)::value) {
              const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              x = ((kj >= klo) & (kj <= khi)) ? x : NEG;
            }
            tmax = fmaxf(tmax, x);
          }
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
          const float tm = tmax > NEG ? tmax * p.c : NEG;  // the sub-block's max of s c over the row
          // Move the running max only when this sub-block would push P above 2^8.
          const bool up = tm > m_run + 8.f;
          if (__ballot(up)) {
            const float m_new = up ? tm : m_run;
            const float alpha = exp2f_hw(m_run - m_new);  // 1 where m stays, 0 on a row's first keys
            l_run *= alpha;
#pragma unroll
            for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
              for (int r = 0; r < 16; r++) acc[dn][r] *= alpha;
            m_run = m_new;
          }
#pragma unroll
          for (int r = 0; r < 16; r++) {
            float pv = exp2f_hw(s[r] * p.c - m_run);
            if (decltype(masked)::value) {
              const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              pv = ((kj >= klo) & (kj <= khi)) ? pv : 0.f;
            }
            l_run += pv;
            pb[r >> 3][r & 7] = TT::cvt(pv);
          }
        };
        if (full)
          softmax(std::false_type{});
        else
          softmax(std::true_type{});
        // O^T += V^T P^T: A = V^T[m = d][k = key] by transposed reads of the V tile, B = P^T.
        mfma_prio_hi();
        {
          uint32_t ab[C::ND][2];
#pragma unroll
          for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
            for (int half = 0; half < 2; half++)
              ab[dn][half] = lds_base_add(lds_addr(kv_s[buf][1]), tr_lane[dn][half]);
          ring_pipeline<2 * C::ND, ATTN_FWD_PF>(
              [&](int n) {
                const int kst = 2 * kb + n / C::ND, dn = n % C::ND;
                return cat8(lds_tr4_at(ab[dn][0] + kst * 32 * D), lds_tr4_at(ab[dn][1] + kst * 32 * D));
              },
              [&](int n, s8v vt) {
                const int dn = n % C::ND;
                acc[dn] = TT::mfma(vt, pb[n / C::ND], acc[dn]);
              });
        }
        mfma_prio_lo();
      }
    }
    wait_vm0();
    __syncthreads();  // next tile landed; this tile consumed
  }

  // o = O^T / l, lse = m + log2(l); a row with no allowed key gets o = 0 and lse = -inf.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qok) {
    short *row = p.o + ((sv.q0 + qi) * p.Hq + h) * D + 4 * hi;
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        s4v v;
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = TT::cvt(acc[dn][4 * j + i] * inv);
        *(s4v *)&row[32 * dn + 8 * j] = v;
      }
    if (hi == 0)
      p.lse[sv.l0 + (int64_t)h * p.Sq + qi] = l_tot > 0.f ? m_run + __builtin_amdgcn_logf(l_tot) : -__builtin_inff();
  }
}

template <class TT, int D, int BK>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t st) {
  const int nqb = ((p.cu ? p.max_seqlen : p.Sq) + FwdCfg<D, BK>::BQ - 1) / FwdCfg<D, BK>::BQ;
  const int64_t blocks = (int64_t)nqb * (p.cu ? p.nseq : p.B) * p.Hq;
  if (blocks < 1) return hipSuccess;
  launch((dense_fwd_kernel<TT, D, BK>), dim3((unsigned)blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

#ifndef ATTN_FWD128_BK
#define ATTN_FWD128_BK 64
#endif
#ifndef ATTN_FWD64_BK
#define ATTN_FWD64_BK 64
#endif

hipError_t launch_dense_fwd(const FwdParams &p, int D, bool bf16, hipStream_t st) {
  constexpr int B128 = ATTN_FWD128_BK, B64 = ATTN_FWD64_BK;
  if (D == 128) return bf16 ? launch_fwd_t<BF16, 128, B128>(p, st) : launch_fwd_t<F16, 128, B128>(p, st);
  if (D == 64) return bf16 ? launch_fwd_t<BF16, 64, B64>(p, st) : launch_fwd_t<F16, 64, B64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
