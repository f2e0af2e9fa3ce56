// dense_dkdv.hip -- dK and dV of the dense (causal / sliding-window / full) backward.
//
// Ownership follows the Tiled program of the TileOPs PR #2281 page ("TileFoundry Description"):
// one workgroup owns a block of keys of one (batch, KV head), keeps it resident, walks the query
// blocks that can see it and accumulates dK and dV in registers; dK and dV leave the workgroup
// once, cast to the input dtype, with the softmax scale applied to dK at the end.  For GQA the
// workgroup walks all G query heads of its KV head for every query block, so dK/dV are written
// directly at Hkv heads with no Hq-shaped intermediate and no atomics (flash-linear-attention
// issue #8, the KV-head-owned kernel it proposes).  Packed sequences without a window take the
// work-queue form below; with an even head group each key block is then split into two items
// (half the group's heads each), which store their f32 blocks into two separate Hkv-shaped slices
// that a landing pass adds in a fixed order and casts -- still no atomics, and deterministic.
//
// CDNA4 layout of one workgroup (512 threads = 8 wave64s, two per SIMD, 128 keys):
//   waves 0..3 ("P role")  own keys [k0 + 32w, +32): hold those K rows in registers as MFMA
//                          B operands, form S = Q K^T, P = exp2(S*c - lse) (masked), hand P to
//                          the partner wave through LDS, and accumulate dV += P^T dO;
//   waves 4..7 ("dS role") own the same four key groups: hold V rows, form dP = dO V^T, read
//                          P, form dS = P (dP - delta) and accumulate dK += dS^T Q.
// Each wave keeps one resident operand and one accumulator, so everything fits in 256 VGPRs
// (no AGPR traffic) and two waves share each SIMD.  P crosses as the fp16 operand of the dV
// product; in the bf16 split form it crosses in f32, so dS is formed from unrounded P and
// rounded once (P and dS then enter their products as hi + lo halves).
// Q/dO tiles (BN query rows of one head) are double-buffered in LDS and filled by direct
// global->LDS loads into unpadded, XOR-swizzled rows; lse and delta rows come the same way.
// P and dS are formed in the accumulator layout and fed to the next product as B operands
// directly; dO and Q enter that product transposed through ds_read_tr16_b64, which leaves dV^T
// and dK^T in the accumulators.  Causal / window tiles entirely outside the mask are never
// visited; tiles fully inside it skip the mask.  At D = 128 a workgroup per CU runs a fixed
// sequence of items, loading the next item's first tile during the current item's last step.
#include <type_traits>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {

#ifndef ATTN_LDS_PREFETCH
#define ATTN_LDS_PREFETCH 3
#endif

template <int D, int BN>
struct DkdvCfg {
  static constexpr int NW = 8;                 // waves per workgroup
  static constexpr int BM = 128;               // keys per workgroup (4 groups of 32)
  static constexpr int KK = D / 16;            // MFMA k-steps over the head dim
  static constexpr int ND = D / 32;            // 32-wide blocks of the head dim
  static constexpr int MB = BN / 32;           // 32-row query blocks per step
  static constexpr int KS = BN / 16;           // 16-query k-steps per step
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int WIW = BN * CPR / (64 * NW);  // 16-byte global->LDS loads per wave per tile
  static_assert(BN * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(BN <= 64, "lse/delta rows are loaded by one wave instruction each");
};

#ifndef ATTN_DKDV_SEQ
#define ATTN_DKDV_SEQ 1
#endif

#ifndef ATTN_P_HALF
#define ATTN_P_HALF 1
#endif

// LDS of one dK/dV workgroup.  P crosses from the P role to the dS role through it.  fp16: as
// the element-type operand the dV product already uses (half the bytes of f32; dS = P (dP -
// delta) then starts from that rounding, 2^-12 relative, next to the rounding of dS itself for
// the dK product; measured 2.7% faster).  bf16 (8-bit mantissa, hence the hi + lo operands): f32.
template <class TT, int D, int BN>
struct DkdvLds {
  static constexpr bool PH = ATTN_P_HALF && !TT::SPLIT;
  __attribute__((aligned(16))) short q_s[3][BN * D];  // Q of steps t-1, t, t+1
  __attribute__((aligned(16))) short do_s[2][BN * D];
  __attribute__((aligned(16))) float lse_s[2][64];
  __attribute__((aligned(16))) float dl_s[2][64];
  f4v p_s[PH ? 1 : 4][BN / 32][4][64];  // f32 P: [key group][query block][reg quarter][lane]
  s8v ph_s[PH ? 4 : 1][BN / 16][64];    // element-type P: [key group][k-step][lane]
};

// Geometry of one work item, uniform over the workgroup: key block kb = item / BH of (sequence or
// batch, KV head, part of the head group).  `rotate`: the one-workgroup-per-item order spreads
// packed sequences over the XCDs.
struct DkdvItem {
  int sp, g, h0, Gs, k0, Sq, Skv, off, qb_lo, qb_hi, nsteps;
  bool live;  // false: the key block starts past the end of its sequence (nothing to store)
  SeqView sv;
};

template <int BM, int BN>
__device__ __forceinline__ DkdvItem dkdv_geo(const Params &p, const int item, const bool rotate) {
  DkdvItem it;
  // hsplit items share a key block: part sp walks query heads [sp * Gs, (sp + 1) * Gs) of the KV
  // head's group and stores its finished f32 block into its own slice.
  const int BH = (p.cu ? p.nseq : p.B) * p.Hkv * p.hsplit;
  const int kb = item / BH;
  // Packed sequences without a window: rotate the (sequence, head) index by the key block.
  // Workgroups go round-robin over the 8 XCDs, so with (sequences x heads) a multiple of 8 every
  // block of one sequence would land on the same few XCDs, and one long sequence would leave the
  // rest idle (measured 3.4x slower).  Under a window, neighbouring key blocks share most of their
  // query rows and the plain order keeps more of them in one L2 (measured 25% faster).
  const int rot = rotate && p.cu && p.window == 0 ? kb : 0;
  const int bgs = (item % BH + rot) % BH;
  const int bg = bgs / p.hsplit;
  it.sp = bgs % p.hsplit;
  it.Gs = p.G / p.hsplit;
  it.g = bg % p.Hkv;
  it.h0 = it.g * p.G + it.sp * it.Gs;
  it.k0 = kb * BM;
  it.sv = seq_view(p.cu, bg / p.Hkv, p.Sq, p.Skv, p.Hq, p.max_seqlen);
  it.Sq = it.sv.Sq;
  it.Skv = it.sv.Skv;
  it.off = it.Skv - it.Sq;
  it.live = it.k0 < it.Skv;
  // Query rows that can see some key of this block.
  int q_lo = 0, q_hi = it.Sq;
  if (p.causal) q_lo = max(0, it.k0 - it.off);
  if (p.window > 0) q_hi = min(it.Sq, it.k0 + BM - 1 - it.off + p.window);
  it.qb_lo = q_lo / BN;
  it.qb_hi = q_hi > q_lo ? (q_hi + BN - 1) / BN : it.qb_lo;
  it.nsteps = it.live ? (it.qb_hi - it.qb_lo) * it.Gs : 0;
  return it;
}

// How a workgroup gets its items: one item per workgroup; a fixed sequence known in advance
// (the next item's first Q/dO tile then goes out at the start of the current item's last step,
// in flight during that step and the epilogue); or drawn from the work queue after each item.
enum { DKDV_ONE = 0, DKDV_SEQ = 1, DKDV_QUEUE = 2 };

// A workgroup runs the items item, next(item), next(next(item)), ... while they are below
// nitems; each next item's K/V rows are loaded after the current item's epilogue.  `down`: the
// query blocks are walked from the last one.
template <class TT, int D, int BN, int MODE, class Next>
__device__ __forceinline__ void dkdv_run(const Params &p, int item, const int nitems, Next next, const bool rotate,
                                         const bool down, DkdvLds<TT, D, BN> &L) {
  using C = DkdvCfg<D, BN>;
  constexpr bool PH = DkdvLds<TT, D, BN>::PH;
  auto &q_s = L.q_s;
  auto &do_s = L.do_s;
  auto &lse_s = L.lse_s;
  auto &dl_s = L.dl_s;
  auto &p_s = L.p_s;
  auto &ph_s = L.ph_s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = w >> 2, kgrp = w & 3;
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;

  // Step t of an item covers query block step_q0(t) / BN and head h0 + t % Gs.  With `down` the
  // walk starts at the last query block, so that the key blocks of one head running side by side
  // (which all end their walks at the sequence's end) read the same Q/dO tiles at about the same
  // time and share them through L2 (measured 3-6% faster on a 16K causal sequence; the
  // work-queue launch, whose neighbours are other sequences, keeps the upward walk: 1-2% faster
  // there).
  auto step_q0 = [&](const DkdvItem &it, int t) {
    return (down ? it.qb_hi - 1 - t / it.Gs : it.qb_lo + t / it.Gs) * BN;
  };

  // Direct global->LDS loads of a step's Q/dO tile and of its lse/delta rows, through buffer
  // resources that start at the step's first row and head and end with the sequence: rows past
  // Sq read as zero (the mask zeroes their scores).  The lanes' byte offsets within a tile are
  // computed once; a step only forms its resources (scalar work).  Step t of item `it` lands in
  // the buffers of the workgroup's running step count T: q_s[T % 3], do_s[T % 2].
  uint32_t ld_off[C::WIW];
#pragma unroll
  for (int u = 0; u < C::WIW; u++) {
    const int s = (w * C::WIW + u) * 64 + lane, row = s / C::CPR, ch = (s % C::CPR) ^ swz<D>(row);
    ld_off[u] = (uint32_t)((row * p.Hq * D + 8 * ch) * 2);
  }
  const uint32_t q_lds = lds_addr(&q_s[0][0]), do_lds = lds_addr(&do_s[0][0]);
  const uint32_t row_lds = lds_addr(w == 0 ? &lse_s[0][0] : &dl_s[0][0]);
  auto issue = [&](const DkdvItem &it, int t, int T) {
    const int qbuf = T % 3, buf = T & 1;
    const int q0 = step_q0(it, t);
    const int h = it.h0 + t % it.Gs;
    const int64_t e0 = ((it.sv.q0 + q0) * p.Hq + h) * D;  // element (row q0, head h)
    const uint64_t nbytes = ((uint64_t)(it.Sq - q0) * p.Hq - h) * D * 2;
    const i4v rq = buf_rsrc(p.q + e0, nbytes), rd = buf_rsrc(p.dout + e0, nbytes);
#pragma unroll
    for (int u = 0; u < C::WIW; u++) {
      const uint32_t slot_b = 16 * (w * C::WIW + u) * 64;
      b2lds16_at(rq, ld_off[u], q_lds + 2 * qbuf * BN * D + slot_b);
      b2lds16_at(rd, ld_off[u], do_lds + 2 * buf * BN * D + slot_b);
    }
    if (w < 2) {
      const int64_t li = it.sv.l0 + (int64_t)h * p.Sq + q0;
      const i4v rl = buf_rsrc((w == 0 ? p.lse : p.ndelta) + li, (uint64_t)(it.Sq - q0) * 4);
      b2lds4_at(rl, (uint32_t)min(lane, BN - 1) * 4, row_lds + 4 * 64 * buf);
    }
  };

  // This wave's 32 K rows (P role) or V rows (dS role) of an item as MFMA B operands
  // B[k=d][n=key] (rows past the sequence read as zero).
  s8v kv[C::KK];
  auto load_kv = [&](const DkdvItem &it) {
    // The resource starts at row k0, head g and ends with the sequence (nothing when the block
    // starts past it).
    const short *base = (role == 0 ? p.k : p.v) + ((int64_t)(it.sv.k0 + it.k0) * p.Hkv + it.g) * D;
    const __amdgpu_buffer_rsrc_t r = buf_rsrc_v(base, ((int64_t)(it.Skv - it.k0) * p.Hkv - it.g) * D * 2);
    const uint32_t off = (uint32_t)(((32 * kgrp + lo) * p.Hkv * D + 8 * hi) * 2);
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) kv[kk] = buf_load16(r, off + 32 * kk);
  };

  f16v acc[C::ND];  // P role: dV^T, dS role: dK^T; [32-wide d block], columns = this wave's keys

  // Per-lane LDS offsets (elements): natural read of query row 32*mb + lo, logical chunk
  // 2*kk + hi; transposed read of rows 16*ks + 8*half + 4*hi + i16/4, columns 32*dn +
  // 16*(g16&1) + 4*(i16&3).  The swizzle has period 16 in the row, so rows lo and 32*mb + lo
  // share it while the two halves of a transposed read need their own.
  const int sw_lo = swz<D>(lo);
  const int tr_row = 4 * hi + (i16 >> 2);
  const int sw_tr0 = swz<D>(tr_row), sw_tr1 = swz<D>(tr_row + 8);
  auto nat_off = [&](int mb, int kk) { return (32 * mb + lo) * D + 8 * ((2 * kk + hi) ^ sw_lo); };
  auto tr_off = [&](int ks, int dn, int half) {
    const int ch = (4 * dn + 2 * (g16 & 1) + ((i16 & 3) >> 1)) ^ (half ? sw_tr1 : sw_tr0);
    return (16 * ks + 8 * half + tr_row) * D + 8 * ch + 4 * (i16 & 1);
  };

  // The two roles run separate copies of the step loop (same trip count, same barriers), so that
  // registers live in one role's loop are not reserved in the other's.
  //   P role:  S = Q K^T; P = exp2(S c - lse) masked -> LDS and B operands; | barrier |
  //            dV^T += dO^T P; | barrier |
  //   dS role: dK^T += Q^T dS of the previous step; dP = dO V^T; | barrier | dS = P (dP - delta)
  //            from the partner's P; | barrier |
  // The dS role applies dK one step late (dS kept in registers, Q of step t-1 in the third Q
  // buffer), so it keeps the matrix core busy while its P-role partner on the same SIMD works
  // through the softmax.
  //
  // B operands of phase 2, P or dS, B[k=query][n=key], with their low halves when TT::SPLIT:
  // register 8*(ks%2)+e of block ks/2 is query 16*ks + 8*(e/4) + 4*hi + e%4, which matches the
  // columns the transposed read of the A operand supplies.
  // Registers 4 j .. 4 j + 3 of block mb.
  auto pack4 = [&](s8v *pa, s8v *pl, int mb, int j, f4v x) {
    put4<TT>(pa[2 * mb + (j >> 1)], pl[2 * mb + (j >> 1)], 4 * (j & 1), x);
  };
  // acc += A B with A[m=d][k=query] read transposed from the row-major tile `src`: acc holds
  // dV^T or dK^T (rows d, columns this wave's keys).  The LDS operands are read PF products ahead
  // through a ring of registers, so that the read latency hides behind the matrix core instead
  // of stalling it before every product.
  // Per-lane byte offsets of both reads within a tile; the step's tile base is added once per
  // offset and the row-block offsets fold into the read instructions.
  uint32_t tr_lane[C::ND][2], nat_lane[C::KK];
#pragma unroll
  for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
    for (int half = 0; half < 2; half++) tr_lane[dn][half] = 2 * tr_off(0, dn, half);
#pragma unroll
  for (int kk = 0; kk < C::KK; kk++) nat_lane[kk] = 2 * nat_off(0, kk);
  auto phase2 = [&](const s8v *pa, const s8v *pl, const short *src) {
    constexpr int N = C::KS * C::ND, PF = ATTN_LDS_PREFETCH;
    uint32_t ab[C::ND][2];
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
      for (int half = 0; half < 2; half++) ab[dn][half] = opaque(lds_addr(src) + tr_lane[dn][half]);
    auto ld = [&](int n) {
      const int ks = n / C::ND, dn = n % C::ND;
      return cat8(lds_tr4_at(ab[dn][0] + ks * 32 * D), lds_tr4_at(ab[dn][1] + ks * 32 * D));
    };
    s8v ring[PF + 1];
#pragma unroll
    for (int n = 0; n < PF; n++) ring[n] = ld(n);
#pragma unroll
    for (int n = 0; n < N; n++) {
      if (n + PF < N) ring[(n + PF) % (PF + 1)] = ld(n + PF);
      sched_fence();
      const int ks = n / C::ND, dn = n % C::ND;
      acc[dn] = TT::mfma(ring[n % (PF + 1)], pa[ks], acc[dn]);
      if (TT::SPLIT) acc[dn] = TT::mfma(ring[n % (PF + 1)], pl[ks], acc[dn]);
    }
  };
  // Phase 1 for M = the step's queries, N = this wave's keys, A rows from `src` (same ring).
  // Accumulates into s as given (the caller sets its starting value).
  auto phase1 = [&](f16v *s, const short *src) {
    constexpr int N = C::KK * C::MB, PF = ATTN_LDS_PREFETCH;
    uint32_t ab[C::KK];
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) ab[kk] = opaque(lds_addr(src) + nat_lane[kk]);
    auto ld = [&](int n) { return lds_rd16_at(ab[n / C::MB] + (n % C::MB) * 64 * D); };
    s8v ring[PF + 1];
#pragma unroll
    for (int n = 0; n < PF; n++) ring[n] = ld(n);
#pragma unroll
    for (int n = 0; n < N; n++) {
      if (n + PF < N) ring[(n + PF) % (PF + 1)] = ld(n + PF);
      sched_fence();
      const int kk = n / C::MB, mb = n % C::MB;
      s[mb] = TT::mfma(ring[n % (PF + 1)], kv[kk], s[mb]);
    }
  };
  const Factors fac = factors(p);

  DkdvItem cur = dkdv_geo<C::BM, BN>(p, item, rotate);
  if (MODE == DKDV_ONE && !cur.live) return;  // a packed sequence shorter than the longest
  load_kv(cur);
  int T = 0;  // steps run so far: buffer parity across items
  if (cur.nsteps > 0) issue(cur, 0, 0);
  wait_vm0();
  __syncthreads();

  for (;;) {
    const int nitem = MODE == DKDV_SEQ ? next(item) : nitems;
    const bool has_next = nitem < nitems;  // known in advance (DKDV_SEQ only)
    const int n = cur.nsteps;
    const int T0 = MODE == DKDV_ONE ? 0 : T;  // running step count at the item's first step
    const int kbase = cur.k0 + 32 * kgrp;
    // The range [qlo, qhi] of query rows allowed to see the lane's key.
    const int kj = kbase + lo;
    const int qlo = p.causal ? kj - cur.off : 0;
    const int qhi = kj >= cur.Skv ? qlo - 1
                    : p.window > 0 ? min(cur.Sq - 1, kj - cur.off + p.window - 1)
                                   : cur.Sq - 1;
    auto step_full = [&](int q0) {
      return (!p.causal || cur.k0 + C::BM - 1 <= q0 + cur.off) &&
             (p.window <= 0 || cur.k0 > q0 + BN - 1 + cur.off - p.window) && (q0 + BN <= cur.Sq) &&
             (cur.k0 + C::BM <= cur.Skv);
    };
    // The loads of step t + 1: the item's own next step, or at its last step the next item's
    // first.  A step ends by waiting for them; in the fixed item sequence the last step leaves the
    // next item's tile in flight (16K GQA: 6% faster), while the one-item launch waits at every
    // step (the conditional wait cost its D = 64 steps 8%).
    auto issue_next = [&](int t) {
      if (t + 1 < n) {
        issue(cur, t + 1, T0 + t + 1);
      } else if (has_next) {
        const DkdvItem nx = dkdv_geo<C::BM, BN>(p, nitem, rotate);
        if (nx.nsteps > 0) issue(nx, 0, T0 + t + 1);
      }
    };
    auto end_step = [&](int t) {
      if (MODE != DKDV_SEQ || t + 1 < n) wait_vm0();
      __syncthreads();
    };
#pragma unroll
    for (int dn = 0; dn < C::ND; dn++) acc[dn] = f16v{};

    if (role == 0) {
      for (int t = 0; t < n; t++) {
        const int buf = (T0 + t) & 1;
        const int q0 = step_q0(cur, t);
        issue_next(t);
        f16v s[C::MB] = {};
        mfma_prio_hi();
        phase1(s, q_s[(T0 + t) % 3]);
        mfma_prio_lo();
        s8v pa[C::KS], pl[C::KS];
        auto softmax = [&](auto masked) {
#pragma unroll
          for (int mb = 0; mb < C::MB; mb++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const f4v l4 = *(const f4v *)&lse_s[buf][32 * mb + 8 * j + 4 * hi];
              f4v pq;
#pragma unroll
              for (int i = 0; i < 4; i++) {
                float x = exp2f_hw(s[mb][4 * j + i] * fac.c - l4[i]);
                if (decltype(masked)::value) {
                  const int qi = q0 + 32 * mb + 8 * j + 4 * hi + i;
                  x = ((qi >= qlo) & (qi <= qhi)) ? x : 0.f;
                }
                pq[i] = x;
              }
              pack4(pa, pl, mb, j, pq);
              if (!PH) p_s[kgrp][mb][j][lane] = pq;
            }
          }
        };
        if (step_full(q0))
          softmax(std::false_type{});
        else
          softmax(std::true_type{});
        if (PH) {
#pragma unroll
          for (int ks = 0; ks < C::KS; ks++) ph_s[kgrp][ks][lane] = pa[ks];
        }
        __syncthreads();  // P visible to the dS-role waves
        phase2(pa, pl, do_s[buf]);  // dV^T += dO^T P
        end_step(t);  // next tile landed; P and this step's dO consumed
      }
    } else {
      s8v da[C::KS], dl[C::KS];  // dS of the previous step (B operands)
      for (int t = 0; t < n; t++) {
        const int buf = (T0 + t) & 1;
        issue_next(t);
        if (t > 0) phase2(da, dl, q_s[(T0 + t + 2) % 3]);  // dK^T += Q^T dS of step t-1
        // dP accumulators start from minus delta of their query rows (register 4 j + i of block
        // mb is row 32 mb + 8 j + 4 hi + i), so the products leave dP - delta in them.
        f16v s[C::MB];
#pragma unroll
        for (int mb = 0; mb < C::MB; mb++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const f4v d4 = *(const f4v *)&dl_s[buf][32 * mb + 8 * j + 4 * hi];
#pragma unroll
            for (int i = 0; i < 4; i++) s[mb][4 * j + i] = d4[i];
          }
        phase1(s, do_s[buf]);  // dP - delta = dO V^T - delta
        __syncthreads();  // P of this step visible
#pragma unroll
        for (int mb = 0; mb < C::MB; mb++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            f4v pq;
            if (PH) {
              const s8v ph = ph_s[kgrp][2 * mb + (j >> 1)][lane];
#pragma unroll
              for (int i = 0; i < 4; i++) pq[i] = TT::tof(ph[4 * (j & 1) + i]);
            } else {
              pq = p_s[kgrp][mb][j][lane];
            }
            f4v dsv;
#pragma unroll
            for (int i = 0; i < 4; i++) dsv[i] = ds_of<TT>(pq[i], s[mb][4 * j + i], fac);
            pack4(da, dl, mb, j, dsv);
          }
        end_step(t);  // next tile landed; P consumed
      }
      if (n > 0) phase2(da, dl, q_s[(T0 + n - 1) % 3]);
    }

    // Epilogue: dV (P role) or scale * dK (dS role), cast once, BSHD at the KV head.  The
    // accumulators hold the transposes: register 4 j + i of block dn is column d = 32 dn + 8 j +
    // 4 hi + i of key kbase + lo.
    if (p.hsplit > 1) {
      // Part sp of the head group stores its unscaled f32 block with plain stores into its own
      // slice [sp][tokens, Hkv, D]; the landing pass adds the slices in a fixed order.
      if (cur.live && kj < cur.Skv) {
        float *row = (role == 0 ? p.dv_acc : p.dk_acc) + (int64_t)cur.sp * p.acc_slice +
                     ((cur.sv.k0 + kj) * p.Hkv + cur.g) * D + 4 * hi;
#pragma unroll
        for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            *(f4v *)(row + 32 * dn + 8 * j) = f4v{acc[dn][4 * j], acc[dn][4 * j + 1], acc[dn][4 * j + 2], acc[dn][4 * j + 3]};
      }
    } else if (cur.live) {
      // The wave's 32 x D block goes through LDS so that the global stores are whole rows (16
      // lanes x 16 bytes per 256-byte row): staged row-major, 16-byte chunk c of row r at chunk
      // c ^ (r mod CPR).  Staging space, 32 D 2 bytes per wave, two waves per buffer: the two Q
      // buffers and the dO buffer not holding the next item's first tile, and the P exchange.
      __syncthreads();  // the dS role's last product has read its Q buffer
      const float sc = role == 0 ? fac.dv : fac.dk;
      constexpr int WB = 32 * D * 2;  // bytes per wave
      static_assert(2 * WB <= (int)sizeof(q_s[0]) && 2 * WB <= (int)sizeof(p_s) + (int)sizeof(ph_s),
                    "staging space");
      const int rg = w >> 1;
      const uint32_t stg = (rg == 0   ? lds_addr(&q_s[(T0 + n + 2) % 3][0])
                            : rg == 1 ? lds_addr(&q_s[(T0 + n + 1) % 3][0])
                            : rg == 2 ? lds_addr(&do_s[(T0 + n + 1) & 1][0])
                                      : (PH ? lds_addr(&ph_s[0][0][0]) : lds_addr(&p_s[0][0][0][0]))) +
                           (w & 1) * WB;
      // Lane terms recomputed here (opaque) rather than hoisted out of the item loop, where they
      // would hold registers through every step.
      const int ln = (int)opaque((uint32_t)lane), lo_e = ln & 31, swl = lo_e & (C::CPR - 1);
      const uint32_t wr = stg + lo_e * D * 2 + 8 * (ln >> 5);
#pragma unroll
      for (int dn = 0; dn < C::ND; dn++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          s4v o;
#pragma unroll
          for (int i = 0; i < 4; i++) o[i] = TT::cvt_out(acc[dn][4 * j + i] * sc);
          const int c = 4 * dn + j;
          *(__attribute__((address_space(3))) s4v *)(size_t)(wr + ((c ^ swl) * 16)) = o;
        }
      {
        constexpr int RPI = 64 / C::CPR;  // rows per store instruction
        const int c = ln % C::CPR;
        short *dst = (role == 0 ? p.dv : p.dk) + (int64_t)cur.g * D + 8 * c;
#pragma unroll
        for (int u = 0; u < 32 / RPI; u++) {
          const int r = RPI * u + ln / C::CPR;
          const s8v v = *(__attribute__((address_space(3))) s8v *)(size_t)(stg + r * D * 2 + ((c ^ (r & (C::CPR - 1))) * 16));
          if (kbase + r < cur.Skv) *(s8v *)(dst + (int64_t)(cur.sv.k0 + kbase + r) * p.Hkv * D) = v;
        }
      }
    }
    if (MODE == DKDV_ONE) break;
    T += n;
    const int ni = MODE == DKDV_SEQ ? nitem : next(item);
    if (ni >= nitems) break;
    cur = dkdv_geo<C::BM, BN>(p, ni, rotate);
    item = ni;
    if ((MODE != DKDV_SEQ || n == 0) && cur.nsteps > 0) issue(cur, 0, T);  // not prefetched
    load_kv(cur);
    wait_vm0();
    __syncthreads();  // the item's first tile and K/V rows landed
  }
}

// One workgroup per item (items = the grid), or (SEQ) workgroup b of `grid` takes items in
// rounds: item b of round 0 and then with the order reversed every other round (keeping each
// item's XCD, b mod 8, when grid is a multiple of 8), so that the long key blocks at the front of
// the item order pair with the short ones at its end.
// D = 64 in the fp16 forms fits 128 VGPRs, i.e. four waves per SIMD: two workgroups per CU (the
// second bound is waves per SIMD).
template <class TT, int D, int BN, int MODE>
__global__ __launch_bounds__(512, (D == 64 && !TT::SPLIT && MODE == DKDV_ONE) ? 4 : 1) void dense_dkdv_kernel(
    const Params p, int nitems) {
  __shared__ DkdvLds<TT, D, BN> L;
  const int b = blockIdx.x, grid = gridDim.x;
  int r = 0;
  auto at = [&](int rr) {
    const int rev = grid % 8 == 0 ? 8 * (grid / 8 - 1 - b / 8) + b % 8 : grid - 1 - b;
    return rr * grid + ((rr & 1) ? rev : b);
  };
  dkdv_run<TT, D, BN, MODE>(p, b, nitems, [&](int) { return at(++r); }, true, true, L);
}

// Work-queue form: one workgroup per CU takes items in index order (key blocks longest first)
// from a counter that starts at zero, so a free CU always gets the next item whatever XCD it is
// on.  Thread 0 draws after each item and hands the id over through LDS; every workgroup leaves
// once the ids pass the item count.
template <class TT, int D, int BN>
__global__ __launch_bounds__(512, 1) void dense_dkdv_queue_kernel(const Params p, int nitems) {
  __shared__ DkdvLds<TT, D, BN> L;
  __shared__ int nid;
  auto next = [&](int) {
    if (threadIdx.x == 0) nid = atomicAdd(p.work, 1);
    __syncthreads();  // read before the item's next barrier; rewritten only after it
    return nid;
  };
  const int first = next(0);
  if (first < nitems) dkdv_run<TT, D, BN, DKDV_QUEUE>(p, first, nitems, next, false, false, L);
}

template <class TT, int D, int BN>
static hipError_t launch_dkdv_t(const Params &p, hipStream_t st) {
  const int nkb = ((p.cu ? p.max_seqlen : p.Skv) + DkdvCfg<D, BN>::BM - 1) / DkdvCfg<D, BN>::BM;
  const int64_t items = (int64_t)nkb * (p.cu ? p.nseq : p.B) * p.Hkv * p.hsplit;
  if (items < 1) return hipSuccess;
  if (items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (p.work) {
    int per_cu = 1;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dense_dkdv_queue_kernel<TT, D, BN>, 512, 0);
    if (e != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>(items, (int64_t)std::max(ncu, 1) * std::max(per_cu, 1));
    launch((dense_dkdv_queue_kernel<TT, D, BN>), dim3(grid), dim3(512), 0, st, p, (int)items);
  } else if constexpr (ATTN_DKDV_SEQ && D == 128) {
    // D = 128 holds one workgroup per CU: it runs its share of the items back to back.
    const int grid = (int)std::min<int64_t>(items, std::max(ncu, 1));
    launch((dense_dkdv_kernel<TT, D, BN, DKDV_SEQ>), dim3(grid), dim3(512), 0, st, p, (int)items);
  } else {
    // D = 64 fits two workgroups per CU, which the hardware fills item by item.
    launch((dense_dkdv_kernel<TT, D, BN, DKDV_ONE>), dim3((unsigned)items), dim3(512), 0, st, p,
                       (int)items);
  }
  return hipGetLastError();
}

// Landing of the split dK/dV (packed calls): dk = DT(scale * (slice 0 + slice 1)), dv = DT(slice 0
// + slice 1), the two slices always added in that order.  Only the rows of each sequence (clamped
// like the kernels' SeqView) are written, so tokens outside every sequence keep their contents.
// Thread: 8 consecutive elements of one sequence's [rows, Hkv, D] block.
template <class TT>
__global__ __launch_bounds__(256) void land_parts_kernel(const Params p, int64_t bps) {
  const int s = (int)(blockIdx.x / bps);
  const int64_t c8 = (int64_t)(blockIdx.x % bps) * 256 + threadIdx.x;
  const SeqView sv = seq_view(p.cu, s, p.Sq, p.Skv, p.Hq, p.max_seqlen);
  const int64_t row_elems = (int64_t)p.Hkv * p.Dqk;
  if (8 * c8 >= sv.Skv * row_elems) return;
  const int64_t e = sv.k0 * row_elems + 8 * c8;
  const float *acc[2] = {p.dk_acc, p.dv_acc};
  short *out[2] = {p.dk, p.dv};
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const float *a0 = acc[t] + e, *a1 = acc[t] + p.acc_slice + e;
    const Factors fac = factors(p);
    const float sc = t == 0 ? fac.dk : fac.dv;
    const f4v x0 = *(const f4v *)a0 + *(const f4v *)a1;
    const f4v x1 = *(const f4v *)(a0 + 4) + *(const f4v *)(a1 + 4);
    s8v o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      o[i] = TT::cvt_out(x0[i] * sc);
      o[4 + i] = TT::cvt_out(x1[i] * sc);
    }
    *(s8v *)(out[t] + e) = o;
  }
}

hipError_t launch_land_parts(const Params &p, int arith, hipStream_t st) {
  const bool bf16 = arith != ARITH_F16;  // the storage dtype decides the output cast
  if (!p.cu || p.hsplit != 2 || (p.Hkv * p.Dqk) % 8 != 0) return hipErrorInvalidValue;
  const int64_t bps = ((int64_t)p.max_seqlen * p.Hkv * p.Dqk / 8 + 255) / 256;
  const int64_t blocks = bps * p.nseq;
  if (blocks < 1) return hipSuccess;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (arith == ARITH_F16B)
    launch(land_parts_kernel<F16B>, dim3((unsigned)blocks), dim3(256), 0, st, p, bps);
  else if (bf16)
    launch(land_parts_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, p, bps);
  else
    launch(land_parts_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, st, p, bps);
  return hipGetLastError();
}

hipError_t launch_dense_dkdv(const Params &p, int arith, hipStream_t st) {
  if (p.Dqk == 128)
    return arith == ARITH_BF16 ? launch_dkdv_t<BF16, 128, 64>(p, st)
           : arith == ARITH_F16B ? launch_dkdv_t<F16B, 128, 64>(p, st)
                                 : launch_dkdv_t<F16, 128, 64>(p, st);
  if (p.Dqk == 64)
    return arith == ARITH_BF16 ? launch_dkdv_t<BF16, 64, 64>(p, st)
           : arith == ARITH_F16B ? launch_dkdv_t<F16B, 64, 64>(p, st)
                                 : launch_dkdv_t<F16, 64, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
