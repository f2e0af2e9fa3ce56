// sparse_bwd.hip -- dQ of the top-k backward: gathered, query-owned; and the f32 accumulator
// zero-fill and landing passes of the top-k path.
//
// TileLang PR #2592 page (sparse MLA backward): each query row attends to its own list of top-k
// keys, shared by all query heads of a KV head; the shape there is H = 64 query heads, one KV
// head, Dqk = 576, Dv = 512, topk = 2048.  The page finds the kernel bound by the gather of K/V
// rows, hidden only by keeping many loads in flight.
//
// dQ kernel (gfx950): one workgroup (4 wave64s, one per SIMD) per (batch, query row, KV head, block
// of 32 query heads).  Waves 0-1 hold the block's Q rows (each half of Dqk) and waves 2-3 its dO
// rows (each half of Dv) in registers as MFMA A operands for the whole walk.  The query's key
// list is walked in chunks of 32 slots whose K and V rows are gathered straight into LDS by
// direct global->LDS loads, double-buffered so that chunk c+1 is in flight while chunk c is
// computed.  Per chunk, on MFMA with f32 accumulation:
//   S = Q K^T and dP = dO V^T   (partial sums over the halves of the head dims, summed in LDS),
//   P = exp2(S*c - lse), dS = P (dP - delta)   (masked slots: padding -1, out of range or past
//                                               the causal diagonal contribute nothing),
//   dQ += dS K                  (owned by the workgroup, kept in registers, written once).
// Each list entry counts once per occurrence.  dK and dV come from the key-owned pass in
// sparse_dkdv.hip.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int DQK, int DV>
struct SpCfg {
  static constexpr int HB = 32;          // query heads per workgroup
  static constexpr int KC = 32;          // key slots per chunk
  static constexpr int CQ = DQK / 8;     // 16-byte chunks per Q/K row
  static constexpr int CV = DV / 8;      // 16-byte chunks per dO/V row
  static constexpr int KQ = DQK / 16;    // MFMA k-steps over Dqk
  static constexpr int KV = DV / 16;     // MFMA k-steps over Dv
  static constexpr int NQ = DQK / 32;    // 32-wide blocks of Dqk
  static constexpr int NV = DV / 32;     // 32-wide blocks of Dv
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims must be multiples of 32");
  static_assert(KQ % 2 == 0 && KV % 2 == 0, "k-steps split over two waves");
  static constexpr int LK = KC * CQ / 256;  // 16-byte gathers per thread: K rows of a chunk
  static constexpr int LV = KC * CV / 256;  // V rows
  static_assert((KC * CQ) % 256 == 0 && (KC * CV) % 256 == 0, "chunks split into whole workgroup loads");
};

// Tile rows are unpadded and their 16-byte chunk c sits at c ^ sw(row).  A Dqk = 576 row is
// 1152 bytes, half a bank line past a multiple of 256, like the 128-byte rows of swz<64>; a
// Dv = 512 row is 1024 bytes, bank-line aligned like the 256-byte rows of swz<128>.  The same
// two properties follow (16 distinct positions for a b128 read of one chunk over 16 rows, and
// for a transposed read of 4 rows x 4 chunks), and the XOR stays inside aligned groups of
// 8 (576) or 16 (512) chunks, so every chunk stays in its row.
template <int ROWLEN>
__device__ __forceinline__ int sp_sw(int row) {
  static_assert((2 * ROWLEN) % 256 == 128 || (2 * ROWLEN) % 256 == 0, "row alignment class");
  static_assert((2 * ROWLEN) % 256 == 0 ? (ROWLEN / 8) % 16 == 0 : (ROWLEN / 8) % 8 == 0, "XOR group");
  return (2 * ROWLEN) % 256 == 0 ? swz<128>(row) : swz<64>(row);
}

template <class TT, int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sparse_dq_kernel(const Params p) {
  using C = SpCfg<DQK, DV>;
  constexpr int PF = 3;
  __shared__ __attribute__((aligned(16))) short k_s[2][C::KC * DQK];
  __shared__ __attribute__((aligned(16))) short v_s[2][C::KC * DV];
  __shared__ __attribute__((aligned(16))) float part_s[4][16][64];  // S/dP partials
  __shared__ __attribute__((aligned(16))) short st_ds[2][C::HB * C::KC];  // dS [head][slot], hi / lo
  // Slot lists of chunks c, c+1 and c+2 (three buffers: the list of c+2 is written while chunk c
  // is still being read).
  __shared__ int idx_s[3][C::KC];  // key of each slot, -1 where the slot is masked
  __shared__ int row_s[3][C::KC];  // row gathered for each slot (a valid key of the chunk)
  __shared__ int any_s[3];         // whether the chunk has a valid slot
  __shared__ int idx_raw[4][C::KC];  // list entries of chunks c+1..c+3, loaded three chunks ahead

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  // Workgroups of the same (query row, KV head) gather the same K/V rows: the nhb head blocks of
  // one query are placed 8 apart in the dispatch order, which the hardware hands to the same XCD
  // at about the same time, so most second gathers of a row hit that XCD's L2.
  const Factors fac = factors(p);
  const int nhb = (p.G + C::HB - 1) / C::HB;
  int x = blockIdx.x;
  int hb;
  {
    const int grp = 8 * nhb, gi = x / grp, r = x % grp;
    if ((gi + 1) * 8 <= p.B * p.Sq * p.Hkv) {  // a full group of 8 queries
      hb = r / 8;
      x = gi * 8 + r % 8;
    } else {  // the ragged last group keeps the plain order
      hb = r % nhb;
      x = gi * 8 + r / nhb;
    }
  }
  const int g = x % p.Hkv;
  x /= p.Hkv;
  const int i = x % p.Sq;
  const int b = x / p.Sq;
  const int h0 = g * p.G + hb * C::HB;  // first query head of this block
  const int nh = min(C::HB, p.G - hb * C::HB);
  const int off = p.Skv - p.Sq;
  const int64_t qrow = ((int64_t)b * p.Sq + i) * p.Hq;  // + h: BSHD row of (b, i, h)

  // Resident A operands A[m = head lo][k = d] (32x32x16 layout): waves 0-1 Q rows over their half
  // of Dqk, waves 2-3 dO rows over their half of Dv.  Rows past nh repeat head nh-1 (masked).
  const bool sw_ = w < 2;
  constexpr int KH = (C::KQ / 2 > C::KV / 2) ? C::KQ / 2 : C::KV / 2;
  const int nk = sw_ ? C::KQ / 2 : C::KV / 2;
  const int k0 = (w & 1) * nk;
  s8v ar[KH];
  {
    const int64_t r = qrow + h0 + min(lo, nh - 1);
#pragma unroll
    for (int u = 0; u < KH; u++) {
      const int kk = k0 + min(u, nk - 1);
      ar[u] = sw_ ? *(const s8v *)(p.q + r * DQK + 16 * kk + 8 * hi) : *(const s8v *)(p.dout + r * DV + 16 * kk + 8 * hi);
    }
  }
  // lse and delta of the lane's rows of the accumulator layout (row m = 8*(r/4) + 4*hi + r%4).
  float lse_r[16], dl_r[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int m = min(8 * (r >> 2) + 4 * hi + (r & 3), nh - 1);
    const int64_t li = ((int64_t)b * p.Hq + h0 + m) * p.Sq + i;
    lse_r[r] = p.lse[li];
    dl_r[r] = p.ndelta[li];  // minus delta
  }

  // dQ accumulators: this wave owns the 32-wide d-blocks w, w+4, ... for the whole walk.
  constexpr int NQW = (C::NQ + 3) / 4;
  f16v dq[NQW];
#pragma unroll
  for (int u = 0; u < NQW; u++) dq[u] = f16v{};

  const int32_t *idx_row = p.idx + (((int64_t)b * p.Sq + i) * p.Hkv + g) * p.topk;
  const int nchunks = (p.topk + C::KC - 1) / C::KC;

  // Raw list entries of chunk c into idx_raw[c % 4] (wave 0, direct global->LDS loads, so that
  // reading them never makes the compiler wait for the gathers in flight); entries past topk
  // load the last entry and are dropped below.
  const i4v ridx = buf_rsrc(idx_row, (uint64_t)p.topk * 4);
  auto load_idx = [&](int c) {
    if (w == 0 && lane < C::KC) b2lds4(ridx, (uint32_t)min(c * C::KC + lane, p.topk - 1) * 4, &idx_raw[c & 3][0]);
  };
  // Slots of chunk c (wave 0): a masked slot (padding, out of range, past the causal diagonal)
  // gathers the row of the chunk's first valid slot, so every gathered row is one this query
  // attends; its own P and dS are forced to zero.
  auto slots = [&](int c) {
    const int buf = c % 3;
    int j = -1;
    if (lane < C::KC) {
      const int t = c * C::KC + lane;
      j = t < p.topk ? idx_raw[c & 3][lane] : -1;
      if (j < 0 || j >= p.Skv || (p.causal && j > i + off)) j = -1;
    }
    const uint64_t m = __ballot(j >= 0);
    const int first = m ? __shfl(j, __builtin_ctzll(m)) : 0;
    if (lane < C::KC) {
      idx_s[buf][lane] = j;
      row_s[buf][lane] = j >= 0 ? j : first;
    }
    if (lane == 0) any_s[buf] = m != 0;
  };
  // Gathers through buffer resources over this (batch, KV head)'s K and V rows; a row's byte
  // offset is row * Hkv * D * 2 (the host checks it fits 32 bits).
  const int64_t kv0 = (int64_t)b * p.Skv * p.Hkv + g, nkv = (int64_t)p.B * p.Skv * p.Hkv;
  const i4v rk = buf_rsrc(p.k + kv0 * DQK, (uint64_t)(nkv - kv0) * DQK * 2);
  const i4v rv = buf_rsrc(p.v + kv0 * p.v_ld, (uint64_t)(nkv - kv0) * p.v_ld * 2);
  // Tile slot s = 256 u + tid is physical chunk s % C of slot row s / C and holds logical chunk
  // (s % C) ^ sw(row); each lane's slot row and column byte offset are computed once, so a
  // gather costs one LDS read of the slot's key row and one multiply-add per load.
  uint32_t krow[C::LK], kcol[C::LK], vrow[C::LV], vcol[C::LV];
#pragma unroll
  for (int u = 0; u < C::LK; u++) {
    const int s = 256 * u + tid, r = s / C::CQ, ch = (s % C::CQ) ^ sp_sw<DQK>(r);
    krow[u] = (uint32_t)r;
    kcol[u] = (uint32_t)(16 * ch);
  }
#pragma unroll
  for (int u = 0; u < C::LV; u++) {
    const int s = 256 * u + tid, r = s / C::CV, ch = (s % C::CV) ^ sp_sw<DV>(r);
    vrow[u] = (uint32_t)r;
    vcol[u] = (uint32_t)(16 * ch);
  }
  const uint32_t k_lds = lds_addr(&k_s[0][0]), v_lds = lds_addr(&v_s[0][0]);
  const uint32_t kstride = (uint32_t)(p.Hkv * DQK * 2), vstride = (uint32_t)(p.Hkv * p.v_ld * 2);
  auto gather = [&](int c) {
    const int buf = c & 1, sb = c % 3;
    const int *rows = row_s[sb];
    const uint32_t kb = k_lds + buf * (C::KC * DQK * 2) + 1024 * w, vb = v_lds + buf * (C::KC * DV * 2) + 1024 * w;
#pragma unroll
    for (int u = 0; u < C::LK; u++) b2lds16_at(rk, (uint32_t)rows[krow[u]] * kstride + kcol[u], kb + 4096 * u);
#pragma unroll
    for (int u = 0; u < C::LV; u++) b2lds16_at(rv, (uint32_t)rows[vrow[u]] * vstride + vcol[u], vb + 4096 * u);
  };
  // B[k][n] = tile[row = 16*ks + 8*hi + e][col = 32*nb + lo] by transposed reads of a row-major
  // [slot][d] tile: per 16-lane group, lanes 4r..4r+3 supply 16 columns of row r and lane i
  // receives column i of the 4 rows.
  auto trB = [&](const short *tile, int ks, int nb) {
    const int col = 32 * nb + 16 * (g16 & 1) + 4 * (i16 & 3);
    s4v part[2];
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int row = 16 * ks + 8 * hi + 4 * half + (i16 >> 2);
      const int ch = (col >> 3) ^ sp_sw<DQK>(row);
      part[half] = lds_tr4(&tile[row * DQK + 8 * ch + (col & 7)]);
    }
    return cat8(part[0], part[1]);
  };

#pragma unroll
  for (int c = 0; c < 3; c++)
    if (c < nchunks) load_idx(c);
  wait_vm0();
  __syncthreads();
  if (w == 0) slots(0);
  __syncthreads();
  gather(0);
  if (w == 0 && nchunks > 1) slots(1);
  wait_vm0();
  __syncthreads();

  for (int c = 0; c < nchunks; c++) {
    const int buf = c & 1, sb = c % 3;
    if (c + 1 < nchunks) gather(c + 1);  // rows of chunk c+1 became visible at the last barrier
    if (c + 3 < nchunks) load_idx(c + 3);  // consumed by slots(c + 3) in the next iteration

    // Phase A: partial S (waves 0-1) or dP (waves 2-3) over this wave's half of the head dim;
    // M = heads, N = slots.  B = K / V rows of the slots, natural reads through a ring; two
    // accumulators so that consecutive products are independent.
    {
      const short *bt = sw_ ? k_s[buf] : v_s[buf];
      const int rowlen = sw_ ? DQK : DV;
      const int sw = sw_ ? sp_sw<DQK>(lo) : sp_sw<DV>(lo);
      f16v a0 = f16v{}, a1 = f16v{};
      ring_pipeline<KH, PF>(
          [&](int u) {
            const int kk = k0 + min(u, nk - 1);
            return *(const s8v *)&bt[lo * rowlen + 8 * ((2 * kk + hi) ^ sw)];
          },
          [&](int u, s8v bv) {
            if (u < nk) {
              if (u & 1)
                a1 = TT::mfma(ar[u], bv, a1);
              else
                a0 = TT::mfma(ar[u], bv, a0);
            }
          });
#pragma unroll
      for (int r = 0; r < 16; r++) part_s[w][r][lane] = a0[r] + a1[r];
    }
    __syncthreads();  // partials visible
    // Phase B: dS for accumulator registers r = 4w..4w+3 (row m = head 8*(r/4) + 4*hi + r%4,
    // column = slot lo); padded head rows and masked slots give 0.
    {
      const bool slot_ok = idx_s[sb][lo] >= 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r = 4 * w + q;
        const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float sv = part_s[0][r][lane] + part_s[1][r][lane];
        const float dpv = part_s[2][r][lane] + part_s[3][r][lane];
        const bool ok = slot_ok && m < nh;
        const float pr = exp2f_hw(sv * fac.c - lse_r[r]);
        const float ds = ok ? ds_of<TT>(pr, dpv + dl_r[r], fac) : 0.f;
        const short dh = TT::cvt(ds);
        st_ds[0][m * C::KC + lo] = dh;
        if (TT::SPLIT) st_ds[1][m * C::KC + lo] = TT::cvt(ds - TT::tof(dh));
      }
    }
    if (w == 0 && c + 2 < nchunks) slots(c + 2);  // read after the next barrier
    __syncthreads();  // dS visible
    // Phase C: dQ += dS K for this wave's d-blocks; A = dS[m = head lo][k = slots 16*ks + 8*hi
    // + e] (natural read), B = K^T by transposed reads through a ring.  A chunk with no valid
    // slot contributes nothing and is skipped (its gathered rows are not this query's keys).
    if (any_s[sb]) {
      s8v da[2], dl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        da[ks] = *(const s8v *)&st_ds[0][lo * C::KC + 16 * ks + 8 * hi];
        dl[ks] = TT::SPLIT ? *(const s8v *)&st_ds[1][lo * C::KC + 16 * ks + 8 * hi] : s8v{};
      }
      constexpr int N = 2 * NQW;
      s8v prev_b = s8v{};
      int prev_n = -1;
      auto lo_product = [&](int n, s8v bb) {
        const int ks = n / NQW, u = n % NQW;
        if (w + 4 * u < C::NQ) dq[u] = TT::mfma(dl[ks], bb, dq[u]);
      };
      ring_pipeline<N, PF>(
          [&](int n) { return trB(k_s[buf], n / NQW, min(w + 4 * (n % NQW), C::NQ - 1)); },
          [&](int n, s8v bb) {
            const int ks = n / NQW, u = n % NQW;
            if (w + 4 * u < C::NQ) dq[u] = TT::mfma(da[ks], bb, dq[u]);
            if (TT::SPLIT) {
              if (prev_n >= 0) lo_product(prev_n, prev_b);
              prev_n = n;
              prev_b = bb;
            }
          });
      if (TT::SPLIT) lo_product(prev_n, prev_b);
    }
    wait_vm0();
    __syncthreads();  // chunk c+1 landed, its rows' successor visible; chunk c consumed
  }

  // dQ = scale * acc for the block's valid heads (row m = head, column = d).
#pragma unroll
  for (int u = 0; u < NQW; u++) {
    const int nb = w + 4 * u;
    if (nb < C::NQ) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m < nh) p.dq[(qrow + h0 + m) * DQK + 32 * nb + lo] = TT::cvt_out(dq[u][r] * fac.dq);
      }
    }
  }
}

// dQ kernel for head groups that are multiples of 64 in fp16 arithmetic (one product per operand;
// the bf16 hi + lo form keeps the 32-head kernel above): one workgroup per (batch, query row, KV
// head, block of 64 query heads).  The K and V rows of a chunk are gathered once for all 64
// heads, half the gathers per product of the 32-head kernel.  Waves 0-1 form S for heads
// 32*(w&1) .. +31 over the whole of Dqk from their resident Q rows; waves 2-3 form dP - delta over
// the whole of Dv from their resident dO rows and hand it to the S waves through LDS; the S waves
// form P and dS; then every wave adds dS K into its 32-wide d-blocks of dQ for all 64 heads (two
// 32-row blocks sharing each B operand).
template <class TT, int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sparse_dq64_kernel(const Params p) {
  using C = SpCfg<DQK, DV>;
  static_assert(!TT::SPLIT, "one product per operand");
  constexpr int PF = 3, HB = 64;
  __shared__ __attribute__((aligned(16))) short k_s[2][C::KC * DQK];
  __shared__ __attribute__((aligned(16))) short v_s[2][C::KC * DV];
  __shared__ __attribute__((aligned(16))) float dpm_s[2][16][64];  // dP - delta of waves 2-3, [register][lane]
  __shared__ __attribute__((aligned(16))) short st_ds[HB * C::KC];  // dS [head][slot]
  __shared__ int idx_s[3][C::KC];    // key of each slot, -1 where the slot is masked
  __shared__ int row_s[3][C::KC];    // row gathered for each slot (a valid key of the chunk)
  __shared__ int any_s[3];           // whether the chunk has a valid slot
  __shared__ int idx_raw[4][C::KC];  // list entries of chunks c+1..c+3, loaded three chunks ahead

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const Factors fac = factors(p);
  // Head blocks of one query row gather the same rows: placed 8 apart in the dispatch order, so
  // that they run on one XCD at about the same time.
  const int nhb = p.G / HB;
  int x = blockIdx.x;
  int hb;
  {
    const int grp = 8 * nhb, gi = x / grp, r = x % grp;
    if ((gi + 1) * 8 <= p.B * p.Sq * p.Hkv) {
      hb = r / 8;
      x = gi * 8 + r % 8;
    } else {
      hb = r % nhb;
      x = gi * 8 + r / nhb;
    }
  }
  const int g = x % p.Hkv;
  x /= p.Hkv;
  const int i = x % p.Sq;
  const int b = x / p.Sq;
  const int h0 = g * p.G + hb * HB;  // first query head of this block
  const int off = p.Skv - p.Sq;
  const int64_t qrow = ((int64_t)b * p.Sq + i) * p.Hq;  // + h: BSHD row of (b, i, h)

  // Resident A operands A[m = head][k = d] (32x32x16 layout) of the wave's 32 heads hw .. hw+31:
  // Q rows (waves 0-1) or dO rows (waves 2-3) over the whole head dim.
  const bool s_wave = w < 2;
  const int hw = 32 * (w & 1);
  constexpr int KA = C::KQ > C::KV ? C::KQ : C::KV;
  const int nk = s_wave ? C::KQ : C::KV;
  s8v ar[KA];
  {
    const int64_t r = qrow + h0 + hw + lo;
#pragma unroll
    for (int u = 0; u < KA; u++) {
      const int kk = min(u, nk - 1);
      ar[u] = s_wave ? *(const s8v *)(p.q + r * DQK + 16 * kk + 8 * hi) : *(const s8v *)(p.dout + r * DV + 16 * kk + 8 * hi);
    }
  }
  // Per accumulator register r (row m = head hw + 8*(r/4) + 4*hi + r%4): lse for the S waves,
  // minus delta for the dP waves (the dP accumulators start from it).
  f16v lr;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int64_t li = ((int64_t)b * p.Hq + h0 + hw + 8 * (r >> 2) + 4 * hi + (r & 3)) * p.Sq + i;
    lr[r] = s_wave ? p.lse[li] : p.ndelta[li];
  }

  // dQ accumulators: d-blocks w, w+4, ... of both 32-head row blocks, for the whole walk.
  constexpr int NQW = (C::NQ + 3) / 4;
  f16v dq[2][NQW];
#pragma unroll
  for (int u = 0; u < NQW; u++) dq[0][u] = dq[1][u] = f16v{};

  const int32_t *idx_row = p.idx + (((int64_t)b * p.Sq + i) * p.Hkv + g) * p.topk;
  const int nchunks = (p.topk + C::KC - 1) / C::KC;
  // Raw list entries of chunk c into idx_raw[c % 4] (wave 0, direct loads; entries past topk
  // load the last entry and are dropped by the slot pass).
  const i4v ridx = buf_rsrc(idx_row, (uint64_t)p.topk * 4);
  auto load_idx = [&](int c) {
    if (w == 0 && lane < C::KC) b2lds4(ridx, (uint32_t)min(c * C::KC + lane, p.topk - 1) * 4, &idx_raw[c & 3][0]);
  };
  // Slots of chunk c (one wave): a masked slot (padding, out of range, past the causal diagonal)
  // gathers the row of the chunk's first valid slot; its own dS is forced to zero.
  auto slots = [&](int c) {
    const int sb = c % 3;
    int j = -1;
    if (lane < C::KC) {
      const int t = c * C::KC + lane;
      j = t < p.topk ? idx_raw[c & 3][lane] : -1;
      if (j < 0 || j >= p.Skv || (p.causal && j > i + off)) j = -1;
    }
    const uint64_t m = __ballot(j >= 0);
    const int first = m ? __shfl(j, __builtin_ctzll(m)) : 0;
    if (lane < C::KC) {
      idx_s[sb][lane] = j;
      row_s[sb][lane] = j >= 0 ? j : first;
    }
    if (lane == 0) any_s[sb] = m != 0;
  };
  // Gathers through buffer resources over this (batch, KV head)'s K and V rows (the host checks
  // that every byte offset fits 32 bits); lane slot rows and column offsets computed once.
  const int64_t kv0 = (int64_t)b * p.Skv * p.Hkv + g, nkv = (int64_t)p.B * p.Skv * p.Hkv;
  const i4v rk = buf_rsrc(p.k + kv0 * DQK, (uint64_t)(nkv - kv0) * DQK * 2);
  const i4v rv = buf_rsrc(p.v + kv0 * p.v_ld, (uint64_t)(nkv - kv0) * p.v_ld * 2);
  // Per load: slot row in the high half, column byte offset in the low half (one register each).
  uint32_t kslot[C::LK], vslot[C::LV];
#pragma unroll
  for (int u = 0; u < C::LK; u++) {
    const int s = 256 * u + tid, r = s / C::CQ, ch = (s % C::CQ) ^ sp_sw<DQK>(r);
    kslot[u] = (uint32_t)r << 16 | (uint32_t)(16 * ch);
  }
#pragma unroll
  for (int u = 0; u < C::LV; u++) {
    const int s = 256 * u + tid, r = s / C::CV, ch = (s % C::CV) ^ sp_sw<DV>(r);
    vslot[u] = (uint32_t)r << 16 | (uint32_t)(16 * ch);
  }
  const uint32_t k_lds = lds_addr(&k_s[0][0]), v_lds = lds_addr(&v_s[0][0]);
  const uint32_t kstride = (uint32_t)(p.Hkv * DQK * 2), vstride = (uint32_t)(p.Hkv * p.v_ld * 2);
  auto gather = [&](int c) {
    const int buf = c & 1;
    const int *rows = row_s[c % 3];
    const uint32_t kb = k_lds + buf * (C::KC * DQK * 2) + 1024 * w, vb = v_lds + buf * (C::KC * DV * 2) + 1024 * w;
#pragma unroll
    for (int u = 0; u < C::LK; u++)
      b2lds16_at(rk, (uint32_t)rows[kslot[u] >> 16] * kstride + (kslot[u] & 0xffffu), kb + 4096 * u);
#pragma unroll
    for (int u = 0; u < C::LV; u++)
      b2lds16_at(rv, (uint32_t)rows[vslot[u] >> 16] * vstride + (vslot[u] & 0xffffu), vb + 4096 * u);
  };
  // LDS read offsets of a lane within a tile, as (per-lane base + compile-time constant) so that
  // the constants fold into the reads' offset fields:
  //  natural read of slot row lo, logical chunk x = 2*kk + hi: the swizzle (below 16) only
  //   changes the low 4 bits of x, so chunk = 16*(kk/8) + ((2*(kk%8) + hi) ^ sw) and the byte
  //   offset is nat[kk % 8] + 256*(kk / 8);
  //  transposed read (B[k = slot 16*ks + 8*hi + e][n = d 32*nb + lo]) of row 16*ks + 8*hi +
  //   4*half + i16/4, column 32*nb + 16*(g16&1) + 4*(i16&3): the row's swizzle does not depend
  //   on ks and changes only the low 3 bits of the chunk 4*nb + t, so the byte offset is
  //   tr[half][nb % 2] + 18432*ks + 128*(nb / 2) (Dqk = 576).
  static_assert(DQK == 576, "transposed-read offsets assume 1152-byte rows");
  uint32_t nat[8], tr[2][2];
  {
    const int rowlen = s_wave ? DQK : DV;
    const int sw = s_wave ? sp_sw<DQK>(lo) : sp_sw<DV>(lo);
#pragma unroll
    for (int j = 0; j < 8; j++) nat[j] = (uint32_t)(2 * lo * rowlen + 16 * ((2 * j + hi) ^ sw));
    const int r4 = i16 >> 2, t = 2 * (g16 & 1) + ((i16 & 3) >> 1);
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int row = 8 * hi + 4 * half + r4, swr = sp_sw<DQK>(row);
#pragma unroll
      for (int par = 0; par < 2; par++)
        tr[half][par] = (uint32_t)(2 * DQK * row + 16 * ((4 * par + t) ^ swr) + 8 * (i16 & 1));
    }
  }

#pragma unroll
  for (int c = 0; c < 3; c++)
    if (c < nchunks) load_idx(c);
  wait_vm0();
  __syncthreads();
  if (w == 0) slots(0);
  __syncthreads();
  gather(0);
  if (w == 0 && nchunks > 1) slots(1);
  wait_vm0();
  __syncthreads();

  for (int c = 0; c < nchunks; c++) {
    const int buf = c & 1, sb = c % 3;
    if (c + 1 < nchunks) gather(c + 1);    // rows of chunk c+1 became visible at the last barrier
    if (c + 3 < nchunks) load_idx(c + 3);  // consumed by slots(c + 3) in the next iteration

    // Phase A: S = Q K^T (waves 0-1) or dP - delta = dO V^T - delta (waves 2-3) for the wave's
    // 32 heads over the whole head dim; M = heads, N = slots; B = K / V rows of the slots,
    // natural reads through a ring; two accumulators so that consecutive products are
    // independent.
    f16v acc;
    {
      const uint32_t tile = s_wave ? lds_addr(k_s[buf]) : lds_addr(v_s[buf]);
      uint32_t ab[8];
#pragma unroll
      for (int j = 0; j < 8; j++) ab[j] = lds_base_add(tile, nat[j]);
      f16v a0 = s_wave ? f16v{} : lr, a1 = f16v{};
      ring_pipeline<KA, PF>(
          [&](int u) {
            const int kk = min(u, nk - 1);
            return lds_rd16_at(ab[kk % 8] + 256 * (kk / 8));
          },
          [&](int u, s8v bv) {
            if (u < nk) {
              if (u & 1)
                a1 = TT::mfma(ar[u], bv, a1);
              else
                a0 = TT::mfma(ar[u], bv, a0);
            }
          });
      acc = a0 + a1;
    }
    if (!s_wave) {
#pragma unroll
      for (int r = 0; r < 16; r++) dpm_s[w - 2][r][lane] = acc[r];
    }
    __syncthreads();  // dP - delta visible
    // Phase B (S waves): P = exp2(S c - lse) and dS = P (dP - delta) of register r: head
    // hw + 8*(r/4) + 4*hi + r%4, slot lo; masked slots give 0.  A dP wave finds the slots of
    // chunk c+2 meanwhile.
    if (s_wave) {
      const bool slot_ok = idx_s[sb][lo] >= 0;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float pr = exp2f_hw(acc[r] * fac.c - lr[r]);
        const float ds = slot_ok ? ds_of<TT>(pr, dpm_s[w][r][lane], fac) : 0.f;
        st_ds[(hw + 8 * (r >> 2) + 4 * hi + (r & 3)) * C::KC + lo] = TT::cvt(ds);
      }
    } else if (w == 2 && c + 2 < nchunks) {
      slots(c + 2);  // read after the next barrier
    }
    __syncthreads();  // dS visible
    // Phase C: dQ += dS K for this wave's d-blocks and both row blocks; A = dS[m = head 32*mb + lo]
    // [k = slots 16*ks + 8*hi + e] (natural reads), B = K^T by transposed reads through a ring,
    // shared by the two row blocks.  A chunk with no valid slot contributes nothing.
    if (any_s[sb]) {
      s8v da[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) da[mb][ks] = *(const s8v *)&st_ds[(32 * mb + lo) * C::KC + 16 * ks + 8 * hi];
      uint32_t at[2][2];
#pragma unroll
      for (int half = 0; half < 2; half++)
#pragma unroll
        for (int par = 0; par < 2; par++) at[half][par] = lds_base_add(lds_addr(k_s[buf]), tr[half][par]);
      ring_pipeline<2 * NQW, PF>(
          [&](int n) {
            const int ks = n / NQW, nb = min(w + 4 * (n % NQW), C::NQ - 1);
            return cat8(lds_tr4_at(at[0][nb % 2] + 18432 * ks + 128 * (nb / 2)),
                        lds_tr4_at(at[1][nb % 2] + 18432 * ks + 128 * (nb / 2)));
          },
          [&](int n, s8v bb) {
            const int ks = n / NQW, u = n % NQW;
            if (w + 4 * u < C::NQ) {
              dq[0][u] = TT::mfma(da[0][ks], bb, dq[0][u]);
              dq[1][u] = TT::mfma(da[1][ks], bb, dq[1][u]);
            }
          });
    }
    wait_vm0();
    __syncthreads();  // chunk c+1 landed, its successor's slots visible; chunk c consumed
  }

  // dQ = scale * acc (row m = head 32*mb + 8*(r/4) + 4*hi + r%4, column 32*nb + lo).
#pragma unroll
  for (int u = 0; u < NQW; u++) {
    const int nb = w + 4 * u;
    if (nb < C::NQ) {
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = 32 * mb + 8 * (r >> 2) + 4 * hi + (r & 3);
          p.dq[(qrow + h0 + m) * DQK + 32 * nb + lo] = TT::cvt_out(dq[mb][u][r] * fac.dq);
        }
    }
  }
}

// Landing pass: dk = scale * dk_acc, dv = dv_acc, cast to the storage dtype (8 elements per
// thread, 32-byte reads and 16-byte writes).
template <class TT>
__global__ __launch_bounds__(256) void land_kernel(const float *__restrict__ acc, short *__restrict__ out, int64_t n8,
                                                   float scale, const float *rescale, int which) {
  if (rescale) scale = rescale[which];  // re-expressed bf16 call: the factor that undoes the scales
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8; v += (int64_t)gridDim.x * 256) {
    const f4v a = *(const f4v *)&acc[8 * v];
    const f4v c = *(const f4v *)&acc[8 * v + 4];
    s8v o;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      o[e] = TT::cvt(a[e] * scale);
      o[4 + e] = TT::cvt(c[e] * scale);
    }
    *(s8v *)&out[8 * v] = o;
  }
}

// Shared-latent landing: dKV = DT(dK_acc * scale + [dV_acc, 0]).  Row r of dK_acc has c8k chunks
// of 8 columns (Dqk / 8), row r of dV_acc c8v (Dv / 8); chunks past Dv take dK alone.
template <class TT>
__global__ __launch_bounds__(256) void land_kv_kernel(const float *__restrict__ dk_acc, const float *__restrict__ dv_acc,
                                                      short *__restrict__ out, int64_t n8, int c8k, int c8v,
                                                      float scale, const float *rescale) {
  const float sv = rescale ? rescale[3] : 1.f;
  if (rescale) scale = rescale[2];
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8; v += (int64_t)gridDim.x * 256) {
    const int64_t r = v / c8k;
    const int c = (int)(v - r * c8k);
    f4v a = *(const f4v *)&dk_acc[8 * v] * scale;
    f4v b = *(const f4v *)&dk_acc[8 * v + 4] * scale;
    if (c < c8v) {
      const float *d = &dv_acc[8 * (r * c8v + c)];
      a += *(const f4v *)d * sv;
      b += *(const f4v *)(d + 4) * sv;
    }
    s8v o;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      o[e] = TT::cvt(a[e]);
      o[4 + e] = TT::cvt(b[e]);
    }
    *(s8v *)&out[8 * v] = o;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float4 *__restrict__ buf, int64_t n4) {
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n4; v += (int64_t)gridDim.x * 256)
    buf[v] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_zero(float *buf, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4 floats
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  launch(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (float4 *)buf, n4);
  return hipGetLastError();
}

#ifndef ATTN_SPARSE_DQ64
#define ATTN_SPARSE_DQ64 1
#endif

hipError_t launch_sparse_dq(const Params &p, int arith, hipStream_t st) {
  if (p.Dqk != 576 || p.Dv != 512) return hipErrorInvalidValue;
  if (ATTN_SPARSE_DQ64 && arith != ARITH_BF16 && p.G % 64 == 0) {
    const int64_t blocks = (int64_t)p.B * p.Sq * p.Hkv * (p.G / 64);
    if (blocks < 1) return hipSuccess;
    if (arith == ARITH_F16B)
      launch((sparse_dq64_kernel<F16B, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    else
      launch((sparse_dq64_kernel<F16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  const int nhb = (p.G + SpCfg<576, 512>::HB - 1) / SpCfg<576, 512>::HB;
  const int64_t blocks = (int64_t)p.B * p.Sq * p.Hkv * nhb;
  if (blocks < 1) return hipSuccess;
  if (arith == ARITH_BF16)
    launch((sparse_dq_kernel<BF16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  else if (arith == ARITH_F16B)
    launch((sparse_dq_kernel<F16B, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  else
    launch((sparse_dq_kernel<F16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_land(const float *acc, short *out, int64_t n, float scale, const float *rescale, int which, bool bf16,
                       hipStream_t st) {
  const int64_t n8 = n / 8;  // callers pass multiples of 8 elements
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  if (bf16)
    launch(land_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, acc, out, n8, scale, rescale, which);
  else
    launch(land_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, st, acc, out, n8, scale, rescale, which);
  return hipGetLastError();
}

hipError_t launch_land_kv(const float *dk_acc, const float *dv_acc, short *out, int64_t rows, int64_t Dqk, int64_t Dv,
                          float scale, const float *rescale, bool bf16, hipStream_t st) {
  if (Dqk % 8 != 0 || Dv % 8 != 0 || Dv > Dqk) return hipErrorInvalidValue;
  const int64_t n8 = rows * (Dqk / 8);
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  if (bf16)
    launch(land_kv_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, dk_acc, dv_acc, out, n8,
                       (int)(Dqk / 8), (int)(Dv / 8), scale, rescale);
  else
    launch(land_kv_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, st, dk_acc, dv_acc, out, n8,
                       (int)(Dqk / 8), (int)(Dv / 8), scale, rescale);
  return hipGetLastError();
}

}  // namespace attn
