// sparse_bwd.hip -- backward of attention over a gathered top-k key set per query.
//
// TileLang PR #2592 page (sparse MLA backward): each query row attends to its own list of
// top-k keys, shared by all query heads of a KV head; gradients for the shape H = 64 query
// heads, one KV head, Dqk = 576, Dv = 512, topk = 2048.  The page describes the kernel as
// bound by the gather of K/V rows ("memory-pipe bound"), whose latency is hidden by having
// many loads in flight.
//
// Kernel (gfx950): one workgroup (4 wave64s) per (batch, query row, KV head, block of 32 query
// heads).  The query block's Q and dO rows sit in LDS for the whole workgroup; the query's key
// list is walked in chunks of 32 slots whose K and V rows are gathered straight into LDS by
// direct global->LDS loads (the gather is the hot memory path; 32 rows x (Dqk + Dv) per chunk
// are in flight at once).  Per chunk, on 32x32x16 MFMA with f32 accumulation:
//   S = Q K^T and dP = dO V^T   (split over the head dim: waves 0-1 form S, 2-3 form dP),
//   P = exp2(S*c - lse), dS = P (dP - delta)   (masked slots: padding -1, out of range or
//                                               past the causal diagonal contribute nothing),
//   dQ += dS K                  (owned by the workgroup, kept in registers, written once),
//   dK[idx] += dS^T Q, dV[idx] += P^T dO   (summed over the 32 heads by the MFMA itself, then
//                                           added with f32 atomics into accumulators at Hkv
//                                           heads; a landing pass scales and casts them).
// Each list entry counts once per occurrence, as the index list defines the multiset of keys.
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
  static_assert((HB * CQ) % 64 == 0 && (HB * CV) % 64 == 0, "rows split into wave loads");
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
__global__ __launch_bounds__(256, 1) void sparse_bwd_kernel(const Params p, float *__restrict__ dk_acc,
                                                            float *__restrict__ dv_acc) {
  using C = SpCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) short q_s[C::HB * DQK];
  __shared__ __attribute__((aligned(16))) short do_s[C::HB * DV];
  __shared__ __attribute__((aligned(16))) short k_s[C::KC * DQK];
  __shared__ __attribute__((aligned(16))) short v_s[C::KC * DV];
  __shared__ __attribute__((aligned(16))) float part_s[4][16][64];  // S/dP partials; later P/dS
  __shared__ int idx_s[C::KC];   // key of each slot, -1 where the slot is masked
  __shared__ int row_s[C::KC];   // row gathered for each slot (a valid key of the chunk)
  __shared__ int any_s;          // whether the chunk has a valid slot
  __shared__ float lse_s[C::HB], dl_s[C::HB];
  // P and dS as 16-bit [head][slot] tiles (hi, then lo halves for bf16) alias part_s.
  short *st_p = (short *)&part_s[0][0][0];  // [2][HB][KC]
  short *st_ds = st_p + 2 * C::HB * C::KC;   // [2][HB][KC]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int nhb = (p.G + C::HB - 1) / C::HB;
  int x = blockIdx.x;
  const int hb = x % nhb;
  x /= nhb;
  const int g = x % p.Hkv;
  x /= p.Hkv;
  const int i = x % p.Sq;
  const int b = x / p.Sq;
  const int h0 = g * p.G + hb * C::HB;  // first query head of this block
  const int nh = min(C::HB, p.G - hb * C::HB);
  const int off = p.Skv - p.Sq;
  const int64_t qrow = ((int64_t)b * p.Sq + i) * p.Hq;  // + h: BSHD row of (b, i, h)

  // Q and dO rows of the block's heads (rows past nh repeat head nh-1; they are masked below).
  for (int s = tid; s < C::HB * C::CQ; s += 256) {
    const int r = s / C::CQ, ch = (s % C::CQ) ^ sp_sw<DQK>(r);
    const int h = h0 + min(r, nh - 1);
    g2lds16(p.q + (qrow + h) * DQK + 8 * ch, &q_s[(s - lane) * 8]);
  }
  for (int s = tid; s < C::HB * C::CV; s += 256) {
    const int r = s / C::CV, ch = (s % C::CV) ^ sp_sw<DV>(r);
    const int h = h0 + min(r, nh - 1);
    g2lds16(p.dout + (qrow + h) * DV + 8 * ch, &do_s[(s - lane) * 8]);
  }
  if (tid < C::HB) {
    const int h = h0 + min(tid, nh - 1);
    const int64_t li = ((int64_t)b * p.Hq + h) * p.Sq + i;
    lse_s[tid] = p.lse[li];
    dl_s[tid] = p.delta[li];
  }

  // dQ accumulators: this wave owns the 32-wide d-blocks w, w+4, ... for the whole walk.
  constexpr int NQW = (C::NQ + 3) / 4;
  f16v dq[NQW];
#pragma unroll
  for (int u = 0; u < NQW; u++) dq[u] = f16v{};

  const int32_t *idx_row = p.idx + (((int64_t)b * p.Sq + i) * p.Hkv + g) * p.topk;
  const int nchunks = (p.topk + C::KC - 1) / C::KC;

  for (int cidx = 0; cidx < nchunks; cidx++) {
    const int t0 = cidx * C::KC;
    __syncthreads();  // the previous chunk is fully consumed (k_s, v_s, idx_s, staging)
    if (w == 0) {
      // Slots are lanes 0..KC-1 of wave 0.  A masked slot (padding, out of range, past the
      // causal diagonal) gathers the row of the chunk's first valid slot, so every row in the
      // tile is one this query attends; its own P and dS are forced to zero.
      int j = -1;
      if (lane < C::KC) {
        const int t = t0 + lane;
        j = t < p.topk ? idx_row[t] : -1;
        if (j < 0 || j >= p.Skv || (p.causal && j > i + off)) j = -1;
      }
      const uint64_t m = __ballot(j >= 0);
      const int first = m ? __shfl(j, __builtin_ctzll(m)) : 0;
      if (lane < C::KC) {
        idx_s[lane] = j;
        row_s[lane] = j >= 0 ? j : first;
      }
      if (lane == 0) any_s = m != 0;
    }
    __syncthreads();
    if (!any_s) continue;  // uniform: nothing in this chunk contributes
    for (int s = tid; s < C::KC * C::CQ; s += 256) {
      const int r = s / C::CQ, ch = (s % C::CQ) ^ sp_sw<DQK>(r);
      g2lds16(p.k + (((int64_t)b * p.Skv + row_s[r]) * p.Hkv + g) * DQK + 8 * ch, &k_s[(s - lane) * 8]);
    }
    for (int s = tid; s < C::KC * C::CV; s += 256) {
      const int r = s / C::CV, ch = (s % C::CV) ^ sp_sw<DV>(r);
      g2lds16(p.v + (((int64_t)b * p.Skv + row_s[r]) * p.Hkv + g) * DV + 8 * ch, &v_s[(s - lane) * 8]);
    }
    wait_vm0();
    __syncthreads();

    // Phase A: S (waves 0, 1: halves of Dqk) and dP (waves 2, 3: halves of Dv); M = heads,
    // N = key slots; A = Q / dO rows and B = K / V rows, both natural b128 reads.
    {
      f16v acc = f16v{};
      if (w < 2) {
        const int sw = sp_sw<DQK>(lo);
        for (int kk = w * (C::KQ / 2); kk < (w + 1) * (C::KQ / 2); kk++) {
          const int ch = (2 * kk + hi) ^ sw;
          acc = TT::mfma(*(const s8v *)&q_s[lo * DQK + 8 * ch], *(const s8v *)&k_s[lo * DQK + 8 * ch], acc);
        }
      } else {
        const int sw = sp_sw<DV>(lo);
        for (int kk = (w - 2) * (C::KV / 2); kk < (w - 1) * (C::KV / 2); kk++) {
          const int ch = (2 * kk + hi) ^ sw;
          acc = TT::mfma(*(const s8v *)&do_s[lo * DV + 8 * ch], *(const s8v *)&v_s[lo * DV + 8 * ch], acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r++) part_s[w][r][lane] = acc[r];
    }
    __syncthreads();
    // Phase B: P and dS in the accumulator layout (row m = head 8*(r/4) + 4*hi + r%4, column =
    // slot lo).  Formed by wave 0 only; padded head rows (m >= nh) and masked slots give 0.
    if (w == 0) {
      const bool slot_ok = idx_s[lo] >= 0;
      float pv[16], dsv[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float sv = part_s[0][r][lane] + part_s[1][r][lane];
        const float dpv = part_s[2][r][lane] + part_s[3][r][lane];
        const bool ok = slot_ok && m < nh;
        const float pr = exp2f_hw(sv * p.c - lse_s[m]);
        pv[r] = ok ? pr : 0.f;
        dsv[r] = ok ? pr * (dpv - dl_s[m]) : 0.f;
      }
      // The staging tiles alias part_s; this wave's reads of it above are complete before its
      // writes below (one wave's LDS instructions execute in order), and no other wave reads
      // part_s in this phase.
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
        const short ph = TT::cvt(pv[r]), dh = TT::cvt(dsv[r]);
        st_p[m * C::KC + lo] = ph;
        st_ds[m * C::KC + lo] = dh;
        st_p[C::HB * C::KC + m * C::KC + lo] = TT::SPLIT ? TT::cvt(pv[r] - TT::tof(ph)) : (short)0;
        st_ds[C::HB * C::KC + m * C::KC + lo] = TT::SPLIT ? TT::cvt(dsv[r] - TT::tof(dh)) : (short)0;
      }
    }
    __syncthreads();

    // Phase C.  B operands B[k][n] = tile[row = 16*ks + 8*hi + e][col = 32*nb + lo] come from
    // the row-major Q, dO and K tiles by transposed reads: per 16-lane group, lanes 4r..4r+3
    // supply 16 columns of row r and lane i receives column i of the 4 rows, so the group
    // 16*(g16&1) + i16 = lo gets its own column and two reads (+4 rows) give the 8 k values.
    auto trB = [&](const short *tile, bool is_q, int ks, int nb) {
      const int rowlen = is_q ? DQK : DV;
      const int col = 32 * nb + 16 * (g16 & 1) + 4 * (i16 & 3);
      s4v part[2];
#pragma unroll
      for (int half = 0; half < 2; half++) {
        const int row = 16 * ks + 8 * hi + 4 * half + (i16 >> 2);
        const int ch = (col >> 3) ^ (is_q ? sp_sw<DQK>(row) : sp_sw<DV>(row));
        part[half] = lds_tr4(&tile[row * rowlen + 8 * ch + (col & 7)]);
      }
      return cat8(part[0], part[1]);
    };
    // A operand of dQ: dS[m = head lo][k = key slots 16*ks + 8*hi + e], natural read.
    auto dsA = [&](int ks, int lohalf) {
      return *(const s8v *)&st_ds[lohalf * C::HB * C::KC + lo * C::KC + 16 * ks + 8 * hi];
    };
    // A operand of dK/dV: X^T[m = key slot lo][k = heads 16*ks + 8*hi + e] from the [head][key]
    // staging tile by transposed reads (4 heads per read).
    auto stT = [&](const short *tile, int ks, int lohalf) {
      const short *t = tile + lohalf * C::HB * C::KC;
      s4v part[2];
#pragma unroll
      for (int half = 0; half < 2; half++) {
        const int row = 16 * ks + 8 * hi + 4 * half + (i16 >> 2);
        const int col = 16 * (g16 & 1) + 4 * (i16 & 3);
        part[half] = lds_tr4(&t[row * C::KC + col]);
      }
      return cat8(part[0], part[1]);
    };

    // dQ += dS K  (this wave's d-blocks)
#pragma unroll
    for (int u = 0; u < NQW; u++) {
      const int nb = w + 4 * u;
      if (nb < C::NQ) {
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          const s8v bb = trB(k_s, true, ks, nb);
          dq[u] = TT::mfma(dsA(ks, 0), bb, dq[u]);
          if (TT::SPLIT) dq[u] = TT::mfma(dsA(ks, 1), bb, dq[u]);
        }
      }
    }
    // dK[idx] += dS^T Q and dV[idx] += P^T dO, one 32x32 block at a time, added atomically.
    auto scatter = [&](float *accbuf, int dlen, int nb, const f16v &c) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int slot = 8 * (r >> 2) + 4 * hi + (r & 3);
        const int j = idx_s[slot];
        if (j >= 0) unsafeAtomicAdd(&accbuf[(((int64_t)b * p.Skv + j) * p.Hkv + g) * dlen + 32 * nb + lo], c[r]);
      }
    };
    for (int nb = w; nb < C::NQ; nb += 4) {
      f16v c = f16v{};
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const s8v bb = trB(q_s, true, ks, nb);
        c = TT::mfma(stT(st_ds, ks, 0), bb, c);
        if (TT::SPLIT) c = TT::mfma(stT(st_ds, ks, 1), bb, c);
      }
      scatter(dk_acc, DQK, nb, c);
    }
    for (int nb = w; nb < C::NV; nb += 4) {
      f16v c = f16v{};
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const s8v bb = trB(do_s, false, ks, nb);
        c = TT::mfma(stT(st_p, ks, 0), bb, c);
        if (TT::SPLIT) c = TT::mfma(stT(st_p, ks, 1), bb, c);
      }
      scatter(dv_acc, DV, nb, c);
    }
  }

  wait_vm0();  // the Q/dO loads, when every chunk was skipped
  // dQ = scale * acc for the block's valid heads (row m = head, column = d).
#pragma unroll
  for (int u = 0; u < NQW; u++) {
    const int nb = w + 4 * u;
    if (nb < C::NQ) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m < nh) p.dq[(qrow + h0 + m) * DQK + 32 * nb + lo] = TT::cvt(dq[u][r] * p.scale);
      }
    }
  }
}

// Landing pass: dk = scale * dk_acc, dv = dv_acc, cast to the storage dtype (8 elements per
// thread, 32-byte reads and 16-byte writes).
template <class TT>
__global__ __launch_bounds__(256) void land_kernel(const float *__restrict__ acc, short *__restrict__ out, int64_t n8,
                                                   float scale) {
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

__global__ __launch_bounds__(256) void zero_kernel(float4 *__restrict__ buf, int64_t n4) {
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n4; v += (int64_t)gridDim.x * 256)
    buf[v] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_zero(float *buf, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4 floats
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (float4 *)buf, n4);
  return hipGetLastError();
}

hipError_t launch_sparse_bwd(const Params &p, float *dk_acc, float *dv_acc, bool bf16, hipStream_t st) {
  if (p.Dqk != 576 || p.Dv != 512) return hipErrorInvalidValue;
  const int nhb = (p.G + SpCfg<576, 512>::HB - 1) / SpCfg<576, 512>::HB;
  const int64_t blocks = (int64_t)p.B * p.Sq * p.Hkv * nhb;
  if (blocks < 1) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL((sparse_bwd_kernel<BF16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p, dk_acc, dv_acc);
  else
    hipLaunchKernelGGL((sparse_bwd_kernel<F16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p, dk_acc, dv_acc);
  return hipGetLastError();
}

hipError_t launch_land(const float *acc, short *out, int64_t n, float scale, bool bf16, hipStream_t st) {
  const int64_t n8 = n / 8;  // callers pass multiples of 8 elements
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(land_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, acc, out, n8, scale);
  else
    hipLaunchKernelGGL(land_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, st, acc, out, n8, scale);
  return hipGetLastError();
}

}  // namespace attn
