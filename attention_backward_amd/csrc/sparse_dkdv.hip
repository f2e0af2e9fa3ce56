// sparse_dkdv.hip -- dK and dV of the top-k backward, owned by key blocks, without atomics in the
// inner loop.
//
// TileLang PR #2592 page (sparse MLA backward): each query row attends to its own list of top-k
// keys; dK and dV of a key sum over every (query, head) whose list holds it.  A query-owned pass
// would have to add each query's dK/dV partials into global accumulators: 73 GB of f32 atomics on
// the 4096 x 8192, 64-head, top-2048 workload, which retire at about 1.36 TB/s on MI355X
// (measured).  Here a key block owns its dK/dV instead and walks the queries that can see it,
// weighting each (query, key) pair by the number of times the key occurs in the query's list:
//   cnt[b, g, i, j] = occurrences of key j in the valid entries of list (b, i, g)
// (built by topk_count_kernel below).  The lists cover about a third of the keys each query may
// see, so the pass does about three times the listed pairs' work, on MFMA, with no per-pair
// atomics.  A key block's query range is cut into chunks so that the grid balances; each chunk
// adds its finished 32-key dK/dV block once into f32 accumulators that a landing pass casts.
//
// Workgroup: 4 wave64s (one per SIMD, up to 512 VGPRs each), 32 keys of one (batch, KV head),
// one query chunk.  A step is one query i and a block of 32 of its KV head's query heads.  Wave w
// owns the 16-key x 16-head block (w&1, w>>1) of S^T = K Q^T and dP^T = V dO^T (v_mfma 16x16x32,
// the block's K and V rows resident in registers), forms P^T = cnt * exp2(S^T c - lse) and
// dS^T = P^T (dP^T - delta) for it, and accumulates a 128-wide slice of dV += P^T dO and a slice
// of dK += dS^T Q (5, 5, 4, 4 blocks of 32), reading the whole step's P^T / dS^T from LDS.
// Q and dO rows of the step (32 heads) are double-buffered in LDS, loaded directly from global
// memory; P^T and dS^T cross as 16-bit [key][head] tiles (hi and, for bf16, lo halves).  Every
// LDS operand is read a few products ahead through a register ring.
#include "common.h"
#include "kernels.h"

namespace attn {

// ---- multiplicity of each key in each query's list -----------------------------------------
// cnt is [B, Hkv, Sq, skv_pad] uint16 (zero-filled beforehand); skv_pad is even, so a pair of
// keys shares one 32-bit word and one atomic add per list entry counts it.  Counts stay below
// 65536 because topk does (checked on the host).
__global__ __launch_bounds__(256) void topk_count_kernel(const int32_t *__restrict__ idx, uint32_t *__restrict__ cnt,
                                                         int64_t n, int topk, int Sq, int Skv, int Hkv, int skv_pad,
                                                         int causal) {
  const int off = Skv - Sq;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) {
    const int j = idx[x];
    const int64_t row = x / topk;  // (b, i, g) in [B, Sq, Hkv] order
    const int g = (int)(row % Hkv);
    const int i = (int)((row / Hkv) % Sq);
    const int64_t b = row / ((int64_t)Hkv * Sq);
    if (j < 0 || j >= Skv || (causal && j > i + off)) continue;
    const int64_t e = (((b * Hkv + g) * Sq + i) * (int64_t)skv_pad) + j;
    atomicAdd(&cnt[e >> 1], 1u << (16 * (int)(e & 1)));
  }
}

// The same counts, one list per workgroup: the row [skv_pad] is built in LDS (LDS atomics) and
// written out whole, zeros included, so it needs no zero-fill beforehand and no global atomics.
// Row (b, i, g) of the lists is row ((b * Hkv + g) * Sq + i) of cnt.
__global__ __launch_bounds__(256) void topk_count_rows_kernel(const int32_t *__restrict__ idx, uint32_t *__restrict__ cnt,
                                                              int topk, int Sq, int Skv, int Hkv, int skv_pad, int causal) {
  extern __shared__ uint32_t crow[];  // skv_pad / 2 words, two 16-bit counts each
  const int64_t row = blockIdx.x;     // (b, i, g) in [B, Sq, Hkv] order
  const int g = (int)(row % Hkv);
  const int i = (int)((row / Hkv) % Sq);
  const int64_t b = row / ((int64_t)Hkv * Sq);
  const int nw = skv_pad / 2;
  for (int t = threadIdx.x; t < nw; t += 256) crow[t] = 0;
  __syncthreads();
  const int off = Skv - Sq;
  for (int x = threadIdx.x; x < topk; x += 256) {
    const int j = idx[row * topk + x];
    if (j < 0 || j >= Skv || (causal && j > i + off)) continue;
    atomicAdd(&crow[j >> 1], 1u << (16 * (j & 1)));
  }
  __syncthreads();
  uint32_t *dst = cnt + ((b * Hkv + g) * Sq + i) * (int64_t)nw;
  for (int t = threadIdx.x; t < nw; t += 256) dst[t] = crow[t];
}

template <int DQK, int DV>
struct SkCfg {
  static constexpr int BM = 32;           // keys per workgroup
  static constexpr int HB = 32;           // query heads per step
  static constexpr int CQ = DQK / 8;      // 16-byte chunks per Q row
  static constexpr int CV = DV / 8;       // 16-byte chunks per dO row
  static constexpr int KQ = DQK / 32;     // 16x16x32 k-steps over Dqk
  static constexpr int KV = DV / 32;      // 16x16x32 k-steps over Dv
  static constexpr int NQ = DQK / 32;     // 32-wide blocks of dK
  static constexpr int NVW = DV / 128;    // 32-wide blocks of dV per wave (4 waves)
  static constexpr int LQ = HB * CQ / 256;  // 16-byte loads per thread: Q tile
  static constexpr int LD = HB * CV / 256;  // dO tile
  static_assert(DV % 128 == 0 && DQK % 32 == 0, "head dims");
  static_assert((HB * CQ) % 256 == 0 && (HB * CV) % 256 == 0, "tiles split into whole workgroup loads");
};

// dK blocks of wave v: [first, first + count) out of NQ (NQ = 18: 5, 5, 4, 4).
__host__ __device__ constexpr int dk_first(int v, int nq) { return v * (nq / 4) + (v < nq % 4 ? v : nq % 4); }
__host__ __device__ constexpr int dk_count(int v, int nq) { return nq / 4 + (v < nq % 4 ? 1 : 0); }

// 16x16x32 products (lane layouts measured on MI355X with an in-bounds probe):
//   A lane l: A[m = l%16][k = 8*(l/16) + e];  B lane l: B[k = 8*(l/16) + e][n = l%16];
//   D lane l, register r: D[m = 4*(l/16) + r][n = l%16].
template <class TT>
__device__ __forceinline__ f4v mfma16(s8v a, s8v b, f4v c);
template <>
__device__ __forceinline__ f4v mfma16<F16>(s8v a, s8v b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f4v mfma16<F16B>(s8v a, s8v b, f4v c) {
  return mfma16<F16>(a, b, c);
}
template <>
__device__ __forceinline__ f4v mfma16<BF16>(s8v a, s8v b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
}

// Row classes of the unpadded LDS tiles (as in the gathered kernel): 1152-byte rows swizzle like
// the 128-byte rows of swz<64>, 1024-byte rows like the 256-byte rows of swz<128>.
template <int ROWLEN>
__device__ __forceinline__ int sk_sw(int row) {
  static_assert((2 * ROWLEN) % 256 == 128 || (2 * ROWLEN) % 256 == 0, "row alignment class");
  return (2 * ROWLEN) % 256 == 0 ? swz<128>(row) : swz<64>(row);
}

#ifndef ATTN_SPARSE_DKDV_SPLIT
#define ATTN_SPARSE_DKDV_SPLIT 1
#endif

template <class TT, int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sparse_dkdv_kernel(const Params p, const uint16_t *__restrict__ cnt,
                                                             int skv_pad, int qchunk, int nchunk,
                                                             float *__restrict__ dk_acc, float *__restrict__ dv_acc) {
  using C = SkCfg<DQK, DV>;
  constexpr int PF = 3;
  constexpr bool SPLIT = TT::SPLIT && ATTN_SPARSE_DKDV_SPLIT;
  __shared__ __attribute__((aligned(16))) short q_s[2][C::HB * DQK];
  __shared__ __attribute__((aligned(16))) short do_s[2][C::HB * DV];
  __shared__ __attribute__((aligned(16))) short st_p[2][C::BM * C::HB];  // P^T [key][head], hi / lo
  __shared__ __attribute__((aligned(16))) short st_ds[2][C::BM * C::HB];
  __shared__ __attribute__((aligned(16))) float lse_s[2][C::HB], dl_s[2][C::HB];
  __shared__ __attribute__((aligned(16))) uint16_t cnt_s[2][C::BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, lo = lane & 31;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int nkb = (p.Skv + C::BM - 1) / C::BM;
  const int BG = p.B * p.Hkv;
  int x = blockIdx.x;
  const int bg = x % BG;
  x /= BG;
  const int kb = x % nkb;
  const int qc = x / nkb;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int j0 = kb * C::BM;
  const int off = p.Skv - p.Sq;
  const Factors fac = factors(p);
  const int nhb = (p.G + C::HB - 1) / C::HB;
  // Query chunk qc, counted from the end: [max(i_lo, Sq - (qc+1)*qchunk), Sq - qc*qchunk).
  const int i_lo = p.causal ? max(0, j0 - off) : 0;
  const int i_end = p.Sq - qc * qchunk;
  const int i_beg = max(i_lo, i_end - qchunk);
  if (qc >= nchunk || i_end <= i_beg) return;  // uniform: the whole workgroup leaves
  const int nsteps = (i_end - i_beg) * nhb;

  // Resident A operands A[m = key][k = d] of this wave's 16 keys (16x16x32 layout): K and V rows.
  // Key rows past Skv are clamped (their counts are 0).
  const int kh = w & 1, hh = w >> 1;
  s8v kr[C::KQ], vr[C::KV];
  {
    const int key = min(j0 + 16 * kh + i16, p.Skv - 1);
    const int64_t r = ((int64_t)b * p.Skv + key) * p.Hkv + g;
#pragma unroll
    for (int kk = 0; kk < C::KQ; kk++) kr[kk] = *(const s8v *)(p.k + r * DQK + 32 * kk + 8 * g16);
#pragma unroll
    for (int kk = 0; kk < C::KV; kk++) vr[kk] = *(const s8v *)(p.v + r * p.v_ld + 32 * kk + 8 * g16);
  }

  // Accumulators (32 keys x 32-wide d blocks): dV blocks [4w, 4w+4), dK blocks [kf, kf + kn).
  constexpr int NKW = (C::NQ + 3) / 4;
  f16v av[C::NVW], ak[NKW];
#pragma unroll
  for (int u = 0; u < C::NVW; u++) av[u] = f16v{};
#pragma unroll
  for (int u = 0; u < NKW; u++) ak[u] = f16v{};
  const int kf = dk_first(w, C::NQ), kn = dk_count(w, C::NQ);

  // Step t -> query i = i_beg + t / nhb, head block t % nhb.  Loads of a step: Q and dO rows of
  // its heads (rows past the group's end repeat its last head; masked below), lse and delta,
  // and the count row of the 32 keys.  Tile slot s = 256 u + tid is physical chunk s % C of
  // row s / C and holds logical chunk (s % C) ^ sw(row); the lanes' byte offsets for a full head
  // block are computed once, and a ragged last block clamps its rows per step.
  uint32_t qoff[C::LQ], doff[C::LD];
#pragma unroll
  for (int u = 0; u < C::LQ; u++) {
    const int s = 256 * u + tid, r = s / C::CQ, ch = (s % C::CQ) ^ sk_sw<DQK>(r);
    qoff[u] = (uint32_t)(r * DQK + 8 * ch) * 2;
  }
#pragma unroll
  for (int u = 0; u < C::LD; u++) {
    const int s = 256 * u + tid, r = s / C::CV, ch = (s % C::CV) ^ sk_sw<DV>(r);
    doff[u] = (uint32_t)(r * DV + 8 * ch) * 2;
  }
  const uint32_t q_lds = lds_addr(&q_s[0][0]), do_lds = lds_addr(&do_s[0][0]);
  auto issue = [&](int t, int buf) {
    const int i = i_beg + t / nhb, hb0 = (t % nhb) * C::HB;
    const int nh = min(C::HB, p.G - hb0);
    const int64_t qrow = ((int64_t)b * p.Sq + i) * p.Hq + g * p.G + hb0;
    const int64_t nrows = (int64_t)p.B * p.Sq * p.Hq;
    const i4v rq = buf_rsrc(p.q + qrow * DQK, (uint64_t)(nrows - qrow) * DQK * 2);
    const i4v rd = buf_rsrc(p.dout + qrow * DV, (uint64_t)(nrows - qrow) * DV * 2);
    const uint32_t qb = q_lds + buf * (C::HB * DQK * 2) + 1024 * w, db = do_lds + buf * (C::HB * DV * 2) + 1024 * w;
    if (nh == C::HB) {
#pragma unroll
      for (int u = 0; u < C::LQ; u++) b2lds16_at(rq, qoff[u], qb + 4096 * u);
#pragma unroll
      for (int u = 0; u < C::LD; u++) b2lds16_at(rd, doff[u], db + 4096 * u);
    } else {
#pragma unroll
      for (int u = 0; u < C::LQ; u++) {
        const int s = 256 * u + tid, r = s / C::CQ, ch = (s % C::CQ) ^ sk_sw<DQK>(r);
        b2lds16_at(rq, (uint32_t)(min(r, nh - 1) * DQK + 8 * ch) * 2, qb + 4096 * u);
      }
#pragma unroll
      for (int u = 0; u < C::LD; u++) {
        const int s = 256 * u + tid, r = s / C::CV, ch = (s % C::CV) ^ sk_sw<DV>(r);
        b2lds16_at(rd, (uint32_t)(min(r, nh - 1) * DV + 8 * ch) * 2, db + 4096 * u);
      }
    }
    // One wave per small row (the LDS base of a direct load is per wave): lane l writes word l.
    if (w >= 2) {
      const int64_t l0 = ((int64_t)b * p.Hq + g * p.G + hb0) * p.Sq + i;
      const int64_t nl = (int64_t)p.B * p.Hq * p.Sq;
      const i4v rl = buf_rsrc((w == 3 ? (const float *)p.lse : (const float *)p.ndelta) + l0, (uint64_t)(nl - l0) * 4);
      if (lane < C::HB) b2lds4(rl, (uint32_t)(min(lane, nh - 1) * p.Sq) * 4, w == 3 ? &lse_s[buf][0] : &dl_s[buf][0]);
    } else if (w == 1) {
      const int64_t e0 = (((int64_t)b * p.Hkv + g) * p.Sq + i) * skv_pad + j0;
      const int64_t ne = (int64_t)p.B * p.Hkv * p.Sq * skv_pad;
      const i4v rc = buf_rsrc(cnt + e0, (uint64_t)(ne - e0) * 2);
      if (lane < C::BM / 2) b2lds4(rc, (uint32_t)(4 * lane), &cnt_s[buf][0]);
    }
  };

  // Transposed read of B[k = head][n = d] from a [head][d] tile (16 heads 16*ks + 8*hi + e).
  auto trB = [&](const short *tile, bool is_q, int ks, int nb) {
    const int rowlen = is_q ? DQK : DV;
    const int col = 32 * nb + 16 * (g16 & 1) + 4 * (i16 & 3);
    s4v part[2];
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int row = 16 * ks + 8 * hi + 4 * half + (i16 >> 2);
      const int ch = (col >> 3) ^ (is_q ? sk_sw<DQK>(row) : sk_sw<DV>(row));
      part[half] = lds_tr4(&tile[row * rowlen + 8 * ch + (col & 7)]);
    }
    return cat8(part[0], part[1]);
  };

  if (nsteps > 0) issue(0, 0);
  wait_vm0();
  __syncthreads();

  const int head = 16 * hh + i16;  // this lane's head column in the S^T / dP^T block
  const int swq = sk_sw<DQK>(head), swv = sk_sw<DV>(head);
  for (int t = 0; t < nsteps; t++) {
    const int buf = t & 1;
    const int nh = min(C::HB, p.G - (t % nhb) * C::HB);
    if (t + 1 < nsteps) issue(t + 1, buf ^ 1);

    // S^T and dP^T of the wave's block: B = Q / dO rows B[k = d][n = head] (natural reads of
    // the head's row).  The S and dP products alternate, so consecutive MFMAs never wait on
    // each other's accumulator; one ring carries the reads of both.
    f4v sv = f4v{}, dpv = f4v{};
    {
      const short *qrow = &q_s[buf][head * DQK];
      const short *drow = &do_s[buf][head * DV];
      // order: S0 P0 S1 P1 ... S(KV-1) P(KV-1) S(KV) ... S(KQ-1)
      auto is_s = [](int n) { return n >= 2 * C::KV || (n & 1) == 0; };
      auto kidx = [](int n) { return n >= 2 * C::KV ? n - C::KV : n >> 1; };
      ring_pipeline<C::KQ + C::KV, PF>(
          [&](int n) {
            const int kk = kidx(n);
            return is_s(n) ? *(const s8v *)&qrow[8 * ((4 * kk + g16) ^ swq)]
                           : *(const s8v *)&drow[8 * ((4 * kk + g16) ^ swv)];
          },
          [&](int n, s8v bv) {
            if (is_s(n))
              sv = mfma16<TT>(kr[kidx(n)], bv, sv);
            else
              dpv = mfma16<TT>(vr[kidx(n)], bv, dpv);
          });
    }
    // P^T and dS^T of the block: register r is key 16*kh + 4*g16 + r, head 16*hh + i16.
    {
      const float l = lse_s[buf][head], dl = dl_s[buf][head];
      const bool hok = head < nh;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int key = 16 * kh + 4 * g16 + r;
        const float c = (float)cnt_s[buf][key];
        const float pr = (hok && c > 0.f) ? c * exp2f_hw(sv[r] * fac.c - l) : 0.f;
        const float ds = ds_of<TT>(pr, dpv[r] + dl, fac);  // dl = minus delta
        const short ph = TT::cvt(pr), dh = TT::cvt(ds);
        st_p[0][key * C::HB + head] = ph;
        st_ds[0][key * C::HB + head] = dh;
        if (SPLIT) {
          st_p[1][key * C::HB + head] = TT::cvt(pr - TT::tof(ph));
          st_ds[1][key * C::HB + head] = TT::cvt(ds - TT::tof(dh));
        }
      }
    }
    __syncthreads();  // P^T, dS^T of the whole step visible
    // dV += P^T dO and dK += dS^T Q: M = 32 keys, N = 32-wide d blocks, K = 32 heads in two
    // 16-steps; A = the staging row of key lo (natural read), B = transposed reads of the tiles.
    {
      s8v pa[2], pl[2], da[2], dl2[2];
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        pa[ks] = *(const s8v *)&st_p[0][lo * C::HB + 16 * ks + 8 * hi];
        da[ks] = *(const s8v *)&st_ds[0][lo * C::HB + 16 * ks + 8 * hi];
        pl[ks] = SPLIT ? *(const s8v *)&st_p[1][lo * C::HB + 16 * ks + 8 * hi] : s8v{};
        dl2[ks] = SPLIT ? *(const s8v *)&st_ds[1][lo * C::HB + 16 * ks + 8 * hi] : s8v{};
      }
      constexpr int NV = 2 * C::NVW, NK = 2 * NKW;
      // For bf16 the lo-half product of operand n runs after the hi-half product of operand n+1,
      // so that two products on one accumulator are never back to back.
      s8v prev_b = s8v{};
      int prev_n = -1;
      auto lo_product = [&](int n, s8v bb) {
        if (n < NV) {
          const int ks = n / C::NVW, u = n % C::NVW;
          av[u] = TT::mfma(pl[ks], bb, av[u]);
        } else {
          const int m = n - NV, ks = m / NKW, u = m % NKW;
          if (u < kn) ak[u] = TT::mfma(dl2[ks], bb, ak[u]);
        }
      };
      ring_pipeline<NV + NK, PF>(
          [&](int n) {
            if (n < NV) return trB(do_s[buf], false, n / C::NVW, 4 * w + n % C::NVW);
            const int m = n - NV;
            return trB(q_s[buf], true, m / NKW, min(kf + m % NKW, C::NQ - 1));
          },
          [&](int n, s8v bb) {
            if (n < NV) {
              const int ks = n / C::NVW, u = n % C::NVW;
              av[u] = TT::mfma(pa[ks], bb, av[u]);
            } else {
              const int m = n - NV, ks = m / NKW, u = m % NKW;
              if (u < kn) ak[u] = TT::mfma(da[ks], bb, ak[u]);
            }
            if (SPLIT) {
              if (prev_n >= 0) lo_product(prev_n, prev_b);
              prev_n = n;
              prev_b = bb;
            }
          });
      if (SPLIT) lo_product(prev_n, prev_b);
    }
    wait_vm0();
    __syncthreads();  // next step's tiles landed; this step's tiles and staging consumed
  }

  // Add the block's dV / dK (unscaled) into the f32 accumulators at Hkv: row m of a block is key
  // j0 + 8*(r/4) + 4*hi + r%4, column 32*(block) + lo.
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (key < p.Skv) {
      const int64_t row = ((int64_t)b * p.Skv + key) * p.Hkv + g;
#pragma unroll
      for (int u = 0; u < C::NVW; u++) unsafeAtomicAdd(&dv_acc[row * DV + 32 * (4 * w + u) + lo], av[u][r]);
#pragma unroll
      for (int u = 0; u < NKW; u++)
        if (u < kn) unsafeAtomicAdd(&dk_acc[row * DQK + 32 * (kf + u) + lo], ak[u][r]);
    }
  }
}

bool topk_count_by_rows(int skv_pad) { return (int64_t)skv_pad * 2 <= kCountRowLdsMax; }

hipError_t launch_topk_count(const int32_t *idx, uint16_t *cnt, int64_t B, int64_t Sq, int64_t Skv, int64_t Hkv,
                             int64_t topk, int skv_pad, int causal, hipStream_t st) {
  if (topk_count_by_rows(skv_pad)) {
    const int64_t rows = B * Sq * Hkv;
    if (rows < 1) return hipSuccess;
    launch(topk_count_rows_kernel, dim3((unsigned)rows), dim3(256), (size_t)skv_pad * 2, st, idx,
                       (uint32_t *)cnt, (int)topk, (int)Sq, (int)Skv, (int)Hkv, skv_pad, causal);
    return hipGetLastError();
  }
  const int64_t n = B * Sq * Hkv * topk;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  launch(topk_count_kernel, dim3((unsigned)blocks), dim3(256), 0, st, idx, (uint32_t *)cnt, n, (int)topk,
                     (int)Sq, (int)Skv, (int)Hkv, skv_pad, causal);
  return hipGetLastError();
}

hipError_t launch_sparse_dkdv(const Params &p, const uint16_t *cnt, int skv_pad, float *dk_acc, float *dv_acc, int arith,
                              hipStream_t st) {
  if (p.Dqk != 576 || p.Dv != 512) return hipErrorInvalidValue;
  constexpr int BM = SkCfg<576, 512>::BM;
  const int nkb = (p.Skv + BM - 1) / BM;
  // Query chunks: about four workgroups' worth of steps per CU over the whole grid, at most the
  // full query range; chunks are counted from the last query, so every key block's first chunk
  // is a full one and the grid runs longest first.
  const int qchunk = 512;
  const int nchunk = (p.Sq + qchunk - 1) / qchunk;
  const int64_t blocks = (int64_t)nchunk * nkb * p.B * p.Hkv;
  if (blocks < 1) return hipSuccess;
  if (arith == ARITH_BF16)
    launch((sparse_dkdv_kernel<BF16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p, cnt, skv_pad,
                       qchunk, nchunk, dk_acc, dv_acc);
  else if (arith == ARITH_F16B)  // rescaled inputs: dS is brought back to its own scale
    launch((sparse_dkdv_kernel<F16B, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p, cnt, skv_pad,
                       qchunk, nchunk, dk_acc, dv_acc);
  else
    launch((sparse_dkdv_kernel<F16, 576, 512>), dim3((unsigned)blocks), dim3(256), 0, st, p, cnt, skv_pad,
                       qchunk, nchunk, dk_acc, dv_acc);
  return hipGetLastError();
}

}  // namespace attn
