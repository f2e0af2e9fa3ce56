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
// Workgroup: 4 wave64s (one per SIMD, up to 512 registers each), 32 keys of one (batch, KV head),
// one query chunk.  A step is one query i and a block of 16 of its KV head's query heads.  The
// waves split by role and run one step apart:
//   - waves 0 and 1 (scoring) hold the K and V rows of keys 16w..16w+15 as the A operands of
//     S^T = K Q^T and dP^T = V dO^T (v_mfma 16x16x32), form P^T = cnt * exp2(S^T c - lse) and
//     dS^T = P^T (dP^T - delta) of step t and stage them in LDS as 16-bit [key][head] blocks
//     (hi and, for bf16, lo halves);
//   - waves 2 and 3 (accumulating) add step t-1 into dV += P^T dO and dK += dS^T Q (32x32x16
//     products, 8 dV and 7 dK blocks of 32 columns each; the scoring waves take the last 4 dK
//     blocks, 2 each), and load the Q / dO tiles of step t+1 straight into LDS.
// Tiles go round three LDS buffers (t+1 stored, t scored, t-1 accumulated) and one barrier per
// step hands them on.  Every LDS operand is read a few products ahead through a register ring.
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
  static constexpr int BM = 32;              // keys per workgroup
  static constexpr int HB = 16;              // query heads per step
  static constexpr int CQ = DQK / 8;         // 16-byte chunks per Q row
  static constexpr int CV = DV / 8;          // 16-byte chunks per dO row
  static constexpr int KQ = DQK / 32;        // 16x16x32 k-steps over Dqk
  static constexpr int KV = DV / 32;         // 16x16x32 k-steps over Dv
  static constexpr int NQ = DQK / 32;        // 32-wide blocks of dK
  static constexpr int NV = DV / 32;         // 32-wide blocks of dV
  static constexpr int NVW = NV / 2;         // dV blocks of each accumulating wave
  static constexpr int NKS = 2;              // dK blocks of each scoring wave (the last 2 NKS)
  static constexpr int NKK = (NQ - 2 * NKS) / 2;  // dK blocks of each accumulating wave
  static constexpr int LQ = HB * CQ / 128;   // 16-byte loads per lane of the two loading waves: Q tile
  static constexpr int LD = HB * CV / 128;   // dO tile
  static constexpr int NLD = LQ + LD;
  static_assert(NV % 2 == 0 && DQK % 32 == 0 && NQ > 2 * NKS && (NQ - 2 * NKS) % 2 == 0, "head dims");
  // An accumulating wave holds NVW + NKK 32x32 f32 blocks in its 256 AGPRs; at 16 blocks the
  // compiler starts copying accumulators through VGPRs inside the loop.
  static_assert(NVW + NKK <= 15, "accumulators of one wave");
  static_assert((HB * CQ) % 128 == 0 && (HB * CV) % 128 == 0, "tiles split into whole loads of two waves");
};

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

template <class TT, int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sparse_dkdv_kernel(const Params p, const uint16_t *__restrict__ cnt,
                                                             int skv_pad, int qchunk, int nchunk,
                                                             float *__restrict__ dk_acc, float *__restrict__ dv_acc) {
  using C = SkCfg<DQK, DV>;
  constexpr int PF = 3;
  constexpr bool SPLIT = TT::SPLIT;
  constexpr int NH = SPLIT ? 2 : 1;                   // staged halves of P^T and dS^T
  constexpr int TQ = C::HB * DQK, TD = C::HB * DV;    // elements per Q / dO tile
  __shared__ __attribute__((aligned(16))) short q_s[3][TQ];
  __shared__ __attribute__((aligned(16))) short do_s[3][TD];
  __shared__ __attribute__((aligned(16))) short st_p[2][NH][C::BM * C::HB];  // P^T [key][head], hi / lo
  __shared__ __attribute__((aligned(16))) short st_ds[2][NH][C::BM * C::HB];
  __shared__ __attribute__((aligned(16))) float lse_s[3][C::HB], dl_s[3][C::HB];
  __shared__ __attribute__((aligned(16))) uint16_t cnt_s[3][C::BM];

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

  // Step t is query i_beg + t / nhb and the head block t % nhb of its KV head's group.  Waves 0
  // and 1 form S^T, dP^T, P^T and dS^T of step t for keys 16w..16w+15 and stage P^T / dS^T; waves
  // 2 and 3 meanwhile add step t-1 into dV and dK and load the tiles of step t+1.  The tiles go
  // round three buffers (t+1 loading, t scored, t-1 accumulated), the staging round two, and
  // one barrier per step hands both on.  The loop runs one extra step to accumulate the last.

  // Transposed read of B[k = head][n = d] from a [head][d] tile (heads 8*hi + e).
  auto trB = [&](const short *tile, bool is_q, int nb) {
    const int rowlen = is_q ? DQK : DV;
    const int col = 32 * nb + 16 * (g16 & 1) + 4 * (i16 & 3);
    s4v part[2];
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int row = 8 * hi + 4 * half + (i16 >> 2);
      const int ch = (col >> 3) ^ (is_q ? sk_sw<DQK>(row) : sk_sw<DV>(row));
      part[half] = lds_tr4(&tile[row * rowlen + 8 * ch + (col & 7)]);
    }
    return cat8(part[0], part[1]);
  };
  // Add finished 32-key blocks (unscaled) into the f32 accumulators at Hkv: register r of a
  // block is key j0 + 8*(r/4) + 4*hi + r%4, column 32*(first + u) + lo.
  // The block count is a template argument: indexing the accumulator array with a run-time
  // count would move the whole array to scratch memory.
  auto add_blocks = [&](auto nblk, const f16v *acc, float *dst, int rowlen, int first) {
    constexpr int N = decltype(nblk)::value;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (key < p.Skv) {
        const int64_t row = ((int64_t)b * p.Skv + key) * p.Hkv + g;
#pragma unroll
        for (int u = 0; u < N; u++) unsafeAtomicAdd(&dst[row * rowlen + 32 * (first + u) + lo], acc[u][r]);
      }
    }
  };

  if (w < 2) {
    // Resident A operands A[m = key][k = d] of this wave's 16 keys (16x16x32 layout): K and V
    // rows.  Key rows past Skv are clamped (their counts are 0).
    s8v kr[C::KQ], vr[C::KV];
    {
      const int key = min(j0 + 16 * w + i16, p.Skv - 1);
      const int64_t r = ((int64_t)b * p.Skv + key) * p.Hkv + g;
#pragma unroll
      for (int kk = 0; kk < C::KQ; kk++) kr[kk] = *(const s8v *)(p.k + r * DQK + 32 * kk + 8 * g16);
#pragma unroll
      for (int kk = 0; kk < C::KV; kk++) vr[kk] = *(const s8v *)(p.v + r * p.v_ld + 32 * kk + 8 * g16);
    }
    const int swq = sk_sw<DQK>(i16), swv = sk_sw<DV>(i16);
    // dK blocks [ks0, ks0 + NKS) of step t-1, added at the start of step t.
    const int ks0 = C::NQ - 2 * C::NKS + C::NKS * w;
    f16v aks[C::NKS];
#pragma unroll
    for (int u = 0; u < C::NKS; u++) aks[u] = f16v{};
    __syncthreads();  // the first step's tiles landed
    int b3 = 0, hb = 0;
    for (int t = 0; t <= nsteps; t++) {
      if (t > 0) {
        const int bp = b3 == 0 ? 2 : b3 - 1, sbp = (t - 1) & 1;
        const s8v da = *(const s8v *)&st_ds[sbp][0][lo * C::HB + 8 * hi];
        const s8v dl2 = SPLIT ? *(const s8v *)&st_ds[sbp][NH - 1][lo * C::HB + 8 * hi] : s8v{};
        s8v bb[C::NKS];
#pragma unroll
        for (int u = 0; u < C::NKS; u++) bb[u] = trB(q_s[bp], true, ks0 + u);
#pragma unroll
        for (int u = 0; u < C::NKS; u++) aks[u] = TT::mfma(da, bb[u], aks[u]);
        if (SPLIT) {
#pragma unroll
          for (int u = 0; u < C::NKS; u++) aks[u] = TT::mfma(dl2, bb[u], aks[u]);
        }
      }
      if (t < nsteps) {
        const int nh = min(C::HB, p.G - hb * C::HB);
        // S^T and dP^T of the wave's block: B = Q / dO rows B[k = d][n = head] (natural reads of
        // the head's row).  The S and dP products alternate, so consecutive MFMAs never wait on
        // each other's accumulator; one ring carries the reads of both.
        f4v sv = f4v{}, dpv = f4v{};
        {
          const short *qrow = &q_s[b3][i16 * DQK];
          const short *drow = &do_s[b3][i16 * DV];
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
        // P^T and dS^T of the block: register r is key 16*w + 4*g16 + r, head i16.
        const float l = lse_s[b3][i16], dl = dl_s[b3][i16];
        const bool hok = i16 < nh;
        const int sb = t & 1;
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int key = 16 * w + 4 * g16 + r;
          const float c = (float)cnt_s[b3][key];
          const float pr = (hok && c > 0.f) ? c * exp2f_hw(sv[r] * fac.c - l) : 0.f;
          const float ds = ds_of<TT>(pr, dpv[r] + dl, fac);  // dl = minus delta
          const short ph = TT::cvt(pr), dh = TT::cvt(ds);
          st_p[sb][0][key * C::HB + i16] = ph;
          st_ds[sb][0][key * C::HB + i16] = dh;
          if (SPLIT) {
            st_p[sb][NH - 1][key * C::HB + i16] = TT::cvt(pr - TT::tof(ph));
            st_ds[sb][NH - 1][key * C::HB + i16] = TT::cvt(ds - TT::tof(dh));
          }
        }
      }
      __syncthreads();  // step t staged; step t+1's tiles landed
      b3 = b3 == 2 ? 0 : b3 + 1;
      hb = hb + 1 == nhb ? 0 : hb + 1;
    }
    add_blocks(std::integral_constant<int, C::NKS>{}, aks, dk_acc, DQK, ks0);
    return;
  }

  // Waves 2 and 3: accumulators (32 keys x 32-wide d blocks) dV blocks [NVW v, NVW v + NVW) and
  // dK blocks [kf, kf + NKK).
  const int v = w - 2;
  f16v av[C::NVW], ak[C::NKK];
#pragma unroll
  for (int u = 0; u < C::NVW; u++) av[u] = f16v{};
#pragma unroll
  for (int u = 0; u < C::NKK; u++) ak[u] = f16v{};
  const int kf = v * C::NKK;

  // Loads of a step, straight into LDS through buffer resources: Q and dO rows of its heads
  // through resources that end after the block's last head of the group (rows past it read as
  // zero; their heads are masked), lse and delta of those heads, and the count row of the 32
  // keys.  Tile slot s = 128 u + 64 v + lane is physical chunk s % C of row s / C and holds
  // logical chunk (s % C) ^ sw(row); load u of the wave writes 1 KB at 2048 u + 1024 v of the
  // tile.  All of a step's loads go out before its products: spread between the products the
  // kernel took 17% longer, and with loads through registers 13% longer (each wave's register
  // loads came back about two steps after issue).
  uint32_t qoff[C::LQ], doff[C::LD];
#pragma unroll
  for (int u = 0; u < C::LQ; u++) {
    const int s = 128 * u + 64 * v + lane, r = s / C::CQ, ch = (s % C::CQ) ^ sk_sw<DQK>(r);
    qoff[u] = (uint32_t)(r * DQK + 8 * ch) * 2;
  }
#pragma unroll
  for (int u = 0; u < C::LD; u++) {
    const int s = 128 * u + 64 * v + lane, r = s / C::CV, ch = (s % C::CV) ^ sk_sw<DV>(r);
    doff[u] = (uint32_t)(r * DV + 8 * ch) * 2;
  }
  const uint32_t q_lds = lds_addr(&q_s[0][0]) + 1024 * v, do_lds = lds_addr(&do_s[0][0]) + 1024 * v;
  const uint32_t lse_lds = lds_addr(&lse_s[0][0]), dl_lds = lds_addr(&dl_s[0][0]), cnt_lds = lds_addr(&cnt_s[0][0]);
  struct StepLd {
    i4v rq, rd;
  };
  auto step_ld = [&](int i, int hb0, int bn) {
    const int nh = min(C::HB, p.G - hb0);
    const int64_t qrow = ((int64_t)b * p.Sq + i) * p.Hq + g * p.G + hb0;
    const int64_t l0 = ((int64_t)b * p.Hq + g * p.G + hb0) * p.Sq + i;
    if (v == 0) {
      const i4v rl = buf_rsrc((const float *)p.lse + l0, ((uint64_t)(nh - 1) * p.Sq + 1) * 4);
      if (lane < C::HB) b2lds4_at(rl, (uint32_t)(lane * p.Sq) * 4, lse_lds + bn * (C::HB * 4));
    } else {
      const i4v rl = buf_rsrc((const float *)p.ndelta + l0, ((uint64_t)(nh - 1) * p.Sq + 1) * 4);
      if (lane < C::HB) b2lds4_at(rl, (uint32_t)(lane * p.Sq) * 4, dl_lds + bn * (C::HB * 4));
      const int64_t e0 = (((int64_t)b * p.Hkv + g) * p.Sq + i) * skv_pad + j0;
      const int64_t ne = (int64_t)p.B * p.Hkv * p.Sq * skv_pad;
      const i4v rc = buf_rsrc(cnt + e0, (uint64_t)(ne - e0) * 2);
      if (lane < C::BM / 2) b2lds4_at(rc, (uint32_t)(4 * lane), cnt_lds + bn * (C::BM * 2));
    }
    return StepLd{buf_rsrc(p.q + qrow * DQK, (uint64_t)nh * DQK * 2), buf_rsrc(p.dout + qrow * DV, (uint64_t)nh * DV * 2)};
  };
  auto load_u = [&](const StepLd &L, int bn, int u) {
    if (u < C::LQ)
      b2lds16_at(L.rq, qoff[u], q_lds + bn * (TQ * 2) + 2048 * u);
    else
      b2lds16_at(L.rd, doff[u - C::LQ], do_lds + bn * (TD * 2) + 2048 * (u - C::LQ));
  };

  // dV += P^T dO and dK += dS^T Q of a staged step: M = 32 keys, N = 32-wide d blocks, K = the
  // step's 16 heads; A = the staging row of key lo (natural read), B = transposed reads of the
  // tiles.
  auto accumulate = [&](int bp, int sbp) {
    const s8v pa = *(const s8v *)&st_p[sbp][0][lo * C::HB + 8 * hi];
    const s8v da = *(const s8v *)&st_ds[sbp][0][lo * C::HB + 8 * hi];
    const s8v pl = SPLIT ? *(const s8v *)&st_p[sbp][NH - 1][lo * C::HB + 8 * hi] : s8v{};
    const s8v dl2 = SPLIT ? *(const s8v *)&st_ds[sbp][NH - 1][lo * C::HB + 8 * hi] : s8v{};
    constexpr int NP = C::NVW + C::NKK;
    // For bf16 the lo-half product of operand n runs after the hi-half product of operand n+1,
    // so that two products on one accumulator are never back to back.
    s8v prev_b = s8v{};
    int prev_n = -1;
    auto lo_product = [&](int n, s8v bb) {
      if (n < C::NVW) {
        av[n] = TT::mfma(pl, bb, av[n]);
      } else {
        const int u = n - C::NVW;
        ak[u] = TT::mfma(dl2, bb, ak[u]);
      }
    };
    ring_pipeline<NP, PF>(
        [&](int n) {
          if (n < C::NVW) return trB(do_s[bp], false, C::NVW * v + n);
          return trB(q_s[bp], true, kf + n - C::NVW);
        },
        [&](int n, s8v bb) {
          if (n < C::NVW) {
            av[n] = TT::mfma(pa, bb, av[n]);
          } else {
            const int u = n - C::NVW;
            ak[u] = TT::mfma(da, bb, ak[u]);
          }
          if (SPLIT) {
            if (prev_n >= 0) lo_product(prev_n, prev_b);
            prev_n = n;
            prev_b = bb;
          }
        });
    if (SPLIT) lo_product(prev_n, prev_b);
  };

  // Step 0's tiles; the staging buffer that step 0 reads as "step -1" holds zeros, so that every
  // step runs the same code (its products add exact zeros to the accumulators).
  {
    const StepLd L = step_ld(i_beg, 0, 0);
#pragma unroll
    for (int u = 0; u < C::NLD; u++) load_u(L, 0, u);
    const int lt = tid - 128;
    for (int e = 8 * lt; e < C::BM * C::HB * NH; e += 8 * 128) {
      *(s8v *)(&st_p[1][0][0] + e) = s8v{};
      *(s8v *)(&st_ds[1][0][0] + e) = s8v{};
    }
  }
  wait_vm0();
  __syncthreads();  // the first step's tiles landed, the zero staging written
  // Step t loads step t + 1 (the last step's rows again at the end, into a buffer no one reads
  // any more) and accumulates step t - 1.  (qi, hb) = that load's step.
  int b3 = 0, qi = i_beg, hb = 0;
  for (int t = 0; t <= nsteps; t++) {
    if (t + 1 < nsteps && ++hb == nhb) {
      hb = 0;
      qi++;
    }
    const int bn = b3 == 2 ? 0 : b3 + 1, bp = b3 == 0 ? 2 : b3 - 1;
    const StepLd L = step_ld(qi, hb * C::HB, bn);
#pragma unroll
    for (int u = 0; u < C::NLD; u++) load_u(L, bn, u);
    accumulate(t == 0 ? 0 : bp, (t + 1) & 1);
    wait_vm0();
    __syncthreads();  // step t+1's tiles landed; step t-1's tiles and staging consumed
    b3 = bn;
  }

  add_blocks(std::integral_constant<int, C::NVW>{}, av, dv_acc, DV, C::NVW * v);
  add_blocks(std::integral_constant<int, C::NKK>{}, ak, dk_acc, DQK, kf);
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
  // Query chunks of 256 queries (1,024 steps of 16 heads at 64 heads per KV head), counted from
  // the last query, so that every key block's first chunk is a full one and the grid runs
  // longest first.  Each chunk pays its K/V row loads and one f32 add of its block; on the
  // 4096 x 8192 top-k workload 192-256 queries measured best (128: +1%, 512: +4%, 1024: +19%).
  const int qchunk = 256;
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
