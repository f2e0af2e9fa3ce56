// kernels.h -- launchers of the attention-backward kernels (host side, C++).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace attn {

// Phase timestamps without extra stream packets: arm_events(start, stop) hands the two events to
// the next kernel that launch() starts on this thread, which takes them as its dispatch
// timestamps (start when it begins, stop when it ends; either may be null).  settle_events()
// records, as ordinary stream events, whichever of them no kernel took.
struct ArmedEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ArmedEvents &armed_events();  // per host thread
inline void arm_events(hipEvent_t start, hipEvent_t stop) { armed_events() = ArmedEvents{start, stop}; }
hipError_t settle_events(hipStream_t st);
template <class F, class... A>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, A... args) {
  ArmedEvents &ev = armed_events();
  if (ev.start || ev.stop) {
    const ArmedEvents take = ev;
    ev = ArmedEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, take.start, take.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

// Arithmetic of a call: fp16; bf16 with hi + lo operands for P and dS; or bf16 inputs re-expressed
// as fp16 copies scaled by powers of two (fp16 products, bf16 outputs, p.rescale set).
enum : int { ARITH_F16 = 0, ARITH_BF16 = 1, ARITH_F16B = 2 };

// delta [B,Hq,Sq] = rowsum(o * dout) (negated when `negate`), Dv in {64, 128, 256, 512}; when
// lse_in is not null also lse_out = lse_in with -inf mapped to +inf (same layout).
hipError_t launch_delta(const short *o, const short *dout, float *delta, const float *lse_in, float *lse_out,
                        bool negate, int64_t B, int64_t Sq, int64_t Hq, int64_t Dv, bool bf16, hipStream_t st);

// Dense path, D = Dqk = Dv in {64, 128}: dK/dV (KV-block owned) and dQ (query-block owned).
hipError_t launch_dense_dkdv(const Params &p, int arith, hipStream_t st);
hipError_t launch_dense_dq(const Params &p, int arith, hipStream_t st);
// Packed calls with the head group split in two (p.hsplit = 2): dk/dv = DT(slice 0 + slice 1) of
// the f32 dK/dV slices, over the rows of each sequence only.
hipError_t launch_land_parts(const Params &p, int arith, hipStream_t st);

// Arguments of the forward kernel (O and the base-2 lse from Q, K, V).
struct FwdParams {
  const short *q, *k, *v;  // element bits of fp16/bf16, BSHD
  short *o;                // [B,Sq,Hq,D]
  float *lse;              // [B,Hq,Sq], base 2
  int B, Sq, Skv, Hq, Hkv, G;
  int causal, window;
  float c;                 // scale * log2(e)
  const int32_t *cu;       // packed sequences: [nseq + 1] token offsets, or null
  int nseq, max_seqlen;
};

// Forward (the step before the backward): O and the base-2 lse, D in {64, 128}.
hipError_t launch_dense_fwd(const FwdParams &p, int D, bool bf16, hipStream_t st);

// Top-k path, (Dqk, Dv) = (576, 512):
//   launch_zero        zero-fills n floats (n a multiple of 4): the accumulators and count mask;
//   launch_topk_count  cnt [B,Hkv,Sq,skv_pad] u16 = occurrences of each key in each valid list;
//   launch_sparse_dq   gathered, query-owned dQ;
//   launch_sparse_dkdv key-owned dK/dV weighted by cnt, added into f32 accumulators
//                      [B,Skv,Hkv,Dqk] / [B,Skv,Hkv,Dv];
//   launch_land        out = storage(scale * acc) over n elements (n a multiple of 8); with
//                      rescale set the factor is rescale[which] instead of scale;
//   launch_land_kv     out [rows, Dqk] = storage(scale * dk_acc + [dv_acc, 0]) (shared-latent dKV;
//                      with rescale: rescale[2] * dk_acc + rescale[3] * [dv_acc, 0]).
hipError_t launch_zero(float *buf, int64_t n, hipStream_t st);
// Rows of up to kCountRowLdsMax bytes are counted one list per workgroup in LDS and written whole
// (no zero-fill needed); longer rows use global atomics on a zero-filled mask.
constexpr int kCountRowLdsMax = 65536;
bool topk_count_by_rows(int skv_pad);
hipError_t launch_topk_count(const int32_t *idx, uint16_t *cnt, int64_t B, int64_t Sq, int64_t Skv, int64_t Hkv,
                             int64_t topk, int skv_pad, int causal, hipStream_t st);
hipError_t launch_sparse_dq(const Params &p, int arith, hipStream_t st);
hipError_t launch_sparse_dkdv(const Params &p, const uint16_t *cnt, int skv_pad, float *dk_acc, float *dv_acc, int arith,
                              hipStream_t st);
hipError_t launch_land(const float *acc, short *out, int64_t n, float scale, const float *rescale, int which, bool bf16,
                       hipStream_t st);
hipError_t launch_land_kv(const float *dk_acc, const float *dv_acc, short *out, int64_t rows, int64_t Dqk, int64_t Dv,
                          float scale, const float *rescale, bool bf16, hipStream_t st);

// Re-expression of bf16 inputs in fp16.  Tensors: 0 q, 1 k, 2 v (with o, which shares v's
// scale), 3 dout.  launch_f16_prepass: maxbits[4][kMaxSlots] (zeroed by the caller) = the largest
// bf16 magnitudes of each group, spread over slots; then one power-of-two scale per group, the
// factors rescale[5] that undo them (exponent scale, dQ, dK, dV, dS) and the scaled fp16 copies.
constexpr int kMaxSlots = 64;
struct F16Copy {
  const short *src;  // bf16
  short *dst;        // fp16 copy
  int64_t n;         // elements (a multiple of 8)
  int group;         // which scale
};
hipError_t launch_f16_prepass(const F16Copy *copies, int ncopies, unsigned *maxbits, float *scales, float *rescale,
                              float c, float scale, hipStream_t st);

}  // namespace attn
