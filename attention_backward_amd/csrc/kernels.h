// kernels.h -- launchers of the attention-backward kernels (host side, C++).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace attn {

// delta [B,Hq,Sq] = rowsum(o * dout), Dv in {64, 128, 256, 512}; when lse_in is not null also
// lse_out = lse_in with -inf mapped to +inf (same layout).
hipError_t launch_delta(const short *o, const short *dout, float *delta, const float *lse_in, float *lse_out,
                        int64_t B, int64_t Sq, int64_t Hq, int64_t Dv, bool bf16, hipStream_t st);

// Dense path, D = Dqk = Dv in {64, 128}: dK/dV (KV-block owned) and dQ (query-block owned).
hipError_t launch_dense_dkdv(const Params &p, bool bf16, hipStream_t st);
hipError_t launch_dense_dq(const Params &p, bool bf16, hipStream_t st);

// Top-k path, (Dqk, Dv) = (576, 512): gathered backward adding dK/dV into f32 accumulators
// [B,Skv,Hkv,Dqk] / [B,Skv,Hkv,Dv] (zeroed first by launch_zero), then the landing pass
// out = storage(scale * acc) over n elements (n a multiple of 8).
hipError_t launch_zero(float *buf, int64_t n, hipStream_t st);
hipError_t launch_sparse_bwd(const Params &p, float *dk_acc, float *dv_acc, bool bf16, hipStream_t st);
hipError_t launch_land(const float *acc, short *out, int64_t n, float scale, bool bf16, hipStream_t st);

}  // namespace attn
