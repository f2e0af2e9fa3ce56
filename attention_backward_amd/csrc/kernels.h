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

}  // namespace attn
