// preprocess.hip -- delta = rowsum(O * dO), the first step of the backward.
//
// TileOPs PR #2281 page, "TileFoundry Description": delta_rows reduces O*dO over the head dim in
// f32 and the main kernel reads it per query row.  The page measured a preprocess that was 8x
// slower in bf16 than fp16 on its old code; here both dtypes take the same path: every lane
// loads 16 contiguous bytes of O and of dO (rows are contiguous in BSHD, so a wave reads
// 1 KiB runs), widens to f32, multiplies and reduces across the Dv/8 lanes of its row with
// cross-lane shuffles.  HBM-bound: 2*Dv*sizeof(T) bytes read and 4 bytes written per row.
#include "common.h"
#include "kernels.h"

namespace attn {

// Also copies lse (when lse_in is not null) into the workspace with -inf replaced by +inf: a row
// whose lse is -inf has no allowed key and must contribute nothing, and exp2(x - inf) = 0
// gives exactly that without a per-element test in the main kernels.
template <class TT, int DV>
__global__ __launch_bounds__(256) void delta_kernel(const short *__restrict__ o, const short *__restrict__ dout,
                                                    float *__restrict__ delta, const float *__restrict__ lse_in,
                                                    float *__restrict__ lse_out, float sgn, int64_t rows, int Sq,
                                                    int Hq) {
  constexpr int TPR = DV / 8;       // lanes per row (16 bytes each)
  constexpr int RPB = 256 / TPR;    // rows per block per iteration
  const int sub = threadIdx.x % TPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR; row < rows; row += (int64_t)gridDim.x * RPB) {
    const s8v a = *(const s8v *)(o + row * DV + 8 * sub);
    const s8v d = *(const s8v *)(dout + row * DV + 8 * sub);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) acc += TT::tof(a[e]) * TT::tof(d[e]);
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (sub == 0) {
      const int64_t h = row % Hq;
      const int64_t i = (row / Hq) % Sq;
      const int64_t b = row / ((int64_t)Hq * Sq);
      const int64_t x = (b * Hq + h) * Sq + i;
      delta[x] = sgn * acc;
      if (lse_in) lse_out[x] = lse_fix(lse_in[x]);
    }
  }
}

template <class TT, int DV>
static hipError_t launch_delta_t(const short *o, const short *dout, float *delta, const float *lse_in, float *lse_out,
                                 bool negate, int64_t B, int64_t Sq, int64_t Hq, hipStream_t st) {
  constexpr int RPB = 256 / (DV / 8);
  const int64_t rows = B * Sq * Hq;
  int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  launch((delta_kernel<TT, DV>), dim3((unsigned)blocks), dim3(256), 0, st, o, dout, delta, lse_in, lse_out,
                     negate ? -1.f : 1.f, rows, (int)Sq, (int)Hq);
  return hipGetLastError();
}

hipError_t launch_delta(const short *o, const short *dout, float *delta, const float *lse_in, float *lse_out,
                        bool negate, int64_t B, int64_t Sq, int64_t Hq, int64_t Dv, bool bf16, hipStream_t st) {
#define DISPATCH_DV(N)                                                                       \
  case N:                                                                                    \
    return bf16 ? launch_delta_t<BF16, N>(o, dout, delta, lse_in, lse_out, negate, B, Sq, Hq, st)    \
                : launch_delta_t<F16, N>(o, dout, delta, lse_in, lse_out, negate, B, Sq, Hq, st);
  switch (Dv) {
    DISPATCH_DV(64)
    DISPATCH_DV(128)
    DISPATCH_DV(256)
    DISPATCH_DV(512)
    default:
      return hipErrorInvalidValue;
  }
#undef DISPATCH_DV
}

}  // namespace attn
