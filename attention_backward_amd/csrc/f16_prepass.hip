// f16_prepass.hip -- bf16 inputs re-expressed as fp16 copies scaled by powers of two.
//
// In bf16 the P and dS operands of the dV, dK and dQ products must enter their MFMAs as hi + lo
// halves to meet the 5e-3 / 1e-2 tolerance against the f64 oracle over long sums (8 mantissa
// bits per rounding are not enough), which doubles those products.  fp16 carries 11 bits, so one
// rounding suffices there.  A bf16 value times a power of two is exactly representable in fp16
// while the result stays in fp16's normal range, so each input tensor is copied to fp16 with one
// power-of-two scale chosen from its largest magnitude (largest scaled value below 2^15); the
// fp16 kernels then run on the copies, and the factors that undo the scales are applied to the
// exponent (S' = s_q s_k S), to dS before its fp16 rounding (dP' - delta' = s_do s_v (dP - delta),
// so dS = P (dP' - delta') / (s_do s_v) enters the dK and dQ products exactly as on the fp16 path)
// and to the outputs (dQ = scale dQ' / s_k, dK = scale dK' / s_q, dV = dV' / s_do).  O shares V's
// scale, so that delta' = rowsum(O' dO') = s_v s_do delta matches dP'; an O row is a convex
// combination of V rows, and its magnitude is included in that scale's maximum anyway.
// Values more than about 2^28 below their tensor's largest magnitude fall into fp16's subnormal
// range; their absolute error stays below 2^-40 of that largest magnitude.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace attn {

constexpr int kMaxCopies = 5;
static_assert(kMaxSlots > 0, "largest-magnitude slots per group");
struct F16CopySet {
  F16Copy c[kMaxCopies];
};

// maxbits[group][slot] = max over the group's tensors of the bf16 bits with the sign cleared, which
// order like the magnitudes (inf and NaN above every finite value).  Atomics on one address retire
// one at a time (about 10 ns each, measured), so the workgroup reduces in registers and LDS first
// and its one atomic goes to slot blockIdx.x % kMaxSlots of its group; the finalize pass reduces
// the slots.
__global__ __launch_bounds__(256) void absmax_kernel(const F16CopySet cs, unsigned *__restrict__ maxbits) {
  __shared__ unsigned wmax[4];
  const F16Copy c = cs.c[blockIdx.y];
  const int64_t n8 = c.n / 8;
  unsigned m = 0;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8; v += (int64_t)gridDim.x * 256) {
    const s8v x = *(const s8v *)(c.src + 8 * v);
#pragma unroll
    for (int e = 0; e < 8; e++) m = max(m, (unsigned)(unsigned short)x[e] & 0x7fffu);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m != 0) atomicMax(&maxbits[c.group * kMaxSlots + blockIdx.x % kMaxSlots], m);
  }
}

// One power of two per group: 2^e with e = 15 - E where max = f 2^E, f in [0.5, 1), so the largest
// scaled magnitude is below 2^15 (fp16's largest finite value is 65504); e is kept within +-40 so
// that the products of scales stay finite in f32.  An all-zero or non-finite group keeps scale 1.
__global__ void f16_finalize_kernel(const unsigned *__restrict__ maxbits, float *__restrict__ scales,
                                    float *__restrict__ rescale, float c, float scale, int v_is_k) {
  if (threadIdx.x != 0) return;
  float s[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    unsigned mb = 0;
    for (int k = 0; k < kMaxSlots; k++) mb = max(mb, maxbits[t * kMaxSlots + k]);
    const float m = __uint_as_float(mb << 16);
    int e = 0;
    if (m > 0.f && m <= 3.3895314e38f) {
      int E;
      frexpf(m, &E);
      e = min(40, max(-40, 15 - E));
    }
    s[t] = ldexpf(1.f, e);
  }
  if (v_is_k) s[2] = s[1];  // shared-latent form: V is part of K's rows and carries its scale
#pragma unroll
  for (int t = 0; t < 4; t++) scales[t] = s[t];
  rescale[0] = c / (s[0] * s[1]);   // S' = s_q s_k S
  rescale[1] = scale / s[1];        // dQ' = sum dS K' = s_k dQ / scale
  rescale[2] = scale / s[0];        // dK' = sum dS Q' = s_q dK / scale
  rescale[3] = 1.f / s[3];          // dV' = sum P dO' = s_do dV
  rescale[4] = 1.f / (s[3] * s[2]); // dS = P (dP' - delta') / (s_do s_v)
}

__global__ __launch_bounds__(256) void to_f16_kernel(const F16CopySet cs, const float *__restrict__ scales) {
  const F16Copy c = cs.c[blockIdx.y];
  if (!c.dst) return;
  const float s = scales[c.group];
  const int64_t n8 = c.n / 8;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8; v += (int64_t)gridDim.x * 256) {
    const s8v x = *(const s8v *)(c.src + 8 * v);
    s8v y;
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = F16::cvt(BF16::tof(x[e]) * s);
    *(s8v *)(c.dst + 8 * v) = y;
  }
}

hipError_t launch_f16_prepass(const F16Copy *copies, int ncopies, unsigned *maxbits, float *scales, float *rescale,
                              float c, float scale, hipStream_t st) {
  if (ncopies < 1 || ncopies > kMaxCopies) return hipErrorInvalidValue;
  F16CopySet cs{};
  int64_t nmax = 0;
  bool v_is_k = true;
  for (int i = 0; i < ncopies; i++) {
    if (copies[i].n % 8 != 0 || copies[i].group < 0 || copies[i].group > 3) return hipErrorInvalidValue;
    cs.c[i] = copies[i];
    nmax = copies[i].n > nmax ? copies[i].n : nmax;
    if (copies[i].group == 2 && copies[i].dst) v_is_k = false;  // a V copy of its own
  }
  int64_t blocks = (nmax / 8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)ncopies);
  launch(absmax_kernel, grid, dim3(256), 0, st, cs, maxbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(f16_finalize_kernel, dim3(1), dim3(64), 0, st, maxbits, scales, rescale, c, scale, (int)v_is_k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(to_f16_kernel, grid, dim3(256), 0, st, cs, scales);
  return hipGetLastError();
}

}  // namespace attn
