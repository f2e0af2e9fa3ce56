// common.h -- device-side types and helpers shared by the attention-backward kernels (gfx950).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_{f16,bf16}, wave64), measured on
// MI355X with an in-bounds probe:
//   A (32 x 16, M x K):  lane l holds A[m = l % 32][k = 8*(l/32) + e], e = 0..7
//   B (16 x 32, K x N):  lane l holds B[k = 8*(l/32) + e][n = l % 32]
//   C (32 x 32, f32):    lane l, register r holds C[m = 8*(r/4) + 4*(l/32) + r%4][n = l % 32]
// Because a contraction may use any order of its k index as long as A and B agree, the C block
// of one product can feed the next product directly: the 8 registers 8s..8s+7 of a lane cover
// the 16 rows m in {16s + 8*(e/4) + 4*(l/32) + e%4}, i.e. a permutation of 16s..16s+15.  The
// matching operand is read with ds_read_tr16_b64 (gfx950), which, within each group of 16
// lanes, takes four 16-element rows supplied by lanes 4r..4r+3 and hands lane i column i of
// those four rows -- two such reads give exactly the 8 permuted k values a lane needs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef short s8v __attribute__((ext_vector_type(8)));    // 8 x 16-bit: one MFMA A or B operand
typedef short s4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));  // one 32x32 f32 accumulator block
typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

struct Params {
  const short *q, *k, *v, *o, *dout;  // element bits of fp16/bf16
  const float *lse;                   // [B,Hq,Sq] base 2, -inf mapped to +inf (workspace copy)
  const float *lse_in;                // the caller's lse (dense dQ kernel: input of its prologue)
  float *lse_ws;                      // the workspace copy the dense dQ kernel writes
  float *ndelta;                      // [B,Hq,Sq] workspace: minus rowsum(o * dout) (the negation
                                      // lets dP accumulators start from it: dP - delta for free)
  const int32_t *idx;                 // [B,Sq,Hkv,topk] or null
  short *dq, *dk, *dv;
  int B, Sq, Skv, Hq, Hkv, G, topk, Dqk, Dv;
  int v_ld;                           // elements between consecutive V rows: Dv, or Dqk when V is
                                      // the first Dv columns of each K row (shared-latent form)
  int causal, window;
  float scale;                        // softmax scale
  float c;                            // scale * log2(e)
  const int32_t *cu;                  // packed sequences: [nseq + 1] token offsets, or null
  int nseq, max_seqlen;               // packed sequences: their number and a bound on each length
  int hsplit = 1;                     // packed dK/dV: items sharing one key block's query heads
  float *dk_acc = nullptr;            // hsplit > 1: f32 [hsplit][tokens, Hkv, D] slices, one per
  float *dv_acc = nullptr;            //   part (plain stores; the landing pass adds them)
  int64_t acc_slice = 0;              // elements per slice (tokens * Hkv * D)
  int *work = nullptr;                // dK/dV work-queue counter (zeroed), or null
  // bf16 calls computed in fp16: the inputs are fp16 copies scaled by powers of two, and the
  // factors that undo those scales live in device memory: [0] the exponent scale c, [1] the dQ
  // output factor, [2] the dK factor, [3] the dV factor, [4] the factor that brings dS back to its
  // own scale before its fp16 rounding (null: c and scale above, dV factor 1).
  const float *rescale = nullptr;
};

// The sequence one workgroup works on.  Dense: batch s of equal-length sequences.  Packed (cu not
// null, batch of one): tokens [cu[s], cu[s+1]) of the token axis, with Sq = Skv = T.  Offsets are
// clamped into [0, T] and lengths to max_seqlen, so no offset table can move an access out of its
// buffer.  lse/delta index of (head h, row i): l0 + h * Sq_total + i.
struct SeqView {
  int64_t q0, k0;  // token index of row 0 of the query and the key rows
  int64_t l0;
  int Sq, Skv;
};
__device__ __forceinline__ SeqView seq_view(const int32_t *cu, int s, int Sq_total, int Skv_total, int Hq,
                                            int max_seqlen) {
  SeqView v;
  if (cu) {
    const int bos = min(max(__builtin_amdgcn_readfirstlane(cu[s]), 0), Sq_total);
    const int eos = min(max(__builtin_amdgcn_readfirstlane(cu[s + 1]), bos), Sq_total);
    v.q0 = v.k0 = v.l0 = bos;
    v.Sq = v.Skv = min(eos - bos, max_seqlen);
  } else {
    v.q0 = (int64_t)s * Sq_total;
    v.k0 = (int64_t)s * Skv_total;
    v.l0 = (int64_t)s * Hq * Sq_total;
    v.Sq = Sq_total;
    v.Skv = Skv_total;
  }
  return v;
}

// SPLIT: whether P and dS enter their MFMA products (dV += P^T dO, dK += dS^T Q, dQ += dS K) as
// hi + lo halves.  bf16 keeps 8 mantissa bits, so one rounding costs up to 2^-9 relative per
// term; over the long sums of dK, dQ and dV that exceeds the 5e-3 / 1e-2 tolerance against the
// f64 oracle (measured), while hi = bf16(x), lo = bf16(x - hi) carries 16 bits.  fp16's 11 bits
// need no split.
struct F16 {
  static constexpr bool SPLIT = false;
  static constexpr bool RESCALED = false;  // inputs are scaled copies (Factors::ds applies)
  static __device__ __forceinline__ f16v mfma(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ short cvt(float x) { return __builtin_bit_cast(short, (_Float16)x); }
  static __device__ __forceinline__ float tof(short x) { return (float)__builtin_bit_cast(_Float16, x); }
  static __device__ __forceinline__ short cvt_out(float x) { return cvt(x); }  // dq, dk, dv
};

struct BF16 {
  static constexpr bool SPLIT = true;
  static constexpr bool RESCALED = false;
  static __device__ __forceinline__ f16v mfma(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ short cvt(float x) { return __builtin_bit_cast(short, (__bf16)x); }
  static __device__ __forceinline__ float tof(short x) {
    return __builtin_bit_cast(float, ((unsigned)(unsigned short)x) << 16);
  }
  static __device__ __forceinline__ short cvt_out(float x) { return cvt(x); }
};

// bf16 calls re-expressed in fp16: operands and products in fp16 (no hi + lo split: P and dS are
// rounded once to fp16's 11 bits, as on the fp16 path), outputs rounded to bf16.
struct F16B : F16 {
  static constexpr bool RESCALED = true;
  static __device__ __forceinline__ short cvt_out(float x) { return BF16::cvt(x); }
};

// Four values into elements e0 .. e0 + 3 (e0 a multiple of 4) of an MFMA A operand, with their
// low halves when TT::SPLIT.  The fp16 forms convert two values per instruction into one 32-bit
// word of the operand.
template <class TT>
__device__ __forceinline__ void put4(s8v &a, s8v &l, int e0, f4v x) {
  if constexpr (TT::SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const short xh = TT::cvt(x[i]);
      a[e0 + i] = xh;
      l[e0 + i] = TT::cvt(x[i] - TT::tof(xh));
    }
  } else {
    typedef int i4w __attribute__((ext_vector_type(4)));
    const h2v lo2 = {(_Float16)x[0], (_Float16)x[1]}, hi2 = {(_Float16)x[2], (_Float16)x[3]};
    i4w w = __builtin_bit_cast(i4w, a);
    w[e0 / 2] = __builtin_bit_cast(int, lo2);
    w[e0 / 2 + 1] = __builtin_bit_cast(int, hi2);
    a = __builtin_bit_cast(s8v, w);
  }
}

// The exponent scale c and the output factors of a call: from device memory when the inputs were
// re-expressed, else c, scale (dQ and dK) and 1 (dV).
struct Factors {
  float c, dq, dk, dv, ds;
};
__device__ __forceinline__ Factors factors(const Params &p) {
  if (p.rescale) return Factors{p.rescale[0], p.rescale[1], p.rescale[2], p.rescale[3], p.rescale[4]};
  return Factors{p.c, p.scale, p.scale, 1.f, 1.f};
}
// dS = P (dP - delta) in its own scale: with rescaled inputs the difference carries s_do s_v.
template <class TT>
__device__ __forceinline__ float ds_of(float p, float dp_minus_delta, const Factors &f) {
  return TT::RESCALED ? p * dp_minus_delta * f.ds : p * dp_minus_delta;
}

__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposed LDS read of four 16-bit values (see the header comment).
__device__ __forceinline__ s4v lds_tr4(const short *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v *)(p));
}

// The same reads at an LDS byte address: written as (lane base + compile-time offset), the
// constant folds into the instruction's offset field instead of costing an add per read.
__device__ __forceinline__ s4v lds_tr4_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v *)(size_t)a);
}
__device__ __forceinline__ s8v lds_rd16_at(uint32_t a) { return *(__attribute__((address_space(3))) s8v *)(size_t)a; }

// A value the compiler must treat as computed here: keeps it from hoisting (address + constant)
// sums out of a loop into one register each, which would cost an add per read inside the loop.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// sbase + voff as one add the compiler cannot see into: it keeps the compiler from hoisting
// (address + constant) sums out of a loop into one register each, which would cost an add per
// read inside the loop; with this the constants fold into the reads' offset fields.
__device__ __forceinline__ uint32_t lds_base_add(uint32_t sbase, uint32_t voff) {
  uint32_t r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(__builtin_amdgcn_readfirstlane(sbase)), "v"(voff));
  return r;
}

__device__ __forceinline__ s8v cat8(s4v a, s4v b) { return s8v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

// LDS tiles are stored without row padding; the 16-byte chunk c of row R sits at chunk
// c ^ swz<D>(R).  gfx950's LDS serves 256 bytes (64 banks) per cycle, i.e. 16 lanes of a
// ds_read_b128 or 32 lanes of a ds_read_tr16_b64 (measured: the transposed reads of these
// kernels run at 62 / 119 / 192 B/clk/CU with no swizzle / a 32-bank swizzle / this one).
//   D = 128 (256-byte rows, one per bank line): swz takes 16 distinct values over 16 aligned
//     rows (the 16 lanes of a b128 read of one chunk hit 16 distinct chunk positions), and
//     swz/4 takes 4 distinct values over 4 aligned rows (the 32 lanes of a transposed read
//     cover 4 rows x 4 chunks, which land in 4 disjoint groups of 4 positions).
//   D = 64 (128-byte rows, two per bank line): the row parity picks the half line and
//     swz(R) = f(R/2) with f bijective on 8 values, and f(x), f(x+1) differing in bit 2 for
//     even x, which gives the same two properties.
template <int D>
__device__ __forceinline__ int swz(int row) {
  static_assert(D == 64 || D == 128, "swizzle defined for 64- and 128-wide rows");
  if (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Asynchronous copy global -> LDS (global_load_lds): lane l of the wave writes lds_base + 16*l
// (or 4*l).  lds_base must be wave-uniform; completion is tracked by vmcnt only (wait_vm0 below,
// then a barrier before other waves read the data).
// The instruction is issued from inline assembly on purpose: when the compiler sees an LDS DMA it
// makes every later LDS read wait for all outstanding vector-memory operations unless it can
// prove the two do not alias, which it cannot for a buffer picked at run time -- that turned
// each step's prefetch of the next tile into a full stall before the step's first LDS read.
// The kernels never read a buffer that has a copy in flight (they wait and synchronise first),
// so no such wait is needed.  M0 carries the LDS base; one wait state separates its write from
// the load.  Waits the compiler places for its own loads stay correct: loads complete in order,
// so an extra load in flight can only make such a wait longer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void g2lds16(const void *g, void *lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base))), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void g2lds4(const void *g, void *lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base))), "v"(g)
               : "memory", "m0");
}
// The same copies through a buffer resource (buffer_load ... lds): measured on MI355X, a wave
// issuing global_load_lds_dwordx4 moves about 5 B/clk (about 20 B/clk for four waves of a CU),
// while buffer_load_dwordx4 ... lds, like plain vector loads, reaches the CU's ~60 B/clk with four
// waves.  The resource covers `bytes` bytes from a wave-uniform `base` (loads beyond read 0);
// each lane passes its byte offset from base.  Waits as for g2lds16 (vmcnt).
typedef int i4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i4v buf_rsrc(const void *base, uint64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i4v r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0: raw bytes
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes > 0xffffffffull ? 0xffffffffull : bytes));
  r[3] = 0x00020000;  // 32-bit data format, no swizzle
  return r;
}
__device__ __forceinline__ void b2lds16(i4v r, uint32_t voff, void *lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base))), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void b2lds4(i4v r, uint32_t voff, void *lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base))), "v"(voff), "s"(r)
               : "memory", "m0");
}
// The same copies to an LDS byte address the caller computed once (no pointer conversion per
// copy); `voff` is the lane's byte offset from the resource base.
__device__ __forceinline__ void b2lds16_at(i4v r, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void b2lds4_at(i4v r, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(voff), "s"(r)
               : "memory", "m0");
}
// A 16-byte load into registers through a buffer resource over `bytes` bytes from `base`:
// offsets past the end read as zero, with no select on the loaded value (which would keep the
// load's destination registers apart from the variable they end in).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_v(const void *base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ s8v buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(s8v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Wait for every outstanding vector-memory operation (vmcnt = 0; expcnt and lgkmcnt left at their
// no-wait maxima in the gfx9 encoding).  Issued through the builtin so that the compiler's own
// wait placement knows the loads it issued itself are complete from here on.
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Keeps the compiler's scheduler from moving instructions across this point: an operand read
// issued ahead of the products that consume it stays ahead of them (the scheduler otherwise
// sinks such reads next to their use to save registers, which exposes the LDS latency).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Software pipeline over N operand loads: ld(n) is issued PF uses ahead of use(n, value), through
// a ring of PF + 1 registers; the fences keep the compiler from sinking the loads to their uses.
template <int N, int PF, class Ld, class Use>
__device__ __forceinline__ void ring_pipeline(Ld ld, Use use) {
  using T = decltype(ld(0));
  T ring[PF + 1];
#pragma unroll
  for (int n = 0; n < PF && n < N; n++) ring[n] = ld(n);
#pragma unroll
  for (int n = 0; n < N; n++) {
    if (n + PF < N) ring[(n + PF) % (PF + 1)] = ld(n + PF);
    sched_fence();
    use(n, ring[n % (PF + 1)]);
  }
}

// Wave priority around MFMA sections (a scheduling hint between the waves sharing a SIMD: the
// wave feeding the matrix core issues first, its partner's vector work fills the gaps).
#ifndef ATTN_MFMA_PRIO
#define ATTN_MFMA_PRIO 0
#endif
__device__ __forceinline__ void mfma_prio_hi() {
  if (ATTN_MFMA_PRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void mfma_prio_lo() {
  if (ATTN_MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
}

// lse as the kernels use it: a row with lse = -inf (no allowed key) must give p = 0, so it is
// mapped to +inf; exp2(x - inf) = 0.
__device__ __forceinline__ float lse_fix(float l) { return l == -__builtin_inff() ? __builtin_inff() : l; }

}  // namespace attn
