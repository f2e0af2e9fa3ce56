/*
 * attn_bwd.h -- C ABI of libattn_bwd.so, the fused softmax-attention backward for AMD gfx950
 * (MI355X).
 *
 * The operation (TileOPs PR #2281 page, "TileFoundry Description", the Reference program; MHA is
 * the grouped-query op with Hkv = Hq, as the same page's summary says):
 *
 *   given q, k, v, the forward output o, its gradient dout and the forward's base-2 log-sum-exp
 *   lse, compute for every batch b, query head h (KV head g = h / (Hq/Hkv)) and query row i
 *     delta_i = sum_d o[i,d] * dout[i,d]
 *     p_ij    = exp2(scale * log2(e) * (q_i . k_j) - lse_i)   for keys j allowed to row i, else 0
 *     ds_ij   = p_ij * (dout_i . v_j - delta_i)
 *     dq_i    = scale * sum_j ds_ij k_j
 *     dk_j    = scale * sum_(h in g) sum_i ds_ij q_i      (summed over the G query heads of g)
 *     dv_j    =         sum_(h in g) sum_i p_ij dout_i
 *
 * Allowed keys of query row i, with off = Skv - Sq (bottom-right alignment):
 *   dense:   causal   => j <= i + off
 *            window>0 => j >  i + off - window   (window = number of visible keys including the
 *                                                 diagonal; flash-linear-attention issue #8,
 *                                                 sliding-window GQA)
 *   top-k:   the entries of topk_idx[b, i, g, 0..topk) (TileLang PR #2592, sparse MLA backward),
 *            once per occurrence; entries < 0, >= Skv, or (causal) > i + off are ignored.
 * A row with no allowed key, or with lse = -inf, contributes nothing.  Key rows that no query
 * reaches get dk = dv = 0.  dk and dv are produced directly at Hkv heads, with no Hq-shaped
 * intermediate (flash-linear-attention issue #8, KV-head-owned dK/dV).
 *
 * Layouts (row-major, contiguous, "BSHD"):
 *   q    [B, Sq,  Hq,  Dqk]    k  [B, Skv, Hkv, Dqk]    v  [B, Skv, Hkv, Dv]
 *   o    [B, Sq,  Hq,  Dv ]    dout like o              lse [B, Hq, Sq]  float32, base 2
 *   dq like q, dk like k, dv like v; element type = dtype (fp16 or bf16) for all of them.
 *   topk_idx [B, Sq, Hkv, topk] int32, or NULL for the dense path.
 *
 * Ownership and execution:
 *   - every pointer is a DEVICE pointer owned by the caller; inputs are never written;
 *   - all work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream);
 *     the call never synchronises, results are ready once the caller synchronises the stream;
 *   - every element of dq, dk and dv is written on every successful call;
 *   - the library keeps no state between calls: calls with distinct outputs and workspaces are
 *     independent and may run concurrently on different streams.
 *
 * Errors: arguments are validated on the host before anything is enqueued.  On error nothing
 * is enqueued, the outputs are untouched and a negative attn_status is returned;
 * attn_bwd_strerror() describes it (for ATTN_E_HIP, with the HIP error string of the last
 * failing call on this thread).
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_DT_F16 = 0, ATTN_DT_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVAL = -1,        /* a null/misaligned pointer, a negative size, Hq % Hkv != 0, ... */
  ATTN_E_UNSUPPORTED = -2,  /* a valid request this build has no kernel for (head dims, dtype) */
  ATTN_E_WORKSPACE = -3,    /* workspace NULL or smaller than attn_bwd_workspace_size()       */
  ATTN_E_HIP = -4           /* a HIP runtime call or kernel launch failed                      */
} attn_status;

/* Full argument set.  Sizes are int64; Sq != Skv and Dqk != Dv are allowed where a kernel
 * exists: dense (Dqk, Dv) in {(64,64), (128,128)}; top-k (Dqk, Dv) = (576, 512) with
 * Skv * Hkv * Dqk * 2 < 2^32, topk <= 65535 and a key-count mask of B * Hkv * Sq * (Skv rounded
 * up to 32) 16-bit counts of at most 1 GiB (ATTN_E_UNSUPPORTED otherwise). */
typedef struct {
  const void *q, *k, *v, *o, *dout; /* 16-byte aligned device pointers, element type = dtype   */
  const float *lse;                 /* [B, Hq, Sq] float32, base-2 log-sum-exp of the forward   */
  const int32_t *topk_idx;          /* NULL => dense; else [B, Sq, Hkv, topk] int32            */
  void *dq, *dk, *dv;               /* outputs, 16-byte aligned, element type = dtype          */
  int64_t B, Sq, Skv, Hq, Hkv, Dqk, Dv, topk;
  float scale;                      /* softmax scale (finite, > 0), typically 1/sqrt(Dqk)      */
  int32_t causal;                   /* 0 or 1                                                  */
  int32_t window;                   /* 0 = no window; > 0 requires causal = 1 and no topk_idx  */
  int32_t dtype;                    /* attn_dtype                                              */
  void *workspace;                  /* caller-allocated device scratch of workspace_bytes, 256-byte
                                       aligned, at least attn_bwd_workspace_size() bytes; NULL or
                                       a smaller size returns ATTN_E_WORKSPACE (the library
                                       allocates nothing)                                        */
  size_t workspace_bytes;
  void *stream;                     /* hipStream_t                                             */
  void *events;                     /* optional, NULL or an array of 4 hipEvent_t created by the
                                       caller, marking on `stream` the phase boundaries: dense =
                                       the start of the call's first kernel (the dQ kernel,
                                       which also forms delta and the lse copy, or the bf16
                                       pre-pass) | the end of the dQ kernel | the end of the
                                       dK/dV kernel | the end of the landing pass of a split
                                       packed call (else recorded right after the dK/dV
                                       kernel); top-k = the start of the preprocess | the end
                                       of the dQ kernel (after the zero-fill and the key
                                       counts) | the end of the dK/dV kernel | the end of the
                                       landing passes.  Events at kernel ends and starts are
                                       taken as those kernels' dispatch timestamps
                                       (hipExtLaunchKernel), with no extra stream packets; the
                                       work is unchanged                                        */
  int32_t kv_shared;                /* 0, or 1 for the shared-latent form of the top-k path (the
                                       TileLang PR #2592 page's sparse MLA op, which returns dq and
                                       dkv): k holds [B,Skv,Hkv,Dqk] rows whose first Dv columns are
                                       V, v and dv must be NULL, and dk receives dKV = dK + [dV, 0],
                                       the gradient with respect to that one tensor.  Requires
                                       topk_idx and Dv <= Dqk.                                   */
  const int32_t *cu_seqlens;        /* NULL, or packed variable-length sequences on the dense
                                       path (flash-linear-attention issue #8: packed varlen with
                                       per-sequence BOS/EOS offsets): a 4-byte aligned device
                                       array of nseq + 1 non-decreasing token offsets, 0 first and
                                       Sq last.  Then B = 1, Sq = Skv = T (the packed length),
                                       every tensor is the batch-of-one layout above (q [1,T,Hq,Dqk],
                                       lse [1,Hq,T], ...), and sequence s is tokens
                                       [cu_seqlens[s], cu_seqlens[s+1]): each is its own attention
                                       problem, the masks taken within it (off = 0).  Offsets are
                                       clamped into [0, T] on the device, so a bad table cannot
                                       move an access out of the buffers, but tokens outside
                                       [0, cu_seqlens[nseq]) and past max_seqlen of a longer
                                       sequence are then left unwritten.                        */
  int64_t nseq;                     /* packed: number of sequences (>= 1); else 0              */
  int64_t max_seqlen;               /* packed: a bound on every sequence length, 1..T (sizes the
                                       grid; a longer sequence is cut there); else 0            */
  int32_t bf16_arith;               /* bf16 calls only (ignored for fp16): ATTN_BF16_AUTO, or
                                       ATTN_BF16_SPLIT: bf16 products, with P and dS entering
                                       them as hi + lo bf16 halves; or ATTN_BF16_FP16: the inputs
                                       are copied to fp16 with one power-of-two scale per tensor
                                       (exact for values within 2^28 of the tensor's largest
                                       magnitude, which lands just below 2^15), the fp16
                                       kernels run on the copies, and dq, dk, dv come back in
                                       bf16 with the scales undone.  AUTO takes FP16 when the
                                       second products of the split form (4 Dqk flops per
                                       attended pair) are estimated to cost more than three
                                       passes over q, k, v, o and dout.  FP16 adds scaled
                                       copies of q, k, v, o and dout to the workspace.          */
} attn_bwd_args;

enum { ATTN_BF16_AUTO = 0, ATTN_BF16_SPLIT = 1, ATTN_BF16_FP16 = 2 };

/* Bytes of workspace the call needs for these sizes (0 if the arguments are invalid), as
 * 256-byte aligned parts:
 *   delta (stored negated) and a sanitised copy of lse, [B,Hq,Sq] f32 each;
 *   top-k only: f32 accumulators dK_acc [B,Skv,Hkv,Dqk] and dV_acc [B,Skv,Hkv,Dv] and the
 *   16-bit key counts [B,Hkv,Sq,Skv rounded up to 32];
 *   packed sequences without a window: when Hq / Hkv is even, two f32 slices each of dK and dV,
 *   [T,Hkv,D] (each half of a head group stores its block into its own slice with plain stores,
 *   and a landing pass adds slice 0 and slice 1 in that order), then 256 bytes for the dK/dV
 *   work-queue counter.
 * Never an Hq-shaped dK/dV buffer, and no atomics on the dense dK/dV.  Dense results (dq, dk, dv)
 * are identical between identical calls.  Top-k results: dq is written once per element; dk and
 * dv (or dKV in the shared-latent form) are sums of f32 atomic additions (one per key block and
 * query chunk), so their last bits may differ between identical calls.  The shared-latent form
 * needs the same workspace. */
size_t attn_bwd_workspace_size(const attn_bwd_args *a);

/* The backward for the full argument set.  Returns an attn_status. */
int attn_bwd_ex(const attn_bwd_args *a);

/* The backward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): attn_bwd_ex with the workspace taken
 * from a static device array of ATTN_NOALLOC_SCRATCH_BYTES that each GPU the library runs on
 * holds until the process ends; a->workspace and a->workspace_bytes are ignored.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine); on its first call on a
 * device it looks up that device's copy of the array.  Arguments, validation and results are
 * those of attn_bwd_ex; a call whose attn_bwd_workspace_size() exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES returns ATTN_E_WORKSPACE before anything is enqueued.  Every call
 * on one GPU shares that GPU's array (the kernels clear what must start at zero), so calls that
 * overlap on one GPU -- on different streams or from different threads -- race and must be
 * ordered by the caller. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_bwd_noalloc(const attn_bwd_args *a);

/* The same operation with Sq = Skv = S and Dqk = Dv = D, arguments in the order
 *   q, k, v, o, dout, lse, dq, dk, dv, B, S, Hq, Hkv, D, scale, causal, window, topk_idx,
 * followed by what the plain list cannot carry: topk, dtype, workspace, workspace_bytes, stream.
 * A single S and D cannot describe the top-k kernel's shapes (Sq != Skv, Dqk = 576 != Dv = 512):
 * with topk_idx set it returns ATTN_E_UNSUPPORTED; use attn_bwd_ex for that path. */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float scale,
             int32_t causal, int32_t window, const int32_t *topk_idx, int64_t topk, int32_t dtype, void *workspace,
             size_t workspace_bytes, void *stream);

/* Only the first step of the backward: delta [B,Hq,Sq] = rowsum(o * dout) in f32, enqueued on
 * `stream`.  o and dout [B,Sq,Hq,Dv] with Dv in {64, 128, 256, 512}; delta 16-byte aligned. */
int attn_bwd_delta(const void *o, const void *dout, float *delta, int64_t B, int64_t Sq, int64_t Hq, int64_t Dv,
                   int32_t dtype, void *stream);

/* The forward pass whose outputs the backward consumes: o and the base-2 lse from q, k, v (the
 * TileOPs PR #2281 page's Reference program defines lse over scores scaled by scale * log2(e)):
 *   lse_i = log2 sum_j exp2(c q_i . k_j),  o_i = sum_j exp2(c q_i . k_j - lse_i) v_j,
 *   c = scale * log2(e), over the keys j allowed to row i by the dense masks above (causal,
 *   window; GQA head h reads KV head h / (Hq/Hkv)).  A row with no allowed key gets o = 0 and
 *   lse = -inf.
 * q [B,Sq,Hq,D], k and v [B,Skv,Hkv,D], o [B,Sq,Hq,D] of dtype with D in {64, 128} (other D:
 * ATTN_E_UNSUPPORTED); lse [B,Hq,Sq] float32, 4-byte aligned; q, k, v, o 16-byte aligned device
 * pointers owned by the caller.  Softmax statistics are kept in f32, P enters the O product in the
 * element type.  Enqueued on `stream`, no workspace, no synchronisation; every element of o and
 * lse is written.  Returns ATTN_E_INVAL for null or misaligned pointers, sizes < 1,
 * Hq % Hkv != 0, causal not 0/1, window < 0, window > 0 without causal, scale not finite and
 * positive, or an unknown dtype. */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t Sq, int64_t Skv,
             int64_t Hq, int64_t Hkv, int64_t D, float scale, int32_t causal, int32_t window, int32_t dtype,
             void *stream);

/* attn_fwd over packed variable-length sequences: q, o [1,T,Hq,D], k, v [1,T,Hkv,D], lse [1,Hq,T],
 * and cu_seqlens, nseq and max_seqlen as in attn_bwd_args (sequence s is tokens
 * [cu_seqlens[s], cu_seqlens[s+1]), each its own attention problem).  Validation as attn_fwd,
 * plus ATTN_E_INVAL for a null or misaligned cu_seqlens, nseq < 1, or max_seqlen outside 1..T. */
int attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu_seqlens,
                    int64_t nseq, int64_t max_seqlen, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                    int32_t causal, int32_t window, int32_t dtype, void *stream);

/* Static description of a status code (never NULL).  For ATTN_E_HIP the string includes the
 * HIP error text of the last failure on the calling thread. */
const char *attn_bwd_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
