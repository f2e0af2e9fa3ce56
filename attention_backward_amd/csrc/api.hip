// api.hip -- the extern "C" boundary of libattn_bwd.so (declared in include/attn_bwd.h).
//
// Validates every argument on the host before anything is enqueued, carves the caller's
// workspace, and enqueues the kernels on the caller's stream:
//   dense:  dQ (query-block owned; its prologue forms delta and the lse copy) -> dK/dV
//           (KV-block owned, stored once at Hkv); packed calls without a window: dK/dV on a work
//           queue, with an even head group split in two halves whose f32 slices a landing pass
//           adds in a fixed order and casts;
//   top-k:  zero the f32 dK/dV accumulators and the key-count mask, delta, count the keys of
//           every list -> gathered dQ (query-owned) -> dK/dV (key-owned, weighted by the
//           counts, added into the accumulators) -> landing (scale, cast).
// The library allocates nothing and keeps no state between calls.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "attn_bwd.h"
#include "kernels.h"

namespace attn {
ArmedEvents &armed_events() {
  static thread_local ArmedEvents ev;
  return ev;
}
hipError_t settle_events(hipStream_t st) {
  ArmedEvents &ev = armed_events();
  const ArmedEvents left = ev;
  ev = ArmedEvents{};
  hipError_t e = hipSuccess;
  if (left.start) e = hipEventRecord(left.start, st);
  if (e == hipSuccess && left.stop) e = hipEventRecord(left.stop, st);
  return e;
}
}  // namespace attn

#ifndef ATTN_TOPK_MASK_MAX
#define ATTN_TOPK_MASK_MAX ((int64_t)1 << 30)  // bytes of the top-k key-count mask
#endif

namespace {

thread_local char g_msg[512];

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int set_hip_error(hipError_t e, const char *what) {
  snprintf(g_msg, sizeof(g_msg), "HIP error in %s: %s", what, hipGetErrorString(e));
  return ATTN_E_HIP;
}

// Structural validation (no pointers dereferenced, no HIP calls).
int validate_sizes(const attn_bwd_args *a) {
  if (!a) return ATTN_E_INVAL;
  if (a->B < 1 || a->Sq < 1 || a->Skv < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1) return ATTN_E_INVAL;
  if (a->Hq % a->Hkv != 0) return ATTN_E_INVAL;
  if (a->causal != 0 && a->causal != 1) return ATTN_E_INVAL;
  if (a->window < 0) return ATTN_E_INVAL;
  if (a->window > 0 && (!a->causal || a->topk_idx)) return ATTN_E_INVAL;
  if (a->topk_idx && a->topk < 1) return ATTN_E_INVAL;
  if (!a->topk_idx && a->topk != 0) return ATTN_E_INVAL;
  if (!(a->scale > 0.f) || !isfinite(a->scale)) return ATTN_E_INVAL;
  if (a->dtype != ATTN_DT_F16 && a->dtype != ATTN_DT_BF16) return ATTN_E_INVAL;
  if (a->kv_shared != 0 && a->kv_shared != 1) return ATTN_E_INVAL;
  if (a->bf16_arith < ATTN_BF16_AUTO || a->bf16_arith > ATTN_BF16_FP16) return ATTN_E_INVAL;
  if (a->kv_shared && !a->topk_idx) return ATTN_E_UNSUPPORTED;  // the dense kernels have no shared form
  if (a->cu_seqlens) {
    // Packed sequences: a batch of one on the dense path, each sequence its own problem.
    if (((uintptr_t)a->cu_seqlens & 3) != 0 || a->B != 1 || a->Sq != a->Skv || a->topk_idx) return ATTN_E_INVAL;
    if (a->nseq < 1 || a->max_seqlen < 1 || a->max_seqlen > a->Sq) return ATTN_E_INVAL;
    if (a->nseq * a->Hq * a->max_seqlen >= ((int64_t)1 << 31)) return ATTN_E_UNSUPPORTED;  // grid size
  } else if (a->nseq != 0 || a->max_seqlen != 0) {
    return ATTN_E_INVAL;
  }
  // 32-bit row indices inside the kernels: every row count must fit comfortably.
  const int64_t lim = (int64_t)1 << 31;
  if (a->B * a->Sq * a->Hq >= lim || a->B * a->Skv * a->Hkv >= lim) return ATTN_E_UNSUPPORTED;
  if (a->topk_idx) {
    if (a->topk > 65535) return ATTN_E_UNSUPPORTED;  // 16-bit key counts
    // The key-count mask holds one 16-bit count per (batch, KV head, query, key).
    if (a->B * a->Hkv * a->Sq * ((a->Skv + 31) / 32 * 32) * 2 > ATTN_TOPK_MASK_MAX) return ATTN_E_UNSUPPORTED;
    if (!(a->Dqk == 576 && a->Dv == 512)) return ATTN_E_UNSUPPORTED;
    // The gathers address one (batch, KV head)'s K or V rows with 32-bit byte offsets.
    if (a->Skv * a->Hkv * a->Dqk * 2 >= ((int64_t)1 << 32)) return ATTN_E_UNSUPPORTED;
  } else if (!((a->Dqk == 64 && a->Dv == 64) || (a->Dqk == 128 && a->Dv == 128))) {
    return ATTN_E_UNSUPPORTED;
  }
  return ATTN_OK;
}

// Workspace, each part 256-byte aligned: delta [B,Hq,Sq] f32, the sanitised lse [B,Hq,Sq] f32,
// and for the top-k path the accumulators dK_acc [B,Skv,Hkv,Dqk] and dV_acc [B,Skv,Hkv,Dv] f32
// and the key counts cnt [B,Hkv,Sq,skv_pad] u16 (skv_pad = Skv rounded up to 32).  Packed calls
// on the dK/dV work queue: [two f32 slices each of dK and dV, [T,Hkv,D], when the head group is
// split,] then the queue counter.
size_t row_stat_bytes(const attn_bwd_args *a) { return align256((size_t)(a->B * a->Hq * a->Sq) * sizeof(float)); }
size_t dk_acc_bytes(const attn_bwd_args *a) { return align256((size_t)(a->B * a->Skv * a->Hkv * a->Dqk) * 4); }
size_t dv_acc_bytes(const attn_bwd_args *a) { return align256((size_t)(a->B * a->Skv * a->Hkv * a->Dv) * 4); }
int64_t skv_pad(const attn_bwd_args *a) { return (a->Skv + 31) / 32 * 32; }
size_t cnt_bytes(const attn_bwd_args *a) { return align256((size_t)(a->B * a->Hkv * a->Sq * skv_pad(a)) * 2); }
#ifndef ATTN_PACKED_QUEUE
#define ATTN_PACKED_QUEUE 1
#endif
// dK/dV work queue.  Packed calls without a window take their key blocks from a device counter:
// their lengths differ, so a fixed block-to-CU mapping leaves CUs idle behind the longest
// sequence.  When the head group splits in two, each item holds one half and stores its f32
// block with plain stores into its own slice [T, Hkv, D]; the landing pass adds slice 0 and
// slice 1 in that order, so the result is deterministic and no atomics are involved.  Dense
// batches keep one workgroup per key block, which stores dK/dV once at Hkv.
bool dkdv_queue(const attn_bwd_args *a) {
  return ATTN_PACKED_QUEUE && a->cu_seqlens && !a->topk_idx && a->window == 0;
}
int dkdv_hsplit(const attn_bwd_args *a) { return dkdv_queue(a) && (a->Hq / a->Hkv) % 2 == 0 ? 2 : 1; }
size_t part_bytes(const attn_bwd_args *a) { return align256((size_t)(a->B * a->Skv * a->Hkv * a->Dqk) * 4 * 2); }
size_t queue_bytes(const attn_bwd_args *a) {
  if (!dkdv_queue(a)) return 0;
  return 256 + (dkdv_hsplit(a) > 1 ? 2 * part_bytes(a) : 0);
}
// bf16 calls re-expressed in fp16 (f16_prepass.hip): a 1280-byte block (largest magnitudes in
// 4 x 64 slots, scales and the factors that undo them) and scaled fp16 copies of q, k, v (none in
// the shared-latent form, where V is part of K's rows), o and dout.
constexpr size_t kF16xHeader = 1280;  // maxbits [4][64] u32, then scales[4] and rescale[5] f32
// Automatic choice between the two bf16 forms, from a cost estimate.  The hi + lo form adds the
// second P and dS products, 4 Dqk flops per (query, key, head) pair; they measured about
// 1.2 PFLOP/s.  The re-expression costs three passes over q, k, v, o and dout, which measured about
// 6.5 TB/s, plus a few launches.  Keys per query: the list length, the window, half the keys
// under a causal mask, or all of them (packed calls: of the longest sequence).
bool f16x(const attn_bwd_args *a) {
  if (a->dtype != ATTN_DT_BF16) return false;
  if (a->bf16_arith == ATTN_BF16_FP16) return true;
  if (a->bf16_arith != ATTN_BF16_AUTO) return false;
  const double skv = (double)(a->cu_seqlens ? a->max_seqlen : a->Skv);
  const double kpq = a->topk_idx ? (double)a->topk
                     : a->window > 0 ? (a->window < skv ? (double)a->window : skv)
                     : a->causal ? skv / 2 : skv;
  const double pairs = (double)a->B * a->Sq * a->Hq * kpq;
  const double nq = (double)a->B * a->Sq * a->Hq, nk = (double)a->B * a->Skv * a->Hkv;
  const double bytes = 2.0 * (nq * a->Dqk + nk * a->Dqk + (a->kv_shared ? 0.0 : nk * a->Dv) + 2.0 * nq * a->Dv);
  const double split_s = 4.0 * a->Dqk * pairs / 1.2e15;
  const double copy_s = 3.0 * bytes / 6.5e12 + 15e-6;
  return split_s > copy_s;
}
size_t f16x_bytes(const attn_bwd_args *a) {
  if (!f16x(a)) return 0;
  const size_t nq = (size_t)(a->B * a->Sq * a->Hq), nk = (size_t)(a->B * a->Skv * a->Hkv);
  size_t n = kF16xHeader + align256(nq * a->Dqk * 2) + align256(nk * a->Dqk * 2) + 2 * align256(nq * a->Dv * 2);
  if (!a->kv_shared) n += align256(nk * a->Dv * 2);
  return n;
}
size_t workspace_bytes_for(const attn_bwd_args *a) {
  size_t n = 2 * row_stat_bytes(a) + f16x_bytes(a);
  if (a->topk_idx) n += dk_acc_bytes(a) + dv_acc_bytes(a) + cnt_bytes(a);
  return n + queue_bytes(a);
}

// The forward for dense batches (cu null) and packed sequences (cu set: B = 1, Sq = Skv = T).
int run_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t Sq, int64_t Skv,
            int64_t Hq, int64_t Hkv, int64_t D, float scale, int32_t causal, int32_t window, int32_t dtype,
            const int32_t *cu, int64_t nseq, int64_t max_seqlen, void *stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3) != 0) return ATTN_E_INVAL;
  if (B < 1 || Sq < 1 || Skv < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return ATTN_E_INVAL;
  if ((causal != 0 && causal != 1) || window < 0 || (window > 0 && !causal)) return ATTN_E_INVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_E_INVAL;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16) return ATTN_E_INVAL;
  if (D != 64 && D != 128) return ATTN_E_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (B * Sq * Hq >= lim || B * Skv * Hkv >= lim) return ATTN_E_UNSUPPORTED;
  if (cu && nseq * Hq * max_seqlen >= lim) return ATTN_E_UNSUPPORTED;  // grid size
  attn::FwdParams p;
  p.q = (const short *)q;
  p.k = (const short *)k;
  p.v = (const short *)v;
  p.o = (short *)o;
  p.lse = lse;
  p.B = (int)B;
  p.Sq = (int)Sq;
  p.Skv = (int)Skv;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.G = (int)(Hq / Hkv);
  p.causal = causal;
  p.window = window;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.cu = cu;
  p.nseq = (int)nseq;
  p.max_seqlen = (int)max_seqlen;
  const hipError_t e = attn::launch_dense_fwd(p, (int)D, dtype == ATTN_DT_BF16, (hipStream_t)stream);
  attn::armed_events() = attn::ArmedEvents{};  // nothing left armed for a later call on this thread
  if (e != hipSuccess) return set_hip_error(e, "kernel launch");
  return ATTN_OK;
}

// Pointer and flag checks of a call (after validate_sizes): non-null, aligned inputs and outputs;
// in the shared-latent form v and dv must be NULL (V is read from k, dV is added into dk).
int validate_ptrs(const attn_bwd_args *a) {
  const bool shared = a->kv_shared != 0;
  if (shared && (a->v || a->dv)) return ATTN_E_INVAL;
  const void *ptrs[] = {a->q, a->k, shared ? a->k : a->v, a->o, a->dout, a->lse, a->dq, a->dk, shared ? a->dk : a->dv};
  for (const void *p : ptrs)
    if (!p || !aligned16(p)) return ATTN_E_INVAL;
  if (a->topk_idx && ((uintptr_t)a->topk_idx & 3) != 0) return ATTN_E_INVAL;
  return ATTN_OK;
}

// The backward on a validated argument set, with `ws` a device workspace of at least
// workspace_bytes_for(a) bytes, 256-byte aligned.
int run_bwd(const attn_bwd_args *a, void *ws) {
  const bool shared = a->kv_shared != 0;
  hipStream_t st = (hipStream_t)a->stream;
  const bool bf16 = a->dtype == ATTN_DT_BF16;
  const int arith = !bf16 ? attn::ARITH_F16 : f16x(a) ? attn::ARITH_F16B : attn::ARITH_BF16;
  // The re-expressed inputs sit at the end of the workspace.
  char *fx = (char *)ws + workspace_bytes_for(a) - f16x_bytes(a);

  attn::Params p;
  p.q = (const short *)a->q;
  p.k = (const short *)a->k;
  p.v = (const short *)(shared ? a->k : a->v);
  p.v_ld = (int)(shared ? a->Dqk : a->Dv);
  p.o = (const short *)a->o;
  p.dout = (const short *)a->dout;
  p.ndelta = (float *)ws;
  p.lse = (const float *)((char *)ws + row_stat_bytes(a));
  p.idx = a->topk_idx;
  p.dq = (short *)a->dq;
  p.dk = (short *)a->dk;
  p.dv = shared ? nullptr : (short *)a->dv;
  p.B = (int)a->B;
  p.Sq = (int)a->Sq;
  p.Skv = (int)a->Skv;
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.G = (int)(a->Hq / a->Hkv);
  p.topk = (int)a->topk;
  p.Dqk = (int)a->Dqk;
  p.Dv = (int)a->Dv;
  p.causal = a->causal;
  p.window = a->window;
  p.scale = a->scale;
  p.c = (float)((double)a->scale * 1.4426950408889634);

  p.lse_in = a->lse;
  p.lse_ws = (float *)p.lse;
  p.cu = a->cu_seqlens;
  p.nseq = (int)a->nseq;
  p.max_seqlen = (int)a->max_seqlen;

  // Phase events ride on the kernels' own dispatch timestamps (no extra stream packets): the
  // call's first kernel takes ev[0] as its start, and the kernel ending each phase its stop.
  hipEvent_t *ev = (hipEvent_t *)a->events;
  hipError_t e = hipSuccess;
  auto phase_end = [&](hipEvent_t stop) {  // arm the next kernel's stop, keeping a pending start
    if (ev) attn::armed_events().stop = stop;
  };
  auto settle = [&]() {
    if (ev && e == hipSuccess) e = attn::settle_events(st);
  };
  if (ev) attn::arm_events(ev[0], nullptr);
  if (arith == attn::ARITH_F16B) {
    // Scaled fp16 copies of the inputs; the kernels then read them and the factors in `rescale`.
    unsigned *maxbits = (unsigned *)fx;
    float *scales = (float *)(fx + 4 * 4 * attn::kMaxSlots), *rescale = scales + 4;
    const size_t nq = (size_t)(a->B * a->Sq * a->Hq), nk = (size_t)(a->B * a->Skv * a->Hkv);
    char *cur = fx + kF16xHeader;
    auto take = [&](size_t elems) {
      short *r = (short *)cur;
      cur += align256(elems * 2);
      return r;
    };
    short *q16 = take(nq * a->Dqk), *k16 = take(nk * a->Dqk);
    short *v16 = shared ? k16 : take(nk * a->Dv);
    short *o16 = take(nq * a->Dv), *do16 = take(nq * a->Dv);
    attn::F16Copy cp[5];
    int ncp = 0;
    cp[ncp++] = attn::F16Copy{p.q, q16, (int64_t)(nq * a->Dqk), 0};
    cp[ncp++] = attn::F16Copy{p.k, k16, (int64_t)(nk * a->Dqk), 1};
    if (!shared) cp[ncp++] = attn::F16Copy{p.v, v16, (int64_t)(nk * a->Dv), 2};
    cp[ncp++] = attn::F16Copy{p.o, o16, (int64_t)(nq * a->Dv), shared ? 1 : 2};  // O carries V's scale
    cp[ncp++] = attn::F16Copy{p.dout, do16, (int64_t)(nq * a->Dv), 3};
    if (e == hipSuccess) e = attn::launch_zero((float *)fx, 4 * attn::kMaxSlots, st);  // the slots
    if (e == hipSuccess) e = attn::launch_f16_prepass(cp, ncp, maxbits, scales, rescale, p.c, p.scale, st);
    p.q = q16;
    p.k = k16;
    p.v = v16;
    p.o = o16;
    p.dout = do16;
    p.rescale = rescale;
  }
  if (!a->topk_idx) {
    // The dQ kernel forms delta and the lse copy in its prologue, so it runs first.
    phase_end(ev ? ev[1] : nullptr);
    if (e == hipSuccess) e = attn::launch_dense_dq(p, arith, st);
    settle();
    if (dkdv_queue(a)) {
      char *qb = (char *)ws + 2 * row_stat_bytes(a);
      p.hsplit = dkdv_hsplit(a);
      if (p.hsplit > 1) {
        p.dk_acc = (float *)qb;
        p.dv_acc = (float *)(qb + part_bytes(a));
        p.acc_slice = a->B * a->Skv * a->Hkv * a->Dqk;
      }
      p.work = (int *)(qb + queue_bytes(a) - 256);
      // Only the counter starts at zero: every slice row inside a sequence is stored by its item.
      if (e == hipSuccess) e = attn::launch_zero((float *)p.work, 64, st);
    }
    phase_end(ev ? ev[2] : nullptr);
    if (e == hipSuccess) e = attn::launch_dense_dkdv(p, arith, st);
    settle();
    if (p.hsplit > 1) {
      phase_end(ev ? ev[3] : nullptr);
      if (e == hipSuccess) e = attn::launch_land_parts(p, arith, st);
      settle();
    } else if (e == hipSuccess && ev) {
      e = hipEventRecord(ev[3], st);  // no landing: the call ends with the dK/dV kernel
    }
  } else {
    if (e == hipSuccess)
      e = attn::launch_delta(p.o, p.dout, p.ndelta, a->lse, (float *)p.lse, true, a->B, a->Sq, a->Hq, a->Dv,
                             arith == attn::ARITH_BF16, st);
    float *dk_acc = (float *)((char *)ws + 2 * row_stat_bytes(a));
    float *dv_acc = (float *)((char *)dk_acc + dk_acc_bytes(a));
    uint16_t *cnt = (uint16_t *)((char *)dv_acc + dv_acc_bytes(a));
    const int64_t nk = a->B * a->Skv * a->Hkv * a->Dqk, nv = a->B * a->Skv * a->Hkv * a->Dv;
    // contiguous; the count rows need no zero-fill when each is written whole
    const size_t zero_bytes =
        dk_acc_bytes(a) + dv_acc_bytes(a) + (attn::topk_count_by_rows((int)skv_pad(a)) ? 0 : cnt_bytes(a));
    if (e == hipSuccess) e = attn::launch_zero(dk_acc, (int64_t)(zero_bytes / 4), st);
    if (e == hipSuccess)
      e = attn::launch_topk_count(a->topk_idx, cnt, a->B, a->Sq, a->Skv, a->Hkv, a->topk, (int)skv_pad(a), a->causal,
                                  st);
    phase_end(ev ? ev[1] : nullptr);
    if (e == hipSuccess) e = attn::launch_sparse_dq(p, arith, st);
    settle();
    phase_end(ev ? ev[2] : nullptr);
    if (e == hipSuccess) e = attn::launch_sparse_dkdv(p, cnt, (int)skv_pad(a), dk_acc, dv_acc, arith, st);
    settle();
    if (shared) {
      phase_end(ev ? ev[3] : nullptr);
      if (e == hipSuccess)
        e = attn::launch_land_kv(dk_acc, dv_acc, p.dk, a->B * a->Skv * a->Hkv, a->Dqk, a->Dv, a->scale, p.rescale, bf16,
                                 st);
    } else {
      if (e == hipSuccess) e = attn::launch_land(dk_acc, p.dk, nk, a->scale, p.rescale, 2, bf16, st);
      phase_end(ev ? ev[3] : nullptr);
      if (e == hipSuccess) e = attn::launch_land(dv_acc, p.dv, nv, 1.0f, p.rescale, 3, bf16, st);
    }
    settle();
  }
  if (e != hipSuccess) return set_hip_error(e, "kernel launch");
  return ATTN_OK;
}

// Device scratch of attn_bwd_noalloc: one file-scope array that each GPU the library runs on
// holds until the process ends.  Host code never uses its name as an address (on the host it is
// only a stand-in for the symbol); it takes the device address once per device, with that device
// current, from hipGetSymbolAddress, and passes that pointer to the kernels.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch address on the current device (set up on its first call there), or an error.
int scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return ATTN_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return set_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & 255) != 0) return set_hip_error(hipErrorInvalidSymbol, "scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_size(const attn_bwd_args *a) {
  if (validate_sizes(a) != ATTN_OK) return 0;
  return workspace_bytes_for(a);
}

int attn_bwd_ex(const attn_bwd_args *a) {
  int rc = validate_sizes(a);
  if (rc == ATTN_OK) rc = validate_ptrs(a);
  if (rc != ATTN_OK) return rc;
  // The caller provides the workspace (the library allocates nothing).
  const size_t need = workspace_bytes_for(a);
  if (!a->workspace || a->workspace_bytes < need) return ATTN_E_WORKSPACE;
  if (((uintptr_t)a->workspace & 255) != 0) return ATTN_E_INVAL;
  return run_bwd(a, a->workspace);
}

int attn_bwd_noalloc(const attn_bwd_args *a) {
  int rc = validate_sizes(a);
  if (rc == ATTN_OK) rc = validate_ptrs(a);
  if (rc != ATTN_OK) return rc;
  if (workspace_bytes_for(a) > kScratchBytes) return ATTN_E_WORKSPACE;
  void *ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != ATTN_OK) return rc;
  return run_bwd(a, ws);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse, void *dq,
             void *dk, void *dv, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float scale, int32_t causal,
             int32_t window, const int32_t *topk_idx, int64_t topk, int32_t dtype, void *workspace,
             size_t workspace_bytes, void *stream) {
  attn_bwd_args a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.topk_idx = topk_idx;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Sq = S;
  a.Skv = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Dqk = D;
  a.Dv = D;
  a.topk = topk;
  a.scale = scale;
  a.causal = causal;
  a.window = window;
  a.dtype = dtype;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = stream;
  return attn_bwd_ex(&a);
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t Sq, int64_t Skv,
             int64_t Hq, int64_t Hkv, int64_t D, float scale, int32_t causal, int32_t window, int32_t dtype,
             void *stream) {
  return run_fwd(q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, scale, causal, window, dtype, nullptr, 0, 0, stream);
}

int attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu_seqlens,
                    int64_t nseq, int64_t max_seqlen, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                    int32_t causal, int32_t window, int32_t dtype, void *stream) {
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3) != 0) return ATTN_E_INVAL;
  if (nseq < 1 || max_seqlen < 1 || max_seqlen > T) return ATTN_E_INVAL;
  return run_fwd(q, k, v, o, lse, 1, T, T, Hq, Hkv, D, scale, causal, window, dtype, cu_seqlens, nseq, max_seqlen,
                 stream);
}

int attn_bwd_delta(const void *o, const void *dout, float *delta, int64_t B, int64_t Sq, int64_t Hq, int64_t Dv,
                   int32_t dtype, void *stream) {
  if (!o || !dout || !delta || !aligned16(o) || !aligned16(dout) || !aligned16(delta)) return ATTN_E_INVAL;
  if (B < 1 || Sq < 1 || Hq < 1) return ATTN_E_INVAL;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16) return ATTN_E_INVAL;
  if (Dv != 64 && Dv != 128 && Dv != 256 && Dv != 512) return ATTN_E_UNSUPPORTED;
  hipError_t e = attn::launch_delta((const short *)o, (const short *)dout, delta, nullptr, nullptr, false, B, Sq, Hq, Dv,
                                    dtype == ATTN_DT_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return set_hip_error(e, "delta launch");
  return ATTN_OK;
}

const char *attn_bwd_strerror(int status) {
  switch (status) {
    case ATTN_OK:
      return "success";
    case ATTN_E_INVAL:
      return "invalid argument (null or misaligned pointer, bad size, Hq % Hkv != 0, bad flag combination)";
    case ATTN_E_UNSUPPORTED:
      return "unsupported: no kernel for this head-dim / variant in this build";
    case ATTN_E_WORKSPACE:
      return "workspace missing or smaller than attn_bwd_workspace_size() (attn_bwd_ex), or the call needs more "
             "than ATTN_NOALLOC_SCRATCH_BYTES of static scratch (attn_bwd_noalloc)";
    case ATTN_E_HIP:
      return g_msg[0] ? g_msg : "HIP runtime error";
    default:
      return "unknown status";
  }
}

}  // extern "C"
