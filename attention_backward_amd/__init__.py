"""MI355X-native fused softmax-attention backward.

The computation lives in libattn_bwd.so (hand-written HIP kernels for gfx950, C ABI declared
in include/attn_bwd.h); this package is its ctypes binding plus the seeded input generator.

    from attention_backward_amd import backward, forward
    o, lse = forward(q, k, v, causal=True)               # dense masks, D in {64, 128}
    dq, dk, dv = backward(q, k, v, o, dout, lse, causal=True)

q [B,Sq,Hq,Dqk], k [B,Skv,Hkv,Dqk], v [B,Skv,Hkv,Dv], o/dout [B,Sq,Hq,Dv] fp16 or bf16 on the
GPU; lse [B,Hq,Sq] float32, base 2 (natural-log LSE times log2(e)).  backward() also takes a
sliding window (window=), a top-k key list per query (topk_idx=, Dqk 576 / Dv 512); packed
variable-length sequences go through make_args(..., cu_seqlens=, max_seqlen=) + attn_bwd_ex and
attn_fwd_varlen.
"""
from __future__ import annotations

import math

import torch

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    AttnBwdError,
    attn_bwd,
    attn_bwd_args,
    attn_bwd_delta,
    attn_bwd_ex,
    attn_bwd_noalloc,
    attn_bwd_strerror,
    attn_bwd_workspace_size,
    attn_fwd,
    attn_fwd_varlen,
    load,
    make_args,
)


def backward(q, k, v, o, dout, lse, *, causal=True, window=0, topk_idx=None, scale=None, workspace=None,
             stream=None, out=None):
    """Allocate dq/dk/dv (and the workspace, with torch) and run attn_bwd_ex on the current stream."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    args = make_args(q, k, v, o, dout, lse, dq, dk, dv, scale=scale, causal=causal, window=window,
                     topk_idx=topk_idx, workspace=workspace, stream=stream)
    if workspace is None:
        need = attn_bwd_workspace_size(args)
        if need == 0:
            attn_bwd_ex(args)  # raises with the validation status
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace, args.workspace_bytes = ws.data_ptr(), need
    attn_bwd_ex(args)
    return dq, dk, dv


def forward(q, k, v, *, causal=True, window=0, scale=None, stream=None):
    """Allocate o and lse (with torch) and run attn_fwd on the current stream: the O and base-2 lse
    the backward takes."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, scale, causal=causal, window=window, stream=stream)
    return o, lse
