"""Forward pass that produces the backward's inputs O and lse -- TEST INFRASTRUCTURE ONLY.

The backward takes O and the base-2 log-sum-exp of a forward pass as inputs (TileOPs PR #2281
page, the Reference program's signature).  For workloads too large for the plain C loop in
attn_oracle.c, this module evaluates the same masked softmax with torch's CPU matmul as the one
library primitive.  Each query row's softmax is still taken over that row's whole key set in one
piece: rows are only evaluated in groups so that the score matrix fits in memory.

    s_ij  = q_i . k_j * scale * log2(e)          over the allowed keys j of row i
    lse_i = log2 sum_j 2^(s_ij)                  (base 2; -inf for a row with no allowed key)
    o_i   = sum_j 2^(s_ij - lse_i) v_j           (0 for a row with no allowed key)

The allowed key sets are the same as attn_oracle.c's: bottom-right causal alignment, a window
of `window` keys ending at the diagonal, or the listed top-k keys (one term per occurrence,
entries outside [0, Skv) or past the causal diagonal dropped).
"""
from __future__ import annotations

import math

import torch

LOG2E = 1.4426950408889634


def _dense_rows(qq, kk, vv, i0, i1, off, causal, window, c):
    """Forward for query rows [i0, i1) of one (b, h) against one KV head's keys."""
    Skv = kk.shape[0]
    jmax = min(Skv, i1 - 1 + off + 1) if causal else Skv
    jmin = max(0, i0 + off - window + 1) if window > 0 else 0
    n = i1 - i0
    if jmax <= jmin:
        return torch.zeros((n, vv.shape[1]), dtype=qq.dtype), torch.full((n,), -math.inf, dtype=qq.dtype)
    s = (qq @ kk[jmin:jmax].T) * c
    ii = torch.arange(i0, i1).unsqueeze(1)
    jj = torch.arange(jmin, jmax).unsqueeze(0)
    allowed = torch.ones(s.shape, dtype=torch.bool)
    if causal:
        allowed &= jj <= ii + off
    if window > 0:
        allowed &= jj > ii + off - window
    return _softmax_rows(s, allowed, vv[jmin:jmax])


def _softmax_rows(s, allowed, vsel):
    s = torch.where(allowed, s, torch.tensor(-math.inf, dtype=s.dtype))
    m = s.amax(dim=-1, keepdim=True)
    empty = torch.isinf(m) & (m < 0)
    m = torch.where(empty, torch.zeros_like(m), m)
    w = torch.exp2(s - m)  # exactly 0 where masked
    tot = w.sum(dim=-1, keepdim=True)
    o = (w @ vsel) if vsel.dim() == 2 else torch.bmm(w, vsel)
    o = torch.where(empty, torch.zeros_like(o), o / torch.where(empty, torch.ones_like(tot), tot))
    lse = torch.where(empty, torch.full_like(m, -math.inf), m + torch.log2(tot))
    return o, lse.squeeze(-1)


def fwd(q, k, v, scale, causal=True, window=0, idx=None, dtype=torch.float64, rows=512):
    """Masked softmax forward.  q [B,Sq,Hq,Dqk], k [B,Skv,Hkv,Dqk], v [B,Skv,Hkv,Dv] (CPU tensors of
    any float dtype, widened exactly); idx [B,Sq,Hkv,topk] int or None.
    Returns o [B,Sq,Hq,Dv] and lse [B,Hq,Sq] in `dtype`."""
    B, Sq, Hq, _ = q.shape
    Skv, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    off = Skv - Sq
    c = scale * LOG2E
    o = torch.empty((B, Sq, Hq, Dv), dtype=dtype)
    lse = torch.empty((B, Hq, Sq), dtype=dtype)
    for b in range(B):
        for g in range(Hkv):
            kk = k[b, :, g, :].to(dtype).contiguous()
            vv = v[b, :, g, :].to(dtype).contiguous()
            if idx is None:
                for h in range(g * G, (g + 1) * G):
                    qh = q[b, :, h, :].to(dtype)
                    for i0 in range(0, Sq, rows):
                        i1 = min(Sq, i0 + rows)
                        oo, ll = _dense_rows(qh[i0:i1], kk, vv, i0, i1, off, causal, window, c)
                        o[b, i0:i1, h] = oo
                        lse[b, h, i0:i1] = ll
            else:
                step = max(1, rows // 64)
                for i0 in range(0, Sq, step):
                    i1 = min(Sq, i0 + step)
                    ix = idx[b, i0:i1, g, :].to(torch.int64)                    # [n, topk]
                    ok = (ix >= 0) & (ix < Skv)
                    if causal:
                        ok &= ix <= torch.arange(i0, i1).unsqueeze(1) + off
                    ixc = torch.where(ok, ix, torch.zeros_like(ix))
                    ksel = kk[ixc]                                                # [n, topk, Dqk]
                    vsel = vv[ixc]                                                # [n, topk, Dv]
                    qq = q[b, i0:i1, g * G:(g + 1) * G, :].to(dtype)              # [n, G, Dqk]
                    s = torch.bmm(qq, ksel.transpose(1, 2).contiguous()) * c      # [n, G, topk]
                    allowed = ok.unsqueeze(1).expand_as(s)
                    oo, ll = _softmax_rows(s, allowed, vsel)                      # [n, G, Dv], [n, G]
                    o[b, i0:i1, g * G:(g + 1) * G] = oo
                    lse[b, g * G:(g + 1) * G, i0:i1] = ll.T
    return o, lse


def fwd_rows(q, k, v, scale, rows, causal=True, window=0):
    """The dense forward of single query rows: rows [n, 3] of (b, i, h) triples; returns
    o [n, Dv] and lse [n] in f64, each row's softmax taken over its whole allowed key set."""
    Sq, Hq, Skv, Hkv = q.shape[1], q.shape[2], k.shape[1], k.shape[2]
    G = Hq // Hkv
    c = scale * LOG2E
    o = torch.empty((len(rows), v.shape[3]), dtype=torch.float64)
    lse = torch.empty((len(rows),), dtype=torch.float64)
    for n, (b, i, h) in enumerate(rows):
        b, i, h = int(b), int(i), int(h)
        qq = q[b, i:i + 1, h, :].to(torch.float64)
        kk = k[b, :, h // G, :].to(torch.float64)
        vv = v[b, :, h // G, :].to(torch.float64)
        oo, ll = _dense_rows(qq, kk, vv, i, i + 1, Skv - Sq, causal, window, c)
        o[n], lse[n] = oo[0], ll[0]
    return o, lse


def make_o_lse(w, inputs, dtype=torch.float64):
    """O rounded to the workload's storage dtype and lse rounded to float32, from a forward pass
    over the drawn inputs.  Both sides of every comparison consume these same bytes."""
    # storage dtype of a workload name (the oracle keeps its own table; it imports nothing of
    # the HIP package)
    DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}
    o, lse = fwd(inputs["q"], inputs["k"], inputs["v"], w.scale, w.causal, w.window, inputs["idx"], dtype=dtype)
    return o.to(DTYPES[w.dtype]), lse.to(torch.float32)
