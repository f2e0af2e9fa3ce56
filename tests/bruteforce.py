"""Brute-force dense restatement of the attention backward, used only to pin the oracle.

It is written independently of oracle/attn_oracle.c: instead of walking allowed keys row by
row, it materialises the full [Sq, Skv] score matrix of every head with numpy and applies a
multiplicity matrix M (how many times key j appears in query i's key set: 0/1 for the dense
masks, a count for a top-k list) built with vectorised comparisons / np.add.at.
"""
import numpy as np

LOG2E = 1.4426950408889634


def multiplicity(Sq, Skv, causal, window, idx_row=None):
    """M [Sq, Skv] for one (b, kv head); idx_row [Sq, topk] or None."""
    off = Skv - Sq
    if idx_row is None:
        i = np.arange(Sq)[:, None]
        j = np.arange(Skv)[None, :]
        m = np.ones((Sq, Skv), bool)
        if causal:
            m &= j <= i + off
        if window > 0:
            m &= j > i + off - window
        return m.astype(np.float64)
    M = np.zeros((Sq, Skv), np.float64)
    ii = np.repeat(np.arange(Sq), idx_row.shape[1])
    jj = idx_row.reshape(-1).astype(np.int64)
    ok = (jj >= 0) & (jj < Skv)
    if causal:
        ok &= jj <= ii + off
    np.add.at(M, (ii[ok], jj[ok]), 1.0)
    return M


def multiplicity_packed(cu, causal, window):
    """M [T, T] for packed sequences (batch of one): key j counts for query i iff both lie in
    the same sequence [cu[s], cu[s+1]) and the masks hold for their positions inside it."""
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    t = np.arange(T)
    seq = np.searchsorted(cu, t, side="right") - 1
    pos = t - cu[seq]
    i, j = pos[:, None], pos[None, :]
    m = seq[:, None] == seq[None, :]
    if causal:
        m &= j <= i
    if window > 0:
        m &= j > i - window
    return m.astype(np.float64)


def forward(q, k, v, scale, causal, window, idx=None, M_all=None):
    B, Sq, Hq, _ = q.shape
    Skv, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Sq, Hq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            M = M_all if M_all is not None else multiplicity(Sq, Skv, causal, window,
                                                             None if idx is None else idx[b, :, g, :])
            s = q[b, :, h, :] @ k[b, :, g, :].T * scale * LOG2E
            has = M.sum(1) > 0
            smax = np.where(M > 0, s, -np.inf).max(1, initial=-np.inf)
            smax = np.where(has, smax, 0.0)
            w = M * np.exp2(np.where(M > 0, s - smax[:, None], -np.inf))
            tot = w.sum(1)
            o[b, :, h, :] = np.where(has[:, None], (w @ v[b, :, g, :]) / np.where(has, tot, 1.0)[:, None], 0.0)
            lse[b, h, :] = np.where(has, smax + np.log2(np.where(has, tot, 1.0)), -np.inf)
    return o, lse


def backward(q, k, v, o, dout, lse, scale, causal, window, idx=None, return_p=False, M_all=None):
    B, Sq, Hq, _ = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    ps = {}
    for b in range(B):
        for h in range(Hq):
            g = h // G
            M = M_all if M_all is not None else multiplicity(Sq, Skv, causal, window,
                                                             None if idx is None else idx[b, :, g, :])
            l = lse[b, h, :]
            live = np.isfinite(l) | (l > 0)
            s = q[b, :, h, :] @ k[b, :, g, :].T
            p = np.where(M > 0, M * np.exp2(s * scale * LOG2E - np.where(live, l, 0.0)[:, None]), 0.0)
            p[~live] = 0.0
            delta = (o[b, :, h, :] * dout[b, :, h, :]).sum(1)
            dp = dout[b, :, h, :] @ v[b, :, g, :].T
            ds = p * (dp - delta[:, None])
            dq[b, :, h, :] = scale * ds @ k[b, :, g, :]
            dk[b, :, g, :] += scale * ds.T @ q[b, :, h, :]
            dv[b, :, g, :] += p.T @ dout[b, :, h, :]
            ps[(b, h)] = (p, dp, ds, delta)
    if return_p:
        return dq, dk, dv, ps
    return dq, dk, dv
