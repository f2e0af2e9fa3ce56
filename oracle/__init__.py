"""f64 CPU oracle for the softmax-attention backward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its binding) never touches it,
and it shares no code with that path.

The arithmetic lives in ``attn_oracle.c`` (plain loops, double precision, OpenMP over rows);
this module only loads the shared object and marshals numpy arrays.  What the C code computes
is the Reference program of the TileOPs PR #2281 page ("TileFoundry Description"),
generalised to grouped-query attention and a sliding window (flash-linear-attention issue #8)
and to a gathered top-k key set with Dqk != Dv (TileLang PR #2592).

Parity status of each entry point (what pins it is in tests/test_oracle_pins.py):
  fwd           pinned: torch f64 autograd-free softmax, brute-force dense, row sums
  delta         pinned: delta == sum_j p_ij dp_ij for a consistent O
  bwd           pinned: central finite differences of sum(O * dO), torch f64 autograd,
                        brute-force dense numpy, dS row sums, dV = P^T dO, closed forms
  bwd_dq_rows   pinned: equals the matching rows of bwd (which is pinned)
  bwd_dkv_rows  pinned: equals the matching rows of bwd
  fwd_varlen,   pinned: brute force over the block-diagonal packed mask, equal lengths equal to
  bwd_varlen            the dense batch, a sequence's outputs blind to the other sequences
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Shape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64),
        ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("Dqk", ctypes.c_int64),
        ("Dv", ctypes.c_int64), ("topk", ctypes.c_int64), ("scale", ctypes.c_double),
        ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            import sys

            torch = sys.modules.get("torch")
            if torch is not None and torch.cuda.is_initialized():
                # No compiler child from a process that has set up the GPU: build beforehand.
                raise RuntimeError(f"{_LIB_PATH} is missing: build it first (python -c 'import oracle; "
                                   "oracle.build()') before any GPU work in this process")
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        sp = ctypes.POINTER(_Shape)
        lib.oracle_fwd.argtypes = [sp, p, p, p, p, p, p]
        lib.oracle_delta.argtypes = [sp, p, p, p]
        lib.oracle_bwd.argtypes = [sp, p, p, p, p, p, p, p, p, p, p]
        lib.oracle_bwd_dq_rows.argtypes = [sp, p, p, p, p, p, p, p, p, ctypes.c_int64, p]
        lib.oracle_bwd_dkv_rows.argtypes = [sp, p, p, p, p, p, p, p, p, ctypes.c_int64, p, p]
        for f in ("oracle_fwd", "oracle_delta", "oracle_bwd", "oracle_bwd_dq_rows", "oracle_bwd_dkv_rows"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    """Exact widening of stored fp16/bf16/f32 values (numpy or torch CPU) to contiguous float64."""
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape(q, k, v, idx, scale, causal, window):
    B, Sq, Hq, Dqk = q.shape
    _, Skv, Hkv, _ = k.shape
    Dv = v.shape[-1]
    topk = 0 if idx is None else idx.shape[-1]
    return _Shape(B, Sq, Skv, Hq, Hkv, Dqk, Dv, topk, float(scale), int(bool(causal)), int(window))


def _idx(idx):
    if idx is None:
        return None
    if hasattr(idx, "detach"):
        idx = idx.detach().to("cpu").numpy()
    return np.ascontiguousarray(idx, dtype=np.int32)


def fwd(q, k, v, scale, causal=True, window=0, idx=None):
    """Masked softmax attention forward in f64: returns (o [B,Sq,Hq,Dv] f64, lse [B,Hq,Sq] f64, base 2)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    idx = _idx(idx)
    s = _shape(q, k, v, idx, scale, causal, window)
    o = np.empty((s.B, s.Sq, s.Hq, s.Dv), np.float64)
    lse = np.empty((s.B, s.Hq, s.Sq), np.float64)
    rc = _load().oracle_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_fwd rejected the shape (rc={rc})")
    return o, lse


def delta(o, dout):
    """delta [B,Hq,Sq] = rowsum(O * dO) in f64."""
    o, dout = _f64(o), _f64(dout)
    B, Sq, Hq, Dv = o.shape
    s = _Shape(B, Sq, Sq, Hq, Hq, 1, Dv, 0, 1.0, 0, 0)
    out = np.empty((B, Hq, Sq), np.float64)
    rc = _load().oracle_delta(ctypes.byref(s), _ptr(o), _ptr(dout), _ptr(out))
    if rc:
        raise ValueError(f"oracle_delta rejected the shape (rc={rc})")
    return out


def bwd(q, k, v, o, dout, lse, scale, causal=True, window=0, idx=None):
    """Full backward in f64: returns (dq, dk, dv) in BSHD, dk/dv at the KV head count."""
    q, k, v, o, dout, lse = (_f64(x) for x in (q, k, v, o, dout, lse))
    idx = _idx(idx)
    s = _shape(q, k, v, idx, scale, causal, window)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(v.shape, np.float64)
    rc = _load().oracle_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                            _ptr(idx), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc:
        raise ValueError(f"oracle_bwd failed (rc={rc})")
    return dq, dk, dv


def bwd_dq_rows(q, k, v, o, dout, lse, scale, rows, causal=True, window=0, idx=None):
    """dq for the listed query rows; rows is an int array [n,3] of (b, i, h).  Returns [n, Dqk]."""
    q, k, v, o, dout, lse = (_f64(x) for x in (q, k, v, o, dout, lse))
    idx = _idx(idx)
    s = _shape(q, k, v, idx, scale, causal, window)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], s.Dqk), np.float64)
    rc = _load().oracle_bwd_dq_rows(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                    _ptr(idx), _ptr(rows), rows.shape[0], _ptr(out))
    if rc:
        raise ValueError(f"oracle_bwd_dq_rows failed (rc={rc})")
    return out


def bwd_dkv_rows(q, k, v, o, dout, lse, scale, rows, causal=True, window=0, idx=None):
    """dk, dv for the listed key rows; rows is an int array [n,3] of (b, j, g).  Returns ([n,Dqk], [n,Dv])."""
    q, k, v, o, dout, lse = (_f64(x) for x in (q, k, v, o, dout, lse))
    idx = _idx(idx)
    s = _shape(q, k, v, idx, scale, causal, window)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    dk = np.empty((rows.shape[0], s.Dqk), np.float64)
    dv = np.empty((rows.shape[0], s.Dv), np.float64)
    rc = _load().oracle_bwd_dkv_rows(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                     _ptr(idx), _ptr(rows), rows.shape[0], _ptr(dk), _ptr(dv))
    if rc:
        raise ValueError(f"oracle_bwd_dkv_rows failed (rc={rc})")
    return dk, dv


def _segments(cu):
    cu = np.asarray(cu.detach().cpu() if hasattr(cu, "detach") else cu, dtype=np.int64).reshape(-1)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(cu.size - 1)]


def fwd_varlen(q, k, v, cu, scale, causal=True, window=0):
    """Packed sequences (flash-linear-attention issue #8, packed varlen): q [1,T,Hq,Dqk],
    k [1,T,Hkv,Dqk], v [1,T,Hkv,Dv] and token offsets cu [nseq + 1]; tokens [cu[s], cu[s+1]) form
    sequence s, its own attention problem with the masks taken inside it.  Returns
    o [1,T,Hq,Dv] and lse [1,Hq,T] in f64 (tokens in no sequence: o = 0, lse = -inf)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, Dv = q.shape[1], q.shape[2], v.shape[3]
    o = np.zeros((1, T, Hq, Dv))
    lse = np.full((1, Hq, T), -np.inf)
    for a, b in _segments(cu):
        if b > a:
            o[:, a:b], lse[:, :, a:b] = fwd(q[:, a:b], k[:, a:b], v[:, a:b], scale, causal, window)
    return o, lse


def bwd_varlen(q, k, v, o, dout, lse, cu, scale, causal=True, window=0):
    """The backward of fwd_varlen's problem: each sequence's slice through bwd.  Returns dq, dk,
    dv in the packed layout (tokens in no sequence: 0)."""
    q, k, v, o, dout, lse = (_f64(x) for x in (q, k, v, o, dout, lse))
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for a, b in _segments(cu):
        if b > a:
            dq[:, a:b], dk[:, a:b], dv[:, a:b] = bwd(q[:, a:b], k[:, a:b], v[:, a:b], o[:, a:b], dout[:, a:b],
                                                     lse[:, :, a:b], scale, causal, window)
    return dq, dk, dv
