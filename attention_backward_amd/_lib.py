"""ctypes binding of libattn_bwd.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (include/attn_bwd.h) and does
nothing but check that torch tensors are on the GPU, contiguous and of the right dtype, and
pass their device pointers, the sizes and torch's current HIP stream.  All arithmetic runs in
the library's kernels.  There is no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_bwd.so")

ATTN_DT_F16, ATTN_DT_BF16 = 0, 1
ATTN_OK, ATTN_E_INVAL, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = 0, -1, -2, -3, -4
ATTN_BF16_AUTO, ATTN_BF16_SPLIT, ATTN_BF16_FP16 = 0, 1, 2
_DT = {torch.float16: ATTN_DT_F16, torch.bfloat16: ATTN_DT_BF16}

EXPORTS = ("attn_bwd", "attn_bwd_ex", "attn_bwd_noalloc", "attn_bwd_workspace_size", "attn_bwd_delta", "attn_fwd",
           "attn_fwd_varlen", "attn_bwd_strerror")
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES of include/attn_bwd.h


class attn_bwd_args(ctypes.Structure):  # noqa: N801  (mirrors the C struct name)
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("topk_idx", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64), ("Hq", ctypes.c_int64),
        ("Hkv", ctypes.c_int64), ("Dqk", ctypes.c_int64), ("Dv", ctypes.c_int64), ("topk", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("events", ctypes.c_void_p),
        ("kv_shared", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("nseq", ctypes.c_int64), ("max_seqlen", ctypes.c_int64),
        ("bf16_arith", ctypes.c_int32),
    ]


class AttnBwdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"attn_bwd status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m attention_backward_amd.build`")
        lib = ctypes.CDLL(path)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.attn_bwd_workspace_size.argtypes = [ctypes.POINTER(attn_bwd_args)]
        lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.attn_bwd_ex.argtypes = [ctypes.POINTER(attn_bwd_args)]
        lib.attn_bwd_ex.restype = ctypes.c_int
        lib.attn_bwd_noalloc.argtypes = [ctypes.POINTER(attn_bwd_args)]
        lib.attn_bwd_noalloc.restype = ctypes.c_int
        lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_float, I32, I32, P, I64,
                                 I32, P, ctypes.c_size_t, P]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_bwd_delta.argtypes = [P, P, P, I64, I64, I64, I64, I32, P]
        lib.attn_bwd_delta.restype = ctypes.c_int
        lib.attn_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, I32, I32, P]
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_fwd_varlen.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, I32,
                                         I32, P]
        lib.attn_fwd_varlen.restype = ctypes.c_int
        lib.attn_bwd_strerror.argtypes = [ctypes.c_int]
        lib.attn_bwd_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def attn_bwd_strerror(status: int) -> str:
    return load().attn_bwd_strerror(int(status)).decode()


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnBwdError(status, attn_bwd_strerror(status))


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_args(q, k, v, o, dout, lse, dq, dk, dv, *, scale, causal=True, window=0, topk_idx=None,
              workspace=None, stream=None, kv_shared=False, cu_seqlens=None, max_seqlen=None,
              bf16_arith=ATTN_BF16_AUTO) -> attn_bwd_args:
    """Fill an attn_bwd_args from torch tensors (shapes taken from q [B,Sq,Hq,Dqk], k and dout).

    kv_shared: the shared-latent form of the top-k path; v and dv are None, V is the first Dv
    columns of k and dk receives dK + [dV, 0].
    cu_seqlens: packed sequences (int32 [nseq + 1] on the GPU; tensors [1, T, H, D]); max_seqlen,
    a host int bounding every length, is then required.

    The struct holds raw device pointers, not the tensors: every tensor passed here must stay
    referenced until the work enqueued with it has run (a temporary such as `o.cuda()` passed
    inline is freed on return, and torch may hand its memory to the next allocation)."""
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if kv_shared and (v is not None or dv is not None):
        raise ValueError("kv_shared: pass v=None and dv=None (V is read from k, dV is added into dk)")
    dt = q.dtype
    B, Sq, Hq, Dqk = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    Dv = dout.shape[3]
    a = attn_bwd_args()
    a.q, a.k, a.v = _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt)
    a.o, a.dout = _dev(o, "o", dt), _dev(dout, "dout", dt)
    a.lse = _dev(lse, "lse", torch.float32)
    a.topk_idx = _dev(topk_idx, "topk_idx", torch.int32)
    a.dq, a.dk, a.dv = _dev(dq, "dq", dt), _dev(dk, "dk", dt), _dev(dv, "dv", dt)
    a.kv_shared = int(bool(kv_shared))
    if cu_seqlens is not None:
        if max_seqlen is None:
            raise ValueError("cu_seqlens needs max_seqlen (a host int bounding every sequence length)")
        a.cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32)
        a.nseq, a.max_seqlen = cu_seqlens.numel() - 1, int(max_seqlen)
    a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.Dqk, a.Dv = B, Sq, Skv, Hq, Hkv, Dqk, Dv
    a.topk = 0 if topk_idx is None else topk_idx.shape[-1]
    a.scale = float(scale)
    a.causal = int(bool(causal))
    a.window = int(window)
    a.dtype = _DT[dt]
    a.bf16_arith = int(bf16_arith)
    if workspace is not None:
        a.workspace = _dev(workspace, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.stream = _stream(stream)
    return a


def attn_bwd_workspace_size(args: attn_bwd_args) -> int:
    return int(load().attn_bwd_workspace_size(ctypes.byref(args)))


def attn_bwd_ex(args: attn_bwd_args) -> None:
    _check(load().attn_bwd_ex(ctypes.byref(args)))


def attn_bwd_noalloc(args: attn_bwd_args) -> None:
    """attn_bwd_ex on the library's static per-device scratch (args.workspace is ignored)."""
    _check(load().attn_bwd_noalloc(ctypes.byref(args)))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, S, Hq, Hkv, D, scale, causal, window, topk_idx=None, topk=0,
             dtype=None, workspace=None, workspace_bytes=0, stream=None) -> None:
    """The plain-argument entry point (Sq = Skv = S, Dqk = Dv = D), tensors or raw pointers."""
    ptr = lambda t: t.data_ptr() if isinstance(t, torch.Tensor) else t  # noqa: E731
    if dtype is None:
        dtype = _DT[q.dtype]
    if isinstance(workspace, torch.Tensor):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load().attn_bwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(dout), ptr(lse), ptr(dq), ptr(dk), ptr(dv), B, S, Hq,
                           Hkv, D, float(scale), int(causal), int(window), ptr(topk_idx), int(topk), int(dtype),
                           ptr(workspace), int(workspace_bytes), _stream(stream)))


def attn_bwd_delta(o, dout, delta, stream=None) -> None:
    """delta [B,Hq,Sq] f32 = rowsum(o * dout) for o, dout [B,Sq,Hq,Dv] (the preprocess alone)."""
    B, Sq, Hq, Dv = o.shape
    dt = o.dtype
    _check(load().attn_bwd_delta(_dev(o, "o", dt), _dev(dout, "dout", dt), _dev(delta, "delta", torch.float32), B, Sq,
                                 Hq, Dv, _DT[dt], _stream(stream)))


def attn_fwd(q, k, v, o, lse, scale, causal=True, window=0, stream=None) -> None:
    """o [B,Sq,Hq,D] and lse [B,Hq,Sq] f32 (base 2) from q [B,Sq,Hq,D], k and v [B,Skv,Hkv,D]."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    dt = q.dtype
    _check(load().attn_fwd(_dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt), _dev(o, "o", dt),
                           _dev(lse, "lse", torch.float32), B, Sq, Skv, Hq, Hkv, D, float(scale), int(causal),
                           int(window), _DT[dt], _stream(stream)))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal=True, window=0, stream=None) -> None:
    """The forward over packed sequences: q, o [1,T,Hq,D], k, v [1,T,Hkv,D], lse [1,Hq,T] f32,
    cu_seqlens int32 [nseq + 1] on the GPU, max_seqlen a host int bounding every length."""
    _, T, Hq, D = q.shape
    Hkv = k.shape[2]
    dt = q.dtype
    _check(load().attn_fwd_varlen(_dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt), _dev(o, "o", dt),
                                  _dev(lse, "lse", torch.float32), _dev(cu_seqlens, "cu_seqlens", torch.int32),
                                  cu_seqlens.numel() - 1, int(max_seqlen), T, Hq, Hkv, D, float(scale), int(causal),
                                  int(window), _DT[dt], _stream(stream)))
