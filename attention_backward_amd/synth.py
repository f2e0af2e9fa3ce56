"""Seeded synthetic inputs for the attention backward.

This module draws random numbers and rounds them to the storage dtype; it holds none of the
attention arithmetic.  Both the test suite (for the oracle and the HIP path alike) and the
benchmark draw their inputs here, so the two sides see identical bytes.

Recipe (one numpy PCG64 generator per workload):
  * q, k, v, dout ~ N(0, 1), drawn in that order as float32 in BSHD shape, then rounded to
    the storage dtype with round-to-nearest-even (torch's fp16/bf16 conversion);
  * for the top-k variant, after the tensors: for every (b, query i, kv head) a set of topk
    distinct key indices drawn uniformly without replacement from the keys that query may
    see under bottom-right causal alignment, [0, i + Skv - Sq], kept in draw order, int32;
  * scale = 1 / sqrt(Dqk).
  * packed variable-length workloads: first the sequence lengths (nseq - 1 distinct cut points
    drawn uniformly from 1..T-1, sorted, so every length is at least 1 and they sum to T), then
    q, k, v, dout as above in the batch-of-one shape [1, T, H, D].
O and lse are not drawn: they are outputs of a forward pass over these inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    Skv: int
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    dtype: str
    causal: bool
    window: int
    topk: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dqk)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(name, B, Sq, Skv, Hq, Hkv, Dqk, Dv, dtype, causal=True, window=0, topk=0, seed=0):
    return Workload(name, B, Sq, Skv, Hq, Hkv, Dqk, Dv, dtype, causal, window, topk, seed)


# The pages' workloads, named by what they are.
WORKLOADS = {
    w.name: w
    for w in [
        # the correctness shape the TileOPs page checks every placement at
        _w("mha_causal_b1_s256_h2_d128_fp16", 1, 256, 256, 2, 2, 128, 128, "fp16", seed=1),
        # the llama-8b-long row of the TileOPs performance table
        _w("mha_causal_b2_s2048_h32_d128_fp16", 2, 2048, 2048, 32, 32, 128, 128, "fp16", seed=2),
        # the representative G=8 long-sequence workload of the flash-linear-attention issue
        _w("gqa_causal_b1_t16384_hq32_hkv4_d128_bf16", 1, 16384, 16384, 32, 4, 128, 128, "bf16", seed=3),
        # sliding-window GQA at head dim 64, tile-aligned and ragged lengths
        _w("swa_gqa_b2_t8192_hq16_hkv8_d64_w1024_fp16", 2, 8192, 8192, 16, 8, 64, 64, "fp16", window=1024, seed=4),
        _w("swa_gqa_b2_t8000_hq16_hkv8_d64_w1024_fp16", 2, 8000, 8000, 16, 8, 64, 64, "fp16", window=1024, seed=5),
        # the sparse MLA backward shape of the TileLang page, top-k gathered keys
        _w("sparse_mla_b1_sq4096_skv8192_h64_dqk576_dv512_top2048_bf16", 1, 4096, 8192, 64, 1, 576, 512, "bf16",
           topk=2048, seed=6),
    ]
}

HEADLINE = "mha_causal_b2_s2048_h32_d128_fp16"


def round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float32 array to the storage dtype (round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype])


def draw_topk(rng: np.random.Generator, B: int, Sq: int, Skv: int, Hkv: int, topk: int,
              causal: bool = True) -> np.ndarray:
    """Distinct key indices per (b, i, g), uniform over the keys query i may see ([0, i + Skv - Sq]
    when causal, else [0, Skv)), in draw order."""
    off = Skv - Sq
    idx = np.empty((B, Sq, Hkv, topk), np.int32)
    for b in range(B):
        for i in range(Sq):
            n = max(0, min(Skv, i + off + 1)) if causal else Skv
            for g in range(Hkv):
                if n >= topk:
                    idx[b, i, g] = rng.choice(n, size=topk, replace=False)
                else:  # fewer visible keys than topk: all of them, then -1 padding
                    idx[b, i, g, :n] = rng.permutation(n)
                    idx[b, i, g, n:] = -1
    return idx


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw q, k, v, dout (torch CPU tensors in the storage dtype) and the top-k indices."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = rng.standard_normal((w.B, w.Sq, w.Hq, w.Dqk), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Skv, w.Hkv, w.Dqk), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Skv, w.Hkv, w.Dv), dtype=np.float32)
    do = rng.standard_normal((w.B, w.Sq, w.Hq, w.Dv), dtype=np.float32)
    out = {
        "q": round_to(q, w.dtype),
        "k": round_to(k, w.dtype),
        "v": round_to(v, w.dtype),
        "dout": round_to(do, w.dtype),
        "idx": None,
    }
    if w.topk:
        out["idx"] = torch.from_numpy(draw_topk(rng, w.B, w.Sq, w.Skv, w.Hkv, w.topk, w.causal))
    return out


@dataclass(frozen=True)
class VarlenWorkload:
    """Packed variable-length sequences: T tokens in nseq sequences, dense masks inside each."""
    name: str
    T: int
    nseq: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool
    window: int
    seed: int
    lens: tuple = ()  # fixed lengths (summing to T) instead of drawn ones

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The packed unequal-length GQA endpoint of the flash-linear-attention issue (flattened total
# 16384, Hq 32 / Hkv 4, D 128, bf16), here ungated; the sliding-window variant at D 64.
VARLEN_WORKLOADS = {
    w.name: w
    for w in [
        VarlenWorkload("varlen_gqa_t16384_n8_hq32_hkv4_d128_bf16", 16384, 8, 32, 4, 128, "bf16", True, 0, 7),
        VarlenWorkload("varlen_swa_gqa_t8192_n5_hq32_hkv4_d64_w512_bf16", 8192, 5, 32, 4, 64, "bf16", True, 512, 8),
    ]
}


def draw_seqlens(rng: np.random.Generator, T: int, nseq: int) -> np.ndarray:
    """nseq lengths >= 1 summing to T: the gaps between nseq - 1 distinct sorted cut points."""
    cuts = np.sort(rng.choice(np.arange(1, T), size=nseq - 1, replace=False)) if nseq > 1 else np.array([], np.int64)
    return np.diff(np.concatenate([[0], cuts, [T]])).astype(np.int64)


def make_varlen_inputs(w: VarlenWorkload) -> dict:
    """Lengths (drawn unless fixed), cu_seqlens (int32 [nseq + 1]) and q, k, v, dout [1, T, H, D]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = np.asarray(w.lens, np.int64) if w.lens else draw_seqlens(rng, w.T, w.nseq)
    assert lens.sum() == w.T and lens.size == w.nseq
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((1, w.T, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((1, w.T, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((1, w.T, w.Hkv, w.D), dtype=np.float32)
    do = rng.standard_normal((1, w.T, w.Hq, w.D), dtype=np.float32)
    return {"q": round_to(q, w.dtype), "k": round_to(k, w.dtype), "v": round_to(v, w.dtype),
            "dout": round_to(do, w.dtype), "cu": torch.from_numpy(cu), "max_seqlen": int(lens.max())}
