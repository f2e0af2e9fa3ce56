"""Shared helpers for the GPU parity tests: inputs, O/lse from the oracle's forward, tolerance."""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
from oracle import forward as oracle_forward
from attention_backward_amd import synth

ATOL, RTOL = 5e-3, 1e-2  # fp16/bf16 outputs vs the f64 oracle: |gpu - ref| <= ATOL + RTOL*|ref|


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def prepare(w: synth.Workload):
    """Inputs (CPU, storage dtype) plus O (storage dtype) and lse (f32) from the f64 forward."""
    t0 = time.time()
    log(f"preparing {w.name}: drawing inputs and running the oracle's forward")
    inp = synth.make_inputs(w)
    small = w.B * w.Sq * w.Skv * w.Hq <= 4 * 2 ** 20 and w.topk == 0
    if small:  # the plain C forward
        o, lse = oracle.fwd(inp["q"], inp["k"], inp["v"], w.scale, w.causal, w.window,
                            None if inp["idx"] is None else inp["idx"].numpy())
        inp["o"] = torch.from_numpy(o).to(synth.DTYPES[w.dtype])
        inp["lse"] = torch.from_numpy(lse).to(torch.float32)
    else:
        inp["o"], inp["lse"] = oracle_forward.make_o_lse(w, inp)
    log(f"prepared {w.name} in {time.time() - t0:.1f}s")
    return inp


def to_gpu(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def poisoned_like(t):
    x = torch.empty_like(t)
    x.view(torch.uint8 if x.element_size() == 1 else torch.int16 if x.element_size() == 2 else torch.int32).fill_(-1)
    return x  # all bits set: NaN in fp16, bf16 and f32


def check_close(name, got, ref, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU output"
    err = np.abs(got - ref)
    viol = err - (atol + rtol * np.abs(ref))
    worst = np.unravel_index(np.argmax(viol), viol.shape) if viol.size else ()
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else float(np.linalg.norm(got))
    log(f"  {name}: max|err| {err.max() if err.size else 0:.3e}  max violation {viol.max() if viol.size else 0:.3e}  "
        f"rel L2 {rel:.3e}")
    assert viol.size == 0 or viol.max() <= 0, f"{name}: tolerance violated at {worst}: got {got[worst]} ref {ref[worst]}"
    return rel


def sample_rows(rng, n, B, S, H, extra_i=()):
    """(b, i, h) triples: edges, tile boundaries and random rows."""
    rows = set()
    for i in list(extra_i) + [0, 1, S - 1, S - 2, min(S - 1, 63), min(S - 1, 64), min(S - 1, 127), min(S - 1, 128),
                              min(S - 1, 255), min(S - 1, 256)]:
        rows.add((int(rng.integers(B)), int(i), int(rng.integers(H))))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(S)), int(rng.integers(H))))
    return np.array(sorted(rows), dtype=np.int64)


def flops_metric(w: synth.Workload) -> float:
    """2.5 x forward flops over the exact unmasked (query, key) pairs, forward = (2 Dqk + 2 Dv) per pair."""
    return 2.5 * pairs(w) * (2 * w.Dqk + 2 * w.Dv)


def pairs(w: synth.Workload) -> int:
    off = w.Skv - w.Sq
    if w.topk:
        return w.B * w.Hq * w.Sq * w.topk  # the drawn lists are distinct and causal
    i = np.arange(w.Sq, dtype=np.int64)
    hi = np.minimum(w.Skv - 1, i + off) if w.causal else np.full_like(i, w.Skv - 1)
    lo = np.maximum(0, i + off - w.window + 1) if w.window > 0 else np.zeros_like(i)
    return int(np.maximum(0, hi - lo + 1).sum()) * w.B * w.Hq


_ = math
