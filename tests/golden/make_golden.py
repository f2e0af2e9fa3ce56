"""Write the stored expected values under tests/golden/ (run from the repository root:
``python -m tests.golden.make_golden``).

The pages print no worked numeric example, so every stored value here comes from the oracle:
seeded inputs from the shared input generator, O and lse from the oracle's forward, and dq, dk,
dv from the oracle's backward (the Reference program of the TileOPs PR #2281 page, "TileFoundry
Description", written out in f64).  The files are a drift guard for the oracle and a fixed
expected output for the HIP path at shapes smaller than one tile of any kernel.  Changing them
means changing the oracle's arithmetic, which a commit must justify from the pages.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from attention_backward_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))

CASES = [
    synth.Workload("mha_causal_b1_s9_h1_d64_fp16", 1, 9, 9, 1, 1, 64, 64, "fp16", True, 0, 0, 201),
    synth.Workload("swa_gqa_b1_s7_hq2_hkv1_d64_w3_bf16", 1, 7, 7, 2, 1, 64, 64, "bf16", True, 3, 0, 202),
]


def _vals(t) -> list:
    a = t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float64)
    return [float(x) for x in a.reshape(-1)]


def make(w: synth.Workload) -> dict:
    inp = synth.make_inputs(w)
    o, lse = oracle.fwd(inp["q"], inp["k"], inp["v"], w.scale, w.causal, w.window, None)
    o_st = torch.from_numpy(o).to(synth.DTYPES[w.dtype])  # O as the backward receives it
    lse32 = torch.from_numpy(lse).to(torch.float32)
    dq, dk, dv = oracle.bwd(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, w.scale, w.causal, w.window, None)
    fields = {f: getattr(w, f) for f in ("B", "Sq", "Skv", "Hq", "Hkv", "Dqk", "Dv", "dtype", "causal", "window",
                                         "topk", "seed")}
    rec = {
        "name": w.name,
        "source": "oracle/ (f64 Reference backward of the TileOPs PR #2281 page); inputs from the seeded generator",
        "workload": fields,
        "scale": w.scale,
        "shapes": {"q": list(inp["q"].shape), "k": list(inp["k"].shape), "v": list(inp["v"].shape),
                   "o": list(o_st.shape), "lse": list(lse32.shape)},
    }
    for name, t in (("q", inp["q"]), ("k", inp["k"]), ("v", inp["v"]), ("dout", inp["dout"]), ("o", o_st),
                    ("lse", lse32), ("dq", dq), ("dk", dk), ("dv", dv)):
        rec[name] = _vals(t)
    return rec


def path(name: str) -> str:
    return os.path.join(HERE, name + ".json")


def main():
    for w in CASES:
        rec = make(w)
        with open(path(w.name), "w") as f:
            json.dump(rec, f, separators=(",", ":"))
            f.write("\n")
        print("wrote", path(w.name))


if __name__ == "__main__":
    main()
