"""Properties of the HIP path that hold whatever the values (GPU, through the C ABI).

- A window at least as wide as the key range is plain causal attention (flash-linear-attention
  issue #8 defines the window as a restriction of the causal mask): same outputs.
- Grouped-query attention is multi-head attention on K and V repeated for every query head of a
  group, with dK and dV summed over the group (same issue, the KV-head-owned backward): dQ is
  the same, and the GQA dK/dV equal the group sums of the MHA dK/dV.
"""
import pytest
import torch

from attention_backward_amd import synth
from tests.helpers import ATOL, RTOL, check_close, log, prepare
from tests.test_gpu_parity import run

pytestmark = pytest.mark.gpu


def wl(name, **kw):
    base = dict(B=1, Sq=300, Skv=300, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp16", causal=True, window=0, topk=0,
                seed=300)
    base.update(kw)
    return synth.Workload(name=name, **base)


@pytest.mark.parametrize("dtype,D", [("fp16", 128), ("bf16", 64)])
def test_wide_window_equals_causal(dtype, D):
    w = wl(f"causal_{dtype}_{D}", Dqk=D, Dv=D, dtype=dtype, seed=301)
    inp = prepare(w)
    a = run(inp, w)
    for window in (w.Skv, w.Skv + 77):
        b = run(inp, w.with_(window=window))
        for name, x, y in zip(("dq", "dk", "dv"), a, b):
            # the same products over the same keys: equal up to the order of a few additions
            check_close(f"{name} window={window}", y.double().numpy(), x.double().numpy(), atol=1e-3, rtol=1e-3)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_gqa_equals_mha_on_repeated_kv(dtype):
    G = 4
    w = wl(f"gqa_{dtype}", Sq=257, Skv=257, Hq=8, Hkv=2, dtype=dtype, seed=302)
    inp = prepare(w)
    dq_g, dk_g, dv_g = run(inp, w)
    # the same problem as MHA: K and V repeated per query head (query head h reads KV head h // G)
    wm = w.with_(Hkv=w.Hq)
    inp_m = dict(inp)
    inp_m["k"] = inp["k"].repeat_interleave(G, dim=2).contiguous()
    inp_m["v"] = inp["v"].repeat_interleave(G, dim=2).contiguous()
    dq_m, dk_m, dv_m = run(inp_m, wm)
    log(f"  GQA G={G} {dtype} vs MHA on repeated K/V")
    check_close("dq", dq_g.double().numpy(), dq_m.double().numpy(), atol=1e-3, rtol=1e-3)
    # the MHA per-head dK/dV are each rounded to the storage dtype before the group sum
    sum_k = dk_m.double().reshape(w.B, w.Skv, w.Hkv, G, w.Dqk).sum(3).numpy()
    sum_v = dv_m.double().reshape(w.B, w.Skv, w.Hkv, G, w.Dv).sum(3).numpy()
    check_close("dk = sum over the group", dk_g.double().numpy(), sum_k, atol=2 * ATOL, rtol=2 * RTOL)
    check_close("dv = sum over the group", dv_g.double().numpy(), sum_v, atol=2 * ATOL, rtol=2 * RTOL)
    assert torch.isfinite(dk_g.float()).all() and torch.isfinite(dv_g.float()).all()
