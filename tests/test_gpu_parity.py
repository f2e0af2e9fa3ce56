"""Parity of the HIP path (through the C ABI) with the f64 CPU oracle on the same seeded inputs.

Small shapes are compared element by element over every output; they span several tiles of
both kernels and have ragged tails.  The pages' full-size workloads run in exactly the launch
configuration the benchmark times and are compared on sampled rows that the oracle computes
one by one (its dq of a query row, its dk/dv of a key row).  Tolerance (fp16/bf16 outputs):
|gpu - ref| <= 5e-3 + 1e-2 |ref| elementwise, the allclose the TileOPs page checks with.
Outputs and workspace are NaN-poisoned before every call.
"""
import numpy as np
import pytest
import torch

import attention_backward_amd as ab
import oracle
from attention_backward_amd import synth
from tests.helpers import check_close, log, poisoned_like, prepare, sample_rows, to_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def run(inp, w, bf16_arith=ab._lib.ATTN_BF16_AUTO):
    g = to_gpu(inp)
    dq, dk, dv = poisoned_like(g["q"]), poisoned_like(g["k"]), poisoned_like(g["v"])
    args = ab.make_args(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq, dk, dv, scale=w.scale,
                        causal=w.causal, window=w.window, topk_idx=g["idx"], bf16_arith=bf16_arith)
    need = ab.attn_bwd_workspace_size(args)
    assert need > 0
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    args.workspace, args.workspace_bytes = ws.data_ptr(), need
    ab.attn_bwd_ex(args)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def full_compare(w, inp=None, bf16_arith=ab._lib.ATTN_BF16_AUTO):
    log(f"case {w.name}: B={w.B} Sq={w.Sq} Skv={w.Skv} Hq={w.Hq} Hkv={w.Hkv} D={w.Dqk}/{w.Dv} {w.dtype} "
        f"causal={w.causal} window={w.window} topk={w.topk} bf16_arith={bf16_arith}")
    inp = inp or prepare(w)
    dq, dk, dv = run(inp, w, bf16_arith)
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale, w.causal, w.window,
                     inp["idx"])
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.double().numpy(), r)
    return inp, (dq, dk, dv)


def small(name, **kw):
    base = dict(B=1, Sq=256, Skv=256, Hq=2, Hkv=2, Dqk=128, Dv=128, dtype="fp16", causal=True, window=0, topk=0,
                seed=100)
    base.update(kw)
    return synth.Workload(name=name, **base)


SMALL = [
    W["mha_causal_b1_s256_h2_d128_fp16"],
    small("gqa_g4_bf16_ragged", B=2, Sq=300, Skv=300, Hq=8, Hkv=2, dtype="bf16", seed=101),
    small("swa_d64_ragged", B=2, Sq=600, Skv=600, Hq=4, Hkv=2, Dqk=64, Dv=64, window=100, seed=102),
    small("full_noncausal_d64_bf16", Sq=200, Skv=200, Hq=2, Hkv=1, Dqk=64, Dv=64, dtype="bf16", causal=False,
          seed=103),
    small("causal_sq_lt_skv", Sq=200, Skv=328, Hq=4, Hkv=4, seed=104),
    small("causal_sq_gt_skv_empty_rows", Sq=300, Skv=130, Hq=2, Hkv=1, seed=105),
    small("swa_g8_d128_window37", B=1, Sq=333, Skv=333, Hq=8, Hkv=1, window=37, seed=106),
    small("swa_window1024_t2500", B=1, Sq=2500, Skv=2500, Hq=4, Hkv=2, Dqk=64, Dv=64, window=1024, seed=107),
    small("mha_causal_s1024_h4_bf16", Sq=1024, Skv=1024, Hq=4, Hkv=4, dtype="bf16", seed=108),
    small("gqa_g8_nowindow_ragged_fp16", Sq=333, Skv=333, Hq=8, Hkv=1, seed=109),
    small("gqa_g8_nowindow_ragged_bf16", B=2, Sq=397, Skv=397, Hq=16, Hkv=2, dtype="bf16", seed=110),
    # More key-block items than CUs: the D = 128 launch runs several items per workgroup, with the
    # next item's first tile loaded during the current item's last step.
    small("mha_items_gt_cus_ragged_fp16", B=2, Sq=700, Skv=700, Hq=24, Hkv=24, seed=111),
    small("gqa_items_gt_cus_ragged_bf16", B=3, Sq=700, Skv=700, Hq=32, Hkv=16, dtype="bf16", seed=112),
    small("swa_items_gt_cus_fp16", B=3, Sq=800, Skv=800, Hq=16, Hkv=16, window=200, seed=113),
] + [small(f"tiny_s{s}", Sq=s, Skv=s, seed=110 + s) for s in (1, 2, 63, 65, 127, 129, 200)]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_full_parity(w):
    full_compare(w)


BF16_SMALL = [w for w in SMALL if w.dtype == "bf16"]


@pytest.mark.parametrize("mode", ["split", "fp16"])
@pytest.mark.parametrize("w", BF16_SMALL, ids=[w.name for w in BF16_SMALL])
def test_small_bf16_both_arithmetics(w, mode):
    """bf16 calls either keep bf16 products with hi + lo P and dS operands, or run the fp16 kernels
    on fp16 copies of the inputs scaled by powers of two (bf16 outputs); both meet the tolerance."""
    full_compare(w, bf16_arith=ab._lib.ATTN_BF16_SPLIT if mode == "split" else ab._lib.ATTN_BF16_FP16)


def test_bf16_reexpression_scales_out_of_fp16_range():
    """Inputs far outside fp16's range (|q| ~ 2^40, |k| ~ 2^-40, |dO| ~ 2^20, V and O ~ 2^-30) in
    bf16: the power-of-two scales bring each tensor into range and the factors undo them."""
    w = small("bf16_far_scales", Sq=200, Skv=200, Hq=4, Hkv=2, dtype="bf16", seed=130)
    inp = synth.make_inputs(w)
    s_q, s_k, s_v, s_do = 2.0 ** 40, 2.0 ** -40, 2.0 ** -30, 2.0 ** 20
    inp["q"] = (inp["q"].double() * s_q).to(torch.bfloat16)
    inp["k"] = (inp["k"].double() * s_k).to(torch.bfloat16)
    inp["v"] = (inp["v"].double() * s_v).to(torch.bfloat16)
    inp["dout"] = (inp["dout"].double() * s_do).to(torch.bfloat16)
    from oracle import forward as oracle_forward
    inp["o"], inp["lse"] = oracle_forward.make_o_lse(w, inp)
    dq, dk, dv = run(inp, w, ab._lib.ATTN_BF16_FP16)
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale, w.causal, w.window)
    # compare in the units of each output's own magnitude
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        m = float(np.abs(r).max())
        assert m > 0 and np.isfinite(m)
        check_close(name + " (relative to its largest magnitude)", got.double().numpy() / m, r / m)


DET = [SMALL[1], SMALL[-2], SMALL[-1]]  # G = 4; G = 8 without a window, fp16 and bf16


@pytest.mark.parametrize("w", DET, ids=[w.name for w in DET])
def test_deterministic_and_both_entry_points(w):
    """Two identical calls give the same bits (dense dK/dV are stored once, dQ is owned), and so
    does the plain-argument entry point with a caller-allocated workspace."""
    log(f"case {w.name} (bit identity)")
    inp = prepare(w)
    a = run(inp, w)
    b = run(inp, w)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "outputs differ between two identical calls"
    # the plain-argument entry point gives the same bits
    g = to_gpu(inp)
    dq, dk, dv = poisoned_like(g["q"]), poisoned_like(g["k"]), poisoned_like(g["v"])
    args = ab.make_args(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq, dk, dv, scale=w.scale,
                        causal=w.causal, window=w.window)
    need = ab.attn_bwd_workspace_size(args)
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    ab.attn_bwd(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq, dk, dv, w.B, w.Sq, w.Hq, w.Hkv, w.Dqk,
                w.scale, w.causal, w.window, workspace=ws, workspace_bytes=need)
    torch.cuda.synchronize()
    for x, y in zip(a, (dq.cpu(), dk.cpu(), dv.cpu())):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # without a workspace the call is refused before anything is enqueued
    with pytest.raises(ab.AttnBwdError) as e:
        ab.attn_bwd(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq, dk, dv, w.B, w.Sq, w.Hq, w.Hkv, w.Dqk,
                    w.scale, w.causal, w.window)
    assert e.value.status == ab._lib.ATTN_E_WORKSPACE


@pytest.mark.parametrize("dtype,Dv", [("fp16", 128), ("bf16", 64), ("bf16", 512), ("fp16", 256)])
def test_delta_preprocess(dtype, Dv):
    r = np.random.default_rng(Dv)
    B, Sq, Hq = 2, 333, 3
    o = synth.round_to(r.standard_normal((B, Sq, Hq, Dv), dtype=np.float32), dtype)
    do = synth.round_to(r.standard_normal((B, Sq, Hq, Dv), dtype=np.float32), dtype)
    delta = poisoned_like(torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda"))
    ab.attn_bwd_delta(o.cuda(), do.cuda(), delta)
    torch.cuda.synchronize()
    ref = oracle.delta(o, do)
    bound = 1e-6 + 1e-5 * np.einsum("bihd->bhi", np.abs(o.double().numpy() * do.double().numpy()))
    err = np.abs(delta.cpu().double().numpy() - ref)
    log(f"  delta {dtype} Dv={Dv}: max err {err.max():.3e}")
    assert np.all(err <= bound)


def test_masked_keys_do_not_matter():
    """Changing K/V rows that no query can see changes no output bit (Sq < Skv, window)."""
    w = small("masked_keys", Sq=128, Skv=1024, Hq=2, Hkv=1, window=200, seed=120)
    inp = prepare(w)
    a = run(inp, w)
    inp2 = dict(inp)
    k2, v2 = inp["k"].clone(), inp["v"].clone()
    # query i sees keys (i + 896 - 200, i + 896]: keys < 697 are never visible
    k2[:, :697] = 3.0
    v2[:, :697] = -3.0
    inp2["k"], inp2["v"] = k2, v2
    b = run(inp2, w)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.all(a[1][:, :697] == 0) and torch.all(a[2][:, :697] == 0)


# Sampled rows (edges, tile boundaries, random rows) of the workloads not compared in full below.
FULL = ["gqa_causal_b1_t16384_hq32_hkv4_d128_bf16"]


# Every element of the output against the full oracle backward, in the benchmark's launch
# configuration.
EVERY = ["mha_causal_b2_s2048_h32_d128_fp16", "swa_gqa_b2_t8192_hq16_hkv8_d64_w1024_fp16",
         "swa_gqa_b2_t8000_hq16_hkv8_d64_w1024_fp16"]


@pytest.mark.parametrize("name", EVERY)
def test_full_size_every_element(name):
    log(f"case {name} (full size, every element)")
    full_compare(W[name])


def group_slice(inp, w, g):
    """The sub-problem of KV head g: its G query heads and its K/V rows.  Heads of different groups
    never interact, so the oracle's full backward over this slice gives every dq row of those
    heads and every dk/dv row of KV head g."""
    G = w.Hq // w.Hkv
    hs = slice(g * G, (g + 1) * G)
    q, o, do = (inp[n][:, :, hs].contiguous() for n in ("q", "o", "dout"))
    k, v = (inp[n][:, :, g : g + 1].contiguous() for n in ("k", "v"))
    lse = inp["lse"][:, hs].contiguous()
    idx = None if inp["idx"] is None else inp["idx"][:, :, g : g + 1].contiguous()
    return oracle.bwd(q, k, v, o, do, lse, w.scale, w.causal, w.window, idx), hs


def test_full_size_gqa_one_group_every_row():
    """The 16K-token GQA workload: every dq row of one KV group's 8 query heads and every dk/dv
    row of that KV head (the last group, batch 0)."""
    name = "gqa_causal_b1_t16384_hq32_hkv4_d128_bf16"
    w = W[name]
    log(f"case {name} (full size, every row of KV group {w.Hkv - 1})")
    inp = prepare(w)
    dq, dk, dv = run(inp, w)
    g = w.Hkv - 1
    (rq, rk, rv), hs = group_slice(inp, w, g)
    check_close("dq group", dq[:, :, hs].double().numpy(), rq)
    check_close("dk group", dk[:, :, g : g + 1].double().numpy(), rk)
    check_close("dv group", dv[:, :, g : g + 1].double().numpy(), rv)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    w = W[name]
    log(f"case {name} (full size, sampled rows)")
    inp = prepare(w)
    dq, dk, dv = run(inp, w)
    rng = np.random.default_rng(7)
    qrows = sample_rows(rng, 48, w.B, w.Sq, w.Hq)
    krows = sample_rows(rng, 48, w.B, w.Skv, w.Hkv)
    args = (inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale)
    ref_dq = oracle.bwd_dq_rows(*args, qrows, w.causal, w.window)
    ref_dk, ref_dv = oracle.bwd_dkv_rows(*args, krows, w.causal, w.window)
    got_dq = dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]].double().numpy()
    got_dk = dk[krows[:, 0], krows[:, 1], krows[:, 2]].double().numpy()
    got_dv = dv[krows[:, 0], krows[:, 1], krows[:, 2]].double().numpy()
    check_close("dq rows", got_dq, ref_dq)
    check_close("dk rows", got_dk, ref_dk)
    check_close("dv rows", got_dv, ref_dv)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
