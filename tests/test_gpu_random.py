"""Randomised parity sweep: seeded small shapes drawn across every dense option, forward and
backward through the C ABI against the f64 oracle, plus random packed-length mixes and random
top-k problems (including corrupted lists: duplicates, padding, out-of-range and non-causal
entries).

Each case is drawn from its own seed (printed before it runs), so a failure names a shape that
reproduces.  Sizes stay small enough for the oracle to finish in about a second, but the draws
cover Sq < Skv and Sq > Skv, ragged tails, GQA ratios 1..8, windows from 1 up to beyond the
sequence, non-causal calls, both head dims and both element types.  Tolerances are those of the
other parity tests.
"""
import numpy as np
import pytest
import torch

import attention_backward_amd as ab
import oracle
from attention_backward_amd import synth
from tests.helpers import check_close, log, poisoned_like, to_gpu
from tests.test_gpu_forward import check_lse

pytestmark = pytest.mark.gpu

N_DENSE = 96
N_PACKED = 32
N_TOPK = 12


def draw_dense(seed):
    r = np.random.default_rng(1000 + seed)
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    causal = bool(r.random() < 0.8)
    Sq = int(r.integers(1, 700))
    Skv = Sq if r.random() < 0.5 else int(r.integers(1, 700))
    window = int(r.choice([0, 0, 1, int(r.integers(2, 300)), 900])) if causal else 0
    B = int(r.integers(1, 3))
    return synth.Workload(f"rand{seed}_b{B}_sq{Sq}_skv{Skv}_hq{Hkv * G}_hkv{Hkv}_d{D}_{'c' if causal else 'n'}"
                          f"_w{window}", B, Sq, Skv, Hkv * G, Hkv, D, D, str(r.choice(["fp16", "bf16"])), causal,
                          window, 0, 2000 + seed)


@pytest.mark.parametrize("seed", range(N_DENSE))
def test_random_dense_forward_and_backward(seed):
    w = draw_dense(seed)
    log(f"random dense case {w.name} {w.dtype}")
    inp = synth.make_inputs(w)
    o64, lse64 = oracle.fwd(inp["q"], inp["k"], inp["v"], w.scale, w.causal, w.window, None)
    g = to_gpu(inp)
    o, lse = poisoned_like(g["q"]), poisoned_like(torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda"))
    ab.attn_fwd(g["q"], g["k"], g["v"], o, lse, w.scale, causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    check_close("o", o.cpu().double().numpy(), o64)
    check_lse("lse", lse.cpu().numpy(), lse64)
    # the backward from the oracle's O and lse
    o_st = torch.from_numpy(o64).to(synth.DTYPES[w.dtype])
    lse32 = torch.from_numpy(lse64).to(torch.float32)
    dq, dk, dv = ab.backward(g["q"], g["k"], g["v"], o_st.cuda(), g["dout"], lse32.cuda(), causal=w.causal,
                             window=w.window)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, w.scale, w.causal, w.window, None)
    for name, got, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.cpu().double().numpy(), r_)


@pytest.mark.parametrize("seed", range(N_PACKED))
def test_random_packed_forward_and_backward(seed):
    r = np.random.default_rng(3000 + seed)
    nseq = int(r.integers(1, 7))
    lens = tuple(int(x) for x in r.choice([0, 1, 2, 31, 63, 64, 65, 127, 200, 257, 400], size=nseq))
    if sum(lens) == 0:
        lens = lens[:-1] + (5,)
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 4, 8]))
    causal = bool(r.random() < 0.8)
    window = int(r.choice([0, 0, 3, 100])) if causal else 0
    w = synth.VarlenWorkload(f"rand_packed{seed}", sum(lens), nseq, Hkv * G, Hkv, D,
                             str(r.choice(["fp16", "bf16"])), causal, window, 4000 + seed, lens)
    log(f"random packed case {w.name}: lens={lens} Hq={w.Hq} Hkv={Hkv} D={D} {w.dtype} causal={causal} "
        f"window={window}")
    inp = synth.make_varlen_inputs(w)
    o64, lse64 = oracle.fwd_varlen(inp["q"], inp["k"], inp["v"], inp["cu"], w.scale, causal, window)
    q, k, v, do, cu = (inp[n].cuda() for n in ("q", "k", "v", "dout", "cu"))
    o, lse = poisoned_like(q), poisoned_like(torch.empty((1, w.Hq, w.T), dtype=torch.float32, device="cuda"))
    ab.attn_fwd_varlen(q, k, v, o, lse, cu, inp["max_seqlen"], w.scale, causal=causal, window=window)
    torch.cuda.synchronize()
    check_close("o", o.cpu().double().numpy(), o64)
    check_lse("lse", lse.cpu().numpy(), lse64)
    o_st = torch.from_numpy(o64).to(synth.DTYPES[w.dtype])
    lse32 = torch.from_numpy(lse64).to(torch.float32)
    # make_args keeps raw device pointers only: the device copies must outlive the call
    o_dev, lse_dev = o_st.cuda(), lse32.cuda()
    dq, dk, dv = poisoned_like(q), poisoned_like(k), poisoned_like(v)
    args = ab.make_args(q, k, v, o_dev, do, lse_dev, dq, dk, dv, scale=w.scale, causal=causal,
                        window=window, cu_seqlens=cu, max_seqlen=inp["max_seqlen"])
    need = ab.attn_bwd_workspace_size(args)
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    args.workspace, args.workspace_bytes = ws.data_ptr(), need
    ab.attn_bwd_ex(args)
    torch.cuda.synchronize()
    ref = oracle.bwd_varlen(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, inp["cu"], w.scale, causal, window)
    for name, got, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.cpu().double().numpy(), r_)


@pytest.mark.parametrize("seed", range(N_TOPK))
def test_random_topk_backward(seed):
    r = np.random.default_rng(5000 + seed)
    Hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 8, 16, 32, 40, 64 // Hkv]))
    Sq, Skv = int(r.integers(1, 120)), int(r.integers(1, 200))
    w = synth.Workload(f"rand_topk{seed}", int(r.integers(1, 3)), Sq, Skv, Hkv * G, Hkv, 576, 512,
                       str(r.choice(["fp16", "bf16"])), bool(r.random() < 0.8), 0, int(r.integers(1, 130)),
                       6000 + seed)
    log(f"random top-k case {w.name}: B={w.B} Sq={Sq} Skv={Skv} Hq={w.Hq} Hkv={Hkv} topk={w.topk} {w.dtype} "
        f"causal={w.causal}")
    inp = synth.make_inputs(w)
    idx = inp["idx"]
    if r.random() < 0.5:  # corrupt a tenth of the entries
        m = torch.from_numpy(r.random(idx.shape) < 0.1)
        idx = torch.where(m, torch.from_numpy(r.integers(-2, Skv + 3, size=idx.shape).astype(np.int32)), idx)
    o64, lse64 = oracle.fwd(inp["q"], inp["k"], inp["v"], w.scale, w.causal, 0, idx.numpy())
    o_st = torch.from_numpy(o64).to(synth.DTYPES[w.dtype])
    lse32 = torch.from_numpy(lse64).to(torch.float32)
    g = to_gpu(inp)
    o_dev, lse_dev, idx_dev = o_st.cuda(), lse32.cuda(), idx.cuda()
    dq, dk, dv = ab.backward(g["q"], g["k"], g["v"], o_dev, g["dout"], lse_dev, causal=w.causal, topk_idx=idx_dev)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, w.scale, w.causal, 0, idx.numpy())
    for name, got, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.cpu().double().numpy(), r_)
