"""Packed variable-length sequences (cu_seqlens) on the GPU against the f64 oracle.

Each sequence [cu[s], cu[s+1]) of the packed token axis is its own attention problem with the
masks taken inside it (flash-linear-attention issue #8: packed varlen with per-sequence BOS/EOS
offsets, and packed sliding-window GQA).  The oracle solves every sequence with its dense
functions on that slice; its packed form is pinned on the CPU against a brute force over one
block-diagonal mask.

Small cases compare every element of the forward (O, lse) and of the backward (dq, dk, dv, from
the oracle's O and lse); the lengths include 0, 1, tile-ragged and multi-block sequences.  The
packed full-size workloads compare sampled rows.  A single packed sequence gives the same bits
as the dense batch of one.  Tolerances are those of the dense tests.
"""
import numpy as np
import pytest
import torch

import attention_backward_amd as ab
import oracle
from oracle import forward as oracle_forward
from attention_backward_amd import synth
from tests.helpers import check_close, log, poisoned_like, sample_rows
from tests.test_gpu_forward import check_lse

pytestmark = pytest.mark.gpu


def vw(name, lens, Hq, Hkv, D, dtype, causal, window, seed):
    return synth.VarlenWorkload(name, sum(lens), len(lens), Hq, Hkv, D, dtype, causal, window, seed, tuple(lens))


SMALL = [
    vw("vl_mha_d128_fp16", (300, 1, 0, 257, 64, 700), 4, 4, 128, "fp16", True, 0, 400),
    vw("vl_gqa_g4_d128_bf16", (513, 255, 33, 1024), 8, 2, 128, "bf16", True, 0, 401),
    vw("vl_swa_d64_fp16", (700, 2, 129, 0, 450), 4, 2, 64, "fp16", True, 100, 402),
    vw("vl_swa_g8_d128_bf16_w37", (333, 95, 400), 8, 1, 128, "bf16", True, 37, 403),
    vw("vl_noncausal_d64_bf16", (200, 63, 65, 1), 2, 1, 64, "bf16", False, 0, 404),
]


def oracle_o_lse(inp, w):
    """O (storage dtype) and lse (f32) of the packed problem from the oracle's forward."""
    o, lse = oracle.fwd_varlen(inp["q"], inp["k"], inp["v"], inp["cu"], w.scale, w.causal, w.window)
    return o, lse, torch.from_numpy(o).to(synth.DTYPES[w.dtype]), torch.from_numpy(lse).to(torch.float32)


def gpu_fwd(inp, w):
    q, k, v, cu = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["cu"].cuda()
    o = poisoned_like(q)
    lse = poisoned_like(torch.empty((1, w.Hq, w.T), dtype=torch.float32, device="cuda"))
    ab.attn_fwd_varlen(q, k, v, o, lse, cu, inp["max_seqlen"], w.scale, causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_bwd(inp, o, lse, w, bf16_arith=0):
    g = {n: inp[n].cuda() for n in ("q", "k", "v", "dout", "cu")}
    o, lse = o.cuda(), lse.cuda()
    dq, dk, dv = poisoned_like(g["q"]), poisoned_like(g["k"]), poisoned_like(g["v"])
    args = ab.make_args(g["q"], g["k"], g["v"], o, g["dout"], lse, dq, dk, dv, scale=w.scale, causal=w.causal,
                        window=w.window, cu_seqlens=g["cu"], max_seqlen=inp["max_seqlen"], bf16_arith=bf16_arith)
    need = ab.attn_bwd_workspace_size(args)
    assert need > 0
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    args.workspace, args.workspace_bytes = ws.data_ptr(), need
    ab.attn_bwd_ex(args)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_varlen_small_full_parity(w):
    log(f"packed case {w.name}: lens={w.lens} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.dtype} causal={w.causal} "
        f"window={w.window}")
    inp = synth.make_varlen_inputs(w)
    ref_o, ref_lse, o_st, lse32 = oracle_o_lse(inp, w)
    o, lse = gpu_fwd(inp, w)
    check_close("o", o.double().numpy(), ref_o)
    check_lse("lse", lse.numpy(), ref_lse)
    dq, dk, dv = gpu_bwd(inp, o_st, lse32, w)
    ref = oracle.bwd_varlen(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, inp["cu"], w.scale, w.causal,
                            w.window)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.double().numpy(), r)


@pytest.mark.parametrize("w", [w for w in SMALL if w.dtype == "bf16"], ids=lambda w: w.name)
def test_varlen_bf16_reexpressed_in_fp16(w):
    """Packed bf16 sequences through the fp16 kernels on scaled fp16 copies (bf16 outputs)."""
    inp = synth.make_varlen_inputs(w)
    _, _, o_st, lse32 = oracle_o_lse(inp, w)
    dq, dk, dv = gpu_bwd(inp, o_st, lse32, w, bf16_arith=ab._lib.ATTN_BF16_FP16)
    ref = oracle.bwd_varlen(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, inp["cu"], w.scale, w.causal,
                            w.window)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got.double().numpy(), r)


def test_single_packed_sequence_is_the_dense_batch_of_one():
    """Same kernels, same per-row arithmetic: a packed call holding one sequence gives the bits of
    the dense call with B = 1 for O, lse and dQ.  dK and dV differ in rounding only: the packed
    call splits each head group into two halves whose f32 blocks go to two slices that the landing
    pass adds in a fixed order, where the dense call sums the whole group in one workgroup.
    Repeated packed calls agree bit for bit."""
    w = vw("vl_one", (777,), 4, 2, 128, "fp16", True, 0, 410)
    inp = synth.make_varlen_inputs(w)
    _, _, o_st, lse32 = oracle_o_lse(inp, w)
    o_p, lse_p = gpu_fwd(inp, w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    o_d, lse_d = poisoned_like(q), poisoned_like(torch.empty((1, 4, 777), dtype=torch.float32, device="cuda"))
    ab.attn_fwd(q, k, v, o_d, lse_d, w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_d.cpu().view(torch.int16))
    assert torch.equal(lse_p.view(torch.int32), lse_d.cpu().view(torch.int32))
    packed = gpu_bwd(inp, o_st, lse32, w)
    again = gpu_bwd(inp, o_st, lse32, w)
    for x, y in zip(packed, again):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "two identical packed calls differ"
    g = {n: inp[n].cuda() for n in ("q", "k", "v", "dout")}
    dq, dk, dv = poisoned_like(g["q"]), poisoned_like(g["k"]), poisoned_like(g["v"])
    ab.backward(g["q"], g["k"], g["v"], o_st.cuda(), g["dout"], lse32.cuda(), causal=True, out=(dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(packed[0].view(torch.int16), dq.cpu().view(torch.int16))
    for name, x, y in zip(("dk", "dv"), packed[1:], (dk.cpu(), dv.cpu())):
        check_close(name, x.double().numpy(), y.double().numpy())


@pytest.mark.parametrize("name", sorted(synth.VARLEN_WORKLOADS))
def test_varlen_full_size_sampled_parity(name):
    w = synth.VARLEN_WORKLOADS[name]
    inp = synth.make_varlen_inputs(w)
    cu = inp["cu"].tolist()
    log(f"packed case {name} (full size, sampled rows): cu={cu}")
    o = torch.empty((1, w.T, w.Hq, w.D), dtype=torch.float64)
    lse = torch.empty((1, w.Hq, w.T), dtype=torch.float64)
    for a, b in zip(cu[:-1], cu[1:]):
        o[:, a:b], lse[:, :, a:b] = oracle_forward.fwd(inp["q"][:, a:b], inp["k"][:, a:b], inp["v"][:, a:b], w.scale,
                                                       w.causal, w.window)
    o_st, lse32 = o.to(synth.DTYPES[w.dtype]), lse.to(torch.float32)
    go, glse = gpu_fwd(inp, w)
    dq, dk, dv = gpu_bwd(inp, o_st, lse32, w)
    rng = np.random.default_rng(13)
    starts = [a for a in cu[:-1]] + [b - 1 for b in cu[1:]]
    qrows = sample_rows(rng, 48, 1, w.T, w.Hq, extra_i=starts)
    krows = sample_rows(rng, 48, 1, w.T, w.Hkv, extra_i=starts)
    seq = np.searchsorted(cu, np.arange(w.T), side="right") - 1  # the sequence of every token

    def by_sequence(rows, fn):
        """fn(slice tensors, rows re-indexed into the slice) per sequence, results in row order."""
        out = [None] * len(rows)
        for s_ in np.unique(seq[rows[:, 1]]):
            a, b = cu[s_], cu[s_ + 1]
            sel = np.nonzero(seq[rows[:, 1]] == s_)[0]
            local = rows[sel].copy()
            local[:, 1] -= a
            sl = {n: inp[n][:, a:b] for n in ("q", "k", "v", "dout")}
            sl["o"], sl["lse"] = o_st[:, a:b], lse32[:, :, a:b]
            for j, r in zip(sel, fn(sl, local)):
                out[j] = r
        return out

    def q_side(sl, local):
        ro, rl = oracle_forward.fwd_rows(sl["q"], sl["k"], sl["v"], w.scale, local, w.causal, w.window)
        rdq = oracle.bwd_dq_rows(sl["q"], sl["k"], sl["v"], sl["o"], sl["dout"], sl["lse"], w.scale, local, w.causal,
                                 w.window)
        return [(ro[j].numpy(), float(rl[j]), rdq[j]) for j in range(len(local))]

    def k_side(sl, local):
        rk, rv = oracle.bwd_dkv_rows(sl["q"], sl["k"], sl["v"], sl["o"], sl["dout"], sl["lse"], w.scale, local,
                                     w.causal, w.window)
        return [(rk[j], rv[j]) for j in range(len(local))]

    qr = by_sequence(qrows, q_side)
    check_close("o rows", go[0, qrows[:, 1], qrows[:, 2]].double().numpy(), np.array([r[0] for r in qr]))
    check_lse("lse rows", glse[0, qrows[:, 2], qrows[:, 1]].numpy(), np.array([r[1] for r in qr]))
    check_close("dq rows", dq[0, qrows[:, 1], qrows[:, 2]].double().numpy(), np.array([r[2] for r in qr]))
    kr = by_sequence(krows, k_side)
    check_close("dk rows", dk[0, krows[:, 1], krows[:, 2]].double().numpy(), np.array([r[0] for r in kr]))
    check_close("dv rows", dv[0, krows[:, 1], krows[:, 2]].double().numpy(), np.array([r[1] for r in kr]))
    for t in (go, glse, dq, dk, dv):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("Hq,Hkv,dtype", [(4, 2, "fp16"), (3, 1, "bf16"), (16, 2, "bf16")],
                         ids=["g2_split_fp16", "g3_odd_bf16", "g8_split_bf16"])
def test_tokens_outside_every_sequence_keep_their_contents(Hq, Hkv, dtype):
    """Offsets ending before T (cu[nseq] < T) and a sequence longer than max_seqlen: the kernels
    (and, for an even head group, the landing of the two f32 halves) write only the rows each
    sequence covers, cut at max_seqlen, so the rows past them keep the poison.  The rows written
    match the oracle over the sequences as cut, and a second call gives the same bits."""
    w = vw(f"vl_outside_{Hq}_{Hkv}", (200, 250, 150), Hq, Hkv, 128, dtype, True, 0, 420 + Hq)
    inp = synth.make_varlen_inputs(w)
    inp["cu"] = torch.tensor([0, 200, 450], dtype=torch.int32)   # tokens 450..599: no sequence
    inp["max_seqlen"] = 230                                        # sequence 1 is cut at token 430
    log(f"packed case {w.name}: cu={inp['cu'].tolist()} T={w.T} max_seqlen=230 {dtype}")
    cut = torch.tensor([0, 200, 430], dtype=torch.int32)
    _, _, o_st, lse32 = oracle_o_lse(dict(inp, cu=cut), w)
    dq, dk, dv = gpu_bwd(inp, o_st, lse32, w)
    again = gpu_bwd(inp, o_st, lse32, w)
    for x, y in zip((dq, dk, dv), again):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "two identical packed calls differ"
    ref = oracle.bwd_varlen(inp["q"], inp["k"], inp["v"], o_st, inp["dout"], lse32, cut, w.scale, True, 0)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_close(name, got[:, :430].double().numpy(), r[:, :430])
        assert torch.all(got[:, 430:].view(torch.int16) == -1), f"{name}: rows outside every sequence were written"
