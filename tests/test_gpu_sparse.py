"""Parity of the top-k (gathered-KV) backward with the f64 oracle, through the C ABI.

The index list of each (b, query i, kv head) is a multiset of keys: every occurrence counts once,
entries < 0, >= Skv or (causal) past the diagonal are ignored, and fewer visible keys than topk
leaves -1 padding (TileLang PR #2592 page, the sparse MLA backward; the oracle's reading).  dK and
dV are summed with f32 atomics, so their bits may differ run to run; every run is held to the
same tolerance, |gpu - ref| <= 5e-3 + 1e-2 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_backward_amd import synth
from tests.helpers import check_close, log, prepare, sample_rows
from tests.test_gpu_parity import full_compare, run

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
C5 = "sparse_mla_b1_sq4096_skv8192_h64_dqk576_dv512_top2048_bf16"


def sparse(name, **kw):
    base = dict(B=1, Sq=70, Skv=150, Hq=64, Hkv=1, Dqk=576, Dv=512, dtype="bf16", causal=True, window=0, topk=100,
                seed=200)
    base.update(kw)
    return synth.Workload(name=name, **base)


SMALL = [
    # topk not a multiple of the 32-slot chunk; queries i < 19 see fewer than 100 keys (-1 padding)
    sparse("mla_h64_bf16_padded"),
    # G = 8 < 32 query heads per workgroup block, two KV heads, B = 2, fp16
    sparse("gqa_g8_fp16", B=2, Sq=40, Skv=64, Hq=16, Hkv=2, dtype="fp16", topk=48, seed=201),
    # G = 40: a full block of 32 heads plus a block of 8; non-causal lists over every key
    sparse("g40_noncausal", Sq=33, Skv=90, Hq=40, Hkv=1, causal=False, topk=64, seed=202),
    # Sq > Skv: the first queries see no key at all (empty rows)
    sparse("causal_sq_gt_skv", Sq=80, Skv=50, Hq=32, Hkv=1, topk=20, seed=203),
    # fp16 with G = 64 (one workgroup per query row and KV head covers every head), two KV heads
    sparse("mla_h64_fp16_two_kv", B=2, Sq=37, Skv=80, Hq=128, Hkv=2, dtype="fp16", topk=40, seed=204),
    # fp16 with G = 128: two 64-head blocks of one query row
    sparse("g128_fp16", Sq=20, Skv=45, Hq=128, Hkv=1, dtype="fp16", topk=33, seed=205),
    # Sq = 600: each key block's queries span three dK/dV query chunks of 256 (counted from the
    # last query: [344, 600), [88, 344), [0, 88)), whose partial blocks add into the accumulators;
    # G = 24 ends with a ragged 8-head block; Skv = 700 ends with a ragged 28-key block
    sparse("multi_chunk_g24_bf16", Sq=600, Skv=700, Hq=24, Hkv=1, topk=96, seed=206),
    sparse("multi_chunk_g24_fp16", B=2, Sq=600, Skv=700, Hq=24, Hkv=1, dtype="fp16", topk=70, seed=207),
]


@pytest.mark.parametrize("w", [w for w in SMALL if w.dtype == "bf16"], ids=lambda w: w.name)
def test_sparse_small_bf16_reexpressed_in_fp16(w):
    """The top-k kernels on fp16 copies of bf16 inputs scaled by powers of two (bf16 outputs)."""
    from attention_backward_amd import _lib

    full_compare(w, bf16_arith=_lib.ATTN_BF16_FP16)


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_sparse_small_full_parity(w):
    inp = prepare(w)
    _, (dq, dk, dv) = full_compare(w, inp)
    # keys that no list selects get exactly zero gradients
    idx = inp["idx"].numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            sel = np.zeros(w.Skv, bool)
            for i in range(w.Sq):
                for j in idx[b, i, g]:
                    if 0 <= j < w.Skv and (not w.causal or j <= i + w.Skv - w.Sq):
                        sel[j] = True
            assert torch.all(dk[b, ~torch.from_numpy(sel), g] == 0)
            assert torch.all(dv[b, ~torch.from_numpy(sel), g] == 0)


@pytest.mark.parametrize("hq,dtype", [(32, "bf16"), (64, "fp16")])
def test_sparse_duplicates_and_out_of_range_entries(hq, dtype):
    """Each occurrence of a key counts; negative, too-large and (causal) future entries are dropped."""
    w = sparse("dups", Sq=48, Skv=96, Hq=hq, Hkv=1, dtype=dtype, topk=72, seed=210)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(211)
    idx = inp["idx"].numpy().copy()
    Sq, Skv, off = w.Sq, w.Skv, w.Skv - w.Sq
    for i in range(Sq):
        row = idx[0, i, 0]
        vis = i + off + 1
        row[:10] = rng.integers(0, vis, 10)           # repeats of visible keys
        row[10:14] = row[0]                            # one key four more times
        row[14] = -7                                   # negative
        row[15] = Skv + 3                              # past the end
        row[16] = min(Skv - 1, i + off + 1 + int(rng.integers(0, 5)))  # future key (ignored when causal)
        if i + off + 1 >= Skv:
            row[16] = -1
    inp["idx"] = torch.from_numpy(idx)
    from oracle import forward as oracle_forward

    inp["o"], inp["lse"] = oracle_forward.make_o_lse(w, inp)
    full_compare(w, inp)


def test_sparse_full_size_sampled_parity():
    """The full top-k workload in the benchmark's launch configuration, on sampled rows."""
    w = W[C5]
    log(f"case {C5} (full size, sampled rows)")
    inp = prepare(w)
    dq, dk, dv = run(inp, w)
    rng = np.random.default_rng(9)
    qrows = sample_rows(rng, 32, w.B, w.Sq, w.Hq)
    # key rows: edges, the last keys (selected by few queries) and random ones
    krows = sample_rows(rng, 32, w.B, w.Skv, w.Hkv, extra_i=(w.Skv - 3, w.Skv // 2))
    args = (inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale)
    ref_dq = oracle.bwd_dq_rows(*args, qrows, w.causal, w.window, inp["idx"])
    ref_dk, ref_dv = oracle.bwd_dkv_rows(*args, krows, w.causal, w.window, inp["idx"])
    check_close("dq rows", dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]].double().numpy(), ref_dq)
    check_close("dk rows", dk[krows[:, 0], krows[:, 1], krows[:, 2]].double().numpy(), ref_dk)
    check_close("dv rows", dv[krows[:, 0], krows[:, 1], krows[:, 2]].double().numpy(), ref_dv)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    # every dq row of one (batch, head) slice: query head 37, all 4096 query rows
    h = 37
    allq = np.array([(0, i, h) for i in range(w.Sq)], np.int64)
    check_close(f"dq head {h}, every row", dq[0, :, h].double().numpy(),
                oracle.bwd_dq_rows(*args, allq, w.causal, w.window, inp["idx"]))
    # contiguous key blocks of the KV head: the first keys (every query may list them), a block in
    # the middle, and the last keys (listed by the last queries only)
    kb = np.array([(0, j, 0) for j in list(range(0, 64)) + list(range(4064, 4128)) + list(range(w.Skv - 64, w.Skv))],
                  np.int64)
    bk, bv = oracle.bwd_dkv_rows(*args, kb, w.causal, w.window, inp["idx"])
    check_close("dk key blocks", dk[0, kb[:, 1], 0].double().numpy(), bk)
    check_close("dv key blocks", dv[0, kb[:, 1], 0].double().numpy(), bv)
    # unattended keys: exactly zero
    idx = inp["idx"].numpy().reshape(-1)
    sel = np.zeros(w.Skv, bool)
    sel[idx[idx >= 0]] = True
    log(f"  {int((~sel).sum())} keys selected by no query")
    unsel = torch.from_numpy(~sel)
    assert torch.all(dk[0, unsel] == 0) and torch.all(dv[0, unsel] == 0)


def prepare_shared(w):
    """Inputs of the shared-latent form: V is the first Dv columns of K (O and lse from the forward
    over that V)."""
    import oracle.forward as oracle_forward

    inp = synth.make_inputs(w)
    inp["v"] = inp["k"][..., : w.Dv].contiguous()
    if w.B * w.Sq * w.Skv * w.Hq <= 4 * 2 ** 20:
        o, lse = oracle.fwd(inp["q"], inp["k"], inp["v"], w.scale, w.causal, w.window, inp["idx"].numpy())
        inp["o"] = torch.from_numpy(o).to(synth.DTYPES[w.dtype])
        inp["lse"] = torch.from_numpy(lse).to(torch.float32)
    else:
        inp["o"], inp["lse"] = oracle_forward.make_o_lse(w, inp)
    return inp


def run_shared(inp, w):
    import attention_backward_amd as ab
    from tests.helpers import poisoned_like, to_gpu

    g = to_gpu(inp)
    dq, dkv = poisoned_like(g["q"]), poisoned_like(g["k"])
    args = ab.make_args(g["q"], g["k"], None, g["o"], g["dout"], g["lse"], dq, dkv, None, scale=w.scale,
                        causal=w.causal, window=w.window, topk_idx=g["idx"], kv_shared=True)
    need = ab.attn_bwd_workspace_size(args)
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    args.workspace, args.workspace_bytes = ws.data_ptr(), need
    ab.attn_bwd_ex(args)
    torch.cuda.synchronize()
    return dq.cpu(), dkv.cpu()


@pytest.mark.parametrize("w", SMALL[:2], ids=[w.name for w in SMALL[:2]])
def test_sparse_shared_latent_parity(w):
    """Shared-latent form (the TileLang PR #2592 page's sparse MLA op returns dq and dkv): one KV
    tensor whose first Dv columns are V; dkv = dK + [dV, 0] of the oracle with V = KV[..., :Dv]."""
    log(f"case {w.name} (shared latent)")
    inp = prepare_shared(w)
    dq, dkv = run_shared(inp, w)
    rdq, rdk, rdv = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale, w.causal,
                               w.window, inp["idx"])
    rdkv = rdk.copy()
    rdkv[..., : w.Dv] += rdv
    check_close("dq", dq.double().numpy(), rdq)
    check_close("dkv", dkv.double().numpy(), rdkv)


def test_sparse_shared_latent_full_size_sampled():
    """The top-k workload in its shared-latent form, in the benchmark's launch configuration, on
    sampled rows."""
    w = W[C5]
    log(f"case {C5} (shared latent, full size, sampled rows)")
    inp = prepare_shared(w)
    dq, dkv = run_shared(inp, w)
    rng = np.random.default_rng(19)
    qrows = sample_rows(rng, 24, w.B, w.Sq, w.Hq)
    krows = sample_rows(rng, 24, w.B, w.Skv, w.Hkv, extra_i=(w.Skv - 3, w.Skv // 2))
    args = (inp["q"], inp["k"], inp["v"], inp["o"], inp["dout"], inp["lse"], w.scale)
    ref_dq = oracle.bwd_dq_rows(*args, qrows, w.causal, w.window, inp["idx"])
    ref_dk, ref_dv = oracle.bwd_dkv_rows(*args, krows, w.causal, w.window, inp["idx"])
    ref_dkv = ref_dk.copy()
    ref_dkv[..., : w.Dv] += ref_dv
    check_close("dq rows", dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]].double().numpy(), ref_dq)
    check_close("dkv rows", dkv[krows[:, 0], krows[:, 1], krows[:, 2]].double().numpy(), ref_dkv)
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dkv.float()).all()
