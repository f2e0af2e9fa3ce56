"""attn_bwd_noalloc, the entry point that allocates nothing, against attn_bwd_ex on the GPU.

Both run the same kernels; the no-allocation entry point takes its workspace from the library's
static per-device scratch instead of the caller's buffer.  Two calls in a row, the second with a
smaller input, each compared with attn_bwd_ex on the same inputs: bit for bit on the dense and
packed paths (deterministic), within the tolerance on the top-k path (its dK/dV sum f32 atomic
additions in no fixed order).  A call needing more than the scratch is refused."""
import numpy as np
import pytest
import torch

import attention_backward_amd as ab
from attention_backward_amd import synth
from tests.helpers import check_close, log, poisoned_like, prepare, to_gpu

pytestmark = pytest.mark.gpu


def args_for(g, w, outs, cu=None, max_seqlen=None):
    dq, dk, dv = outs
    return ab.make_args(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], dq, dk, dv, scale=w.scale,
                        causal=w.causal, window=w.window, topk_idx=g.get("idx"), cu_seqlens=cu, max_seqlen=max_seqlen)


def both(g, w, cu=None, max_seqlen=None):
    """(attn_bwd_ex with a torch workspace, attn_bwd_noalloc) outputs on the same inputs."""
    ref = tuple(poisoned_like(g[n]) for n in ("q", "k", "v"))
    a = args_for(g, w, ref, cu, max_seqlen)
    need = ab.attn_bwd_workspace_size(a)
    assert 0 < need <= ab._lib.NOALLOC_SCRATCH_BYTES
    ws = poisoned_like(torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda"))
    a.workspace, a.workspace_bytes = ws.data_ptr(), need
    ab.attn_bwd_ex(a)
    got = tuple(poisoned_like(g[n]) for n in ("q", "k", "v"))
    ab.attn_bwd_noalloc(args_for(g, w, got, cu, max_seqlen))
    torch.cuda.synchronize()
    return [x.cpu() for x in ref], [x.cpu() for x in got]


def same_bits(ref, got):
    for name, x, y in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{name} differs from attn_bwd_ex"


def dense(name, **kw):
    base = dict(B=1, Sq=256, Skv=256, Hq=2, Hkv=2, Dqk=128, Dv=128, dtype="fp16", causal=True, window=0, topk=0,
                seed=900)
    base.update(kw)
    return synth.Workload(name=name, **base)


def test_dense_two_calls_second_smaller():
    for w in (dense("na_gqa_g4_bf16", B=2, Sq=777, Skv=777, Hq=8, Hkv=2, dtype="bf16", seed=901),
              dense("na_swa_d64_fp16", Sq=300, Skv=300, Hq=4, Hkv=2, Dqk=64, Dv=64, window=50, seed=902)):
        log(f"no-alloc case {w.name}")
        g = to_gpu(prepare(w))
        same_bits(*both(g, w))


def test_packed_split_two_calls_second_smaller():
    """Packed calls with an even head group use the scratch for the work-queue counter and the
    two f32 dK/dV slices: the counter must start at zero on every call."""
    for lens, seed in (((500, 3, 260, 0, 129), 910), ((97, 64), 911)):
        w = synth.VarlenWorkload(f"na_vl_{seed}", sum(lens), len(lens), 8, 2, 128, "bf16", True, 0, seed, lens)
        inp = synth.make_varlen_inputs(w)
        from tests.test_gpu_varlen import oracle_o_lse
        _, _, o_st, lse32 = oracle_o_lse(inp, w)
        log(f"no-alloc packed case lens={lens}")
        g = {n: inp[n].cuda() for n in ("q", "k", "v", "dout")}
        g["o"], g["lse"] = o_st.cuda(), lse32.cuda()
        same_bits(*both(g, w, cu=inp["cu"].cuda(), max_seqlen=inp["max_seqlen"]))


def test_topk_two_calls_second_smaller():
    for Sq, Skv, topk, seed in ((40, 96, 24, 920), (9, 33, 5, 921)):
        w = synth.Workload(name=f"na_topk_{seed}", B=1, Sq=Sq, Skv=Skv, Hq=16, Hkv=1, Dqk=576, Dv=512, dtype="bf16",
                           causal=True, window=0, topk=topk, seed=seed)
        log(f"no-alloc top-k case Sq={Sq} Skv={Skv} topk={topk}")
        g = to_gpu(prepare(w))
        ref, got = both(g, w)
        assert torch.equal(ref[0].view(torch.int16), got[0].view(torch.int16)), "dq differs from attn_bwd_ex"
        for name, x, y in zip(("dk", "dv"), ref[1:], got[1:]):
            check_close(name, y.double().numpy(), x.double().numpy())


def test_over_the_scratch_is_refused():
    w = dense("na_big", B=8, Sq=65536, Skv=65536, Hq=32, Hkv=32)
    t = torch.empty((1, 16, 1, 128), dtype=torch.float16, device="cuda")  # never read: refused first
    a = ab.make_args(t, t, t, t, t, torch.empty((1, 1, 16), device="cuda"), t, t, t, scale=w.scale)
    a.B, a.Sq, a.Skv, a.Hq, a.Hkv = w.B, w.Sq, w.Skv, w.Hq, w.Hkv
    assert ab.attn_bwd_workspace_size(a) > ab._lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ab.AttnBwdError) as e:
        ab.attn_bwd_noalloc(a)
    assert e.value.status == ab._lib.ATTN_E_WORKSPACE
    _ = np
