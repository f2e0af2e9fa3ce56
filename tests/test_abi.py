"""The C-ABI library on the CPU: it loads, exports every entry point include/attn_bwd.h declares,
and rejects invalid arguments on the host (before any HIP call) with the documented status."""
import ctypes
import os
import re

import pytest

import attention_backward_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_bwd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = ab.load()
    names = declared_functions()
    assert set(names) == set(ab.EXPORTS), names
    for n in names:
        assert getattr(lib, n) is not None


PACKED = dict(cu_seqlens=0x100000, nseq=3, max_seqlen=2000, B=1, Sq=4096, Skv=4096)


def valid_args(**kw):
    a = ab.attn_bwd_args()
    fake = 0x100000  # aligned, never dereferenced: every case below fails validation first
    for f in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"):
        setattr(a, f, fake)
    a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.Dqk, a.Dv, a.topk = 2, 2048, 2048, 32, 32, 128, 128, 0
    a.scale, a.causal, a.window, a.dtype = 0.088, 1, 0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_workspace_size():
    assert ab.attn_bwd_workspace_size(valid_args()) == 2 * (2 * 32 * 2048 * 4)
    # never Hq-shaped dK/dV: a head group of 2 or 4 needs the same delta-only workspace
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=8)) == 2 * (2 * 32 * 2048 * 4)
    # dense batches store dK/dV once at Hkv from one workgroup per key block, whatever the head
    # group: no f32 dK/dV accumulators and no work-queue counter
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=4)) == 2 * (2 * 32 * 2048 * 4)
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=1)) == 2 * (2 * 32 * 2048 * 4)
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=4, window=64)) == 2 * (2 * 32 * 2048 * 4)
    assert ab.attn_bwd_workspace_size(valid_args(B=1, Sq=3, Hq=2, Hkv=2)) == 512  # 256-byte granularity
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=5)) == 0
    # top-k: delta and lse rows, f32 dK/dV accumulators at Hkv, u16 key counts [B,Hkv,Sq,Skv]
    a = valid_args(topk_idx=0x100000, topk=2048, B=1, Sq=4096, Skv=8192, Hq=64, Hkv=1, Dqk=576, Dv=512)
    assert ab.attn_bwd_workspace_size(a) == 2 * (64 * 4096 * 4) + 8192 * 576 * 4 + 8192 * 512 * 4 + 4096 * 8192 * 2
    # Skv is padded to a multiple of 32 in the count rows
    a = valid_args(topk_idx=0x100000, topk=8, B=1, Sq=10, Skv=50, Hq=64, Hkv=1, Dqk=576, Dv=512)
    assert ab.attn_bwd_workspace_size(a) == 2 * 2560 + 115200 + 102400 + 1280


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=0), -1),
        (dict(dk=0x100008), -1),          # misaligned output
        (dict(lse=0x100004), -1),
        (dict(B=0), -1),
        (dict(Sq=-1), -1),
        (dict(Hq=32, Hkv=5), -1),         # Hq % Hkv != 0
        (dict(causal=2), -1),
        (dict(window=-3), -1),
        (dict(window=16, causal=0), -1),  # a window needs the causal mask
        (dict(scale=0.0), -1),
        (dict(scale=float("inf")), -1),
        (dict(dtype=7), -1),
        (dict(topk=4), -1),               # topk without an index list
        (dict(Dqk=96, Dv=96), -2),        # no kernel for this head dim
        (dict(Dqk=128, Dv=64), -2),
        (dict(topk_idx=0x100000, topk=8), -2),  # top-k kernels exist for Dqk=576, Dv=512 only
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, window=4), -1),  # no window with top-k
        (dict(topk_idx=0x100002, topk=8, Dqk=576, Dv=512), -1),  # misaligned index list
        (dict(topk_idx=0x100000, topk=0, Dqk=576, Dv=512), -1),
        (dict(topk_idx=0x100000, topk=65536, Dqk=576, Dv=512), -2),  # key counts are 16-bit
        # gathers use 32-bit byte offsets within one (batch, KV head)'s K rows
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, Skv=1 << 22, Hkv=1, Hq=64), -2),
        # the 16-bit key-count mask [B,Hkv,Sq,Skv rounded up to 32] is bounded at 1 GiB
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, B=1, Sq=16384, Skv=32769, Hkv=1, Hq=64), -2),
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, B=1, Sq=16384, Skv=32768, Hkv=1, Hq=64,
              workspace=0x100000, workspace_bytes=16), -3),  # exactly 1 GiB: valid up to the workspace
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, workspace=0x100000, workspace_bytes=1 << 20), -3),
        (dict(workspace=0x100000, workspace_bytes=16), -3),
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, kv_shared=2), -1),
        (dict(kv_shared=1), -2),  # the shared-latent form exists on the top-k path only
        (dict(bf16_arith=3), -1),
        (dict(bf16_arith=-1), -1),
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, kv_shared=1), -1),  # v and dv must be NULL
        # a valid shared-latent call up to the workspace check
        (dict(topk_idx=0x100000, topk=8, Dqk=576, Dv=512, kv_shared=1, v=0, dv=0, workspace=0x100000,
              workspace_bytes=16), -3),
        (dict(workspace=0x100080, workspace_bytes=1 << 30), -1),  # workspace not 256-byte aligned
        # the library allocates nothing: a call without a workspace is refused
        (dict(workspace=0, workspace_bytes=0), -3),
        (dict(workspace=0, workspace_bytes=1 << 30), -3),
        # packed sequences: a batch of one on the dense path
        (dict(PACKED, B=2), -1),
        (dict(PACKED, Skv=4000), -1),
        (dict(PACKED, topk_idx=0x100000, topk=8, Dqk=576, Dv=512), -1),
        (dict(PACKED, nseq=0), -1),
        (dict(PACKED, max_seqlen=0), -1),
        (dict(PACKED, max_seqlen=4097), -1),                  # longer than the packed length
        (dict(PACKED, cu_seqlens=0x100002), -1),                # misaligned offsets
        (dict(nseq=3), -1),                                     # sequence sizes without offsets
        (dict(max_seqlen=100), -1),
        (dict(PACKED, nseq=1 << 20, max_seqlen=4096), -2),      # grid too large
        (dict(PACKED, workspace=0x100000, workspace_bytes=16), -3),  # valid up to the workspace
    ],
)
def test_validation_statuses(kw, status):
    a = valid_args(**kw)
    rc = ab.load().attn_bwd_ex(ctypes.byref(a))
    assert rc == status, (kw, rc, ab.attn_bwd_strerror(rc))
    assert ab.attn_bwd_strerror(rc)


def test_plain_entry_point_validates():
    lib = ab.load()
    rc = lib.attn_bwd(None, None, None, None, None, None, None, None, None, 1, 128, 2, 2, 128, 0.1, 1, 0, None, 0, 0,
                      None, 0, None)
    assert rc == -1
    rc = lib.attn_bwd_delta(None, None, None, 1, 1, 1, 128, 0, None)
    assert rc == -1
    rc = lib.attn_bwd_delta(0x1000, 0x1000, 0x1000, 1, 1, 1, 96, 0, None)
    assert rc == -2


FWD_OK = dict(q=0x100000, k=0x100000, v=0x100000, o=0x100000, lse=0x100000, B=1, Sq=128, Skv=128, Hq=4, Hkv=2,
              D=128, scale=0.088, causal=1, window=0, dtype=0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(lse=None), -1),
    (dict(o=0x100008), -1),          # not 16-byte aligned
    (dict(lse=0x100002), -1),        # not 4-byte aligned
    (dict(Sq=0), -1),
    (dict(Skv=0), -1),
    (dict(Hkv=3), -1),               # Hq % Hkv != 0
    (dict(causal=2), -1),
    (dict(window=-1), -1),
    (dict(causal=0, window=8), -1),  # a window needs the causal mask
    (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1),
    (dict(dtype=7), -1),
    (dict(D=96), -2),
    (dict(D=576), -2),
])
def test_forward_entry_point_validates(kw, status):
    """Every case fails validation on the host, so no kernel is launched."""
    a = dict(FWD_OK, **kw)
    rc = ab.load().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"], a["Skv"], a["Hq"], a["Hkv"],
                            a["D"], a["scale"], a["causal"], a["window"], a["dtype"], None)
    assert rc == status


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), -1),
    (dict(cu=0x100002), -1),
    (dict(nseq=0), -1),
    (dict(max_seqlen=0), -1),
    (dict(max_seqlen=129), -1),     # longer than the packed length
    (dict(causal=0, window=8), -1),
    (dict(D=96), -2),
    (dict(nseq=1 << 20, T=4096, max_seqlen=4096), -2),  # grid too large
])
def test_forward_varlen_entry_point_validates(kw, status):
    a = dict(q=0x100000, k=0x100000, v=0x100000, o=0x100000, lse=0x100000, cu=0x100000, nseq=2, max_seqlen=100,
             T=128, Hq=4, Hkv=2, D=128, scale=0.088, causal=1, window=0, dtype=0)
    a.update(kw)
    rc = ab.load().attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["nseq"], a["max_seqlen"],
                                   a["T"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["window"],
                                   a["dtype"], None)
    assert rc == status


def test_bf16_reexpression_workspace():
    """bf16 calls computed on fp16 copies add a 1280-byte block (largest magnitudes in 4 x 64
    slots, scales, factors) and the copies of q, k, v, o, dout; fp16 calls never do.  The automatic
    choice weighs the split form's second products (4 Dqk flops per attended pair at 1.2 PFLOP/s)
    against three passes over the inputs (at 6.5 TB/s, plus 15 us)."""
    rows = 2 * (2 * 32 * 2048 * 4)
    nq, nk = 2 * 2048 * 32 * 128, 2 * 2048 * 8 * 128
    copies = 1280 + 2 * nq + 2 * nk + 2 * nk + 2 * (2 * nq)
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=8, dtype=1, bf16_arith=2)) == rows + copies
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=8, dtype=1, bf16_arith=1)) == rows
    assert ab.attn_bwd_workspace_size(valid_args(Hkv=8, dtype=0, bf16_arith=2)) == rows

    def auto_copies(**kw):
        a = valid_args(dtype=1, bf16_arith=0, **kw)
        return ab.attn_bwd_workspace_size(a) > 2 * align(a.B * a.Hq * a.Sq * 4)

    # 2 x 2048 causal, 32 heads, D = 128: 134M pairs, 57 us of second products against 69 us of
    # copies -> split; 16K-token causal GQA: 2.75 ms against 0.22 ms -> copies
    assert not auto_copies(Hkv=8)
    assert auto_copies(B=1, Sq=16384, Skv=16384, Hq=32, Hkv=4)
    # a 512-key window over 8192 tokens at D = 64: 29 us against 65 us -> split
    assert not auto_copies(B=1, Sq=8192, Skv=8192, Hq=32, Hkv=4, Dqk=64, Dv=64, window=512)
    # small calls keep the bf16 products
    assert not auto_copies(B=1, Sq=256, Skv=256, Hq=2, Hkv=2)


def align(n):
    return (n + 255) // 256 * 256


def test_packed_workspace():
    """delta and lse as for the batch of one; without a window, two f32 [T,Hkv,D] slices each of
    dK and dV when the head group (here 32 / 8) splits in two halves, then 256 bytes for the
    dK/dV work-queue counter."""
    acc = 4096 * 8 * 128 * 4
    assert ab.attn_bwd_workspace_size(valid_args(**dict(PACKED, Hkv=8))) == 2 * (32 * 4096 * 4) + 4 * acc + 256
    assert ab.attn_bwd_workspace_size(valid_args(**dict(PACKED, Hkv=16))) == 2 * (32 * 4096 * 4) + 8 * acc + 256
    # a head group of one cannot split: the counter only
    assert ab.attn_bwd_workspace_size(valid_args(**PACKED)) == 2 * (32 * 4096 * 4) + 256
    assert ab.attn_bwd_workspace_size(valid_args(**dict(PACKED, window=100))) == 2 * (32 * 4096 * 4)


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 4, 1, 128, dtype=torch.float16)
    with pytest.raises(TypeError):
        ab.make_args(q, q, q, q, q, torch.zeros(1, 1, 4), q, q, q, scale=0.1)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1),
    (dict(Hq=32, Hkv=5), -1),
    (dict(Dqk=96, Dv=96), -2),
    # more workspace than the static scratch: refused before any HIP call
    (dict(B=8, Sq=65536, Skv=65536, Hq=32, Hkv=32), -3),
])
def test_noalloc_entry_point_validates_on_the_host(kw, status):
    a = valid_args(**kw)
    if status == -3:
        assert ab.attn_bwd_workspace_size(a) > ab._lib.NOALLOC_SCRATCH_BYTES
    rc = ab.load().attn_bwd_noalloc(ctypes.byref(a))
    assert rc == status, (kw, rc, ab.attn_bwd_strerror(rc))


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ab._lib.NOALLOC_SCRATCH_BYTES
