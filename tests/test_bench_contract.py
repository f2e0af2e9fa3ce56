"""The benchmark's contract on the CPU: one GPU only, and the flop count of its metric.

The metric is 2.5 x the forward over the exact unmasked (query, key, head) pairs, forward =
(2 Dqk + 2 Dv) flops per pair.  The pair counts are pinned here to closed forms: S(S+1)/2 per head
for a causal square call, sum_i min(i + 1, W) for a window of W keys (7,864,832 per head at
T = 8192, W = 1024), Sq * topk for the top-k lists, and the sum over sequences for packed calls.
"""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_backward_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pair_counts_closed_forms():
    w = synth.WORKLOADS
    S = 2048
    assert bench.pairs(w["mha_causal_b2_s2048_h32_d128_fp16"]) == S * (S + 1) // 2 * 2 * 32
    assert bench.pairs(w["gqa_causal_b1_t16384_hq32_hkv4_d128_bf16"]) == 16384 * 16385 // 2 * 32
    # window of 1024 keys including the diagonal
    assert bench.pairs(w["swa_gqa_b2_t8192_hq16_hkv8_d64_w1024_fp16"]) == 7_864_832 * 2 * 16
    assert bench.pairs(w["swa_gqa_b2_t8000_hq16_hkv8_d64_w1024_fp16"]) == 7_668_224 * 2 * 16
    assert bench.pairs(w["sparse_mla_b1_sq4096_skv8192_h64_dqk576_dv512_top2048_bf16"]) == 4096 * 2048 * 64
    # bottom-right alignment: Sq < Skv adds Skv - Sq visible keys to every row
    x = w["mha_causal_b1_s256_h2_d128_fp16"].with_(Sq=100, Skv=160, B=1, Hq=1, Hkv=1)
    assert bench.pairs(x) == sum(i + 60 + 1 for i in range(100))
    # Sq > Skv: the first Sq - Skv rows see nothing
    y = x.with_(Sq=160, Skv=100)
    assert bench.pairs(y) == sum(max(0, i - 60 + 1) for i in range(160))


def test_metric_flops_of_the_headline():
    w = synth.WORKLOADS["mha_causal_b2_s2048_h32_d128_fp16"]
    flops = 2.5 * bench.pairs(w) * (2 * w.Dqk + 2 * w.Dv)
    assert abs(flops - 171.88e9) < 0.01e9


def test_packed_pair_count_is_the_sum_over_sequences():
    vw = synth.VARLEN_WORKLOADS["varlen_gqa_t16384_n8_hq32_hkv4_d128_bf16"]
    lens = synth.draw_seqlens(np.random.Generator(np.random.PCG64(vw.seed)), vw.T, vw.nseq)  # drawn first
    assert bench.varlen_pairs(vw, lens) == sum(int(n) * (int(n) + 1) // 2 for n in lens) * vw.Hq
    vs = synth.VARLEN_WORKLOADS["varlen_swa_gqa_t8192_n5_hq32_hkv4_d64_w512_bf16"]
    lens = synth.draw_seqlens(np.random.Generator(np.random.PCG64(vs.seed)), vs.T, vs.nseq)
    assert bench.varlen_pairs(vs, lens) == sum(sum(min(i + 1, 512) for i in range(int(n))) for n in lens) * vs.Hq
