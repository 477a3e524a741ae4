"""bench.py's algorithmic work figures (the denominators of every roofline fraction it
reports), checked against the totals the scope table states for each configuration, and
its refusal of more than one GPU. CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402


def test_prefill_flops_match_the_stated_totals():
    # 587.1 GFLOP (batch 4 x seq 512), 4.523 TFLOP (1 x 8192), 55.33 TFLOP (SmolLM3-3B shape, 2 x 4096)
    for name, total, tol in (("prefill_bf16", 587.1e9, 0.05e9), ("long_prefill_bf16", 4.523e12, 0.5e9),
                             ("smollm3_prefill_bf16", 55.33e12, 5e9)):
        f = bench.prefill_flops(S.workload(name))
        assert abs(f["total"] - total) <= tol, (name, f["total"])
        assert f["total"] == sum(v for k, v in f.items() if k not in ("per_launch", "total"))


def test_prefill_flops_by_counting_products():
    # the same total from the individual matrix products of one layer, counted one by one
    s = S.workload("prefill_bf16")
    M, H, d = s.batch * s.seq, s.hidden, s.head_dim
    products = [(M, H, s.n_heads * d), (M, H, s.n_kv_heads * d), (M, H, s.n_kv_heads * d),  # q, k, v
                (M, s.n_heads * d, H),                                                     # o_proj
                (M, H, s.intermediate), (M, H, s.intermediate), (M, s.intermediate, H)]   # gate, up, down
    layer = sum(2 * m * k * n for m, k, n in products)
    visible = s.batch * sum(t + 1 for t in range(s.seq))  # causal (query, key) pairs per head
    attn = s.n_heads * visible * 2 * (2 * d)                # q.k and p.v, 2 FLOP per multiply-add
    want = s.n_layers * (layer + attn) + 2 * M * H * s.vocab
    assert bench.prefill_flops(s)["total"] == want


def test_decode_bytes_match_the_stated_total():
    # 3.295 GB per step: KV 3.018 GB, layer weights 0.212 GB, embedding 0.0566 GB, logits, KV append
    s = S.workload("decode_bf16")
    b = bench.decode_bytes(s, s.cache_len)
    assert abs(b["total"] - 3.295e9) <= 2e6
    assert abs(b["kv_read"] - 3.018e9) <= 2e6
    assert b["decode_attention_per_launch"] * s.n_layers == b["kv_read"]
    # the one-launch step is everything but the head: the embedding matrix it reads and
    # the logits it writes, less the embedding rows the step gathers itself
    head_only = 2 * s.vocab * s.hidden + b["logits"] - 2 * s.batch * s.hidden
    assert b["decode_step_per_launch"] == b["total"] - head_only


def test_backward_flops():
    # three products per linear layer (43.5 GFLOP) and 12 d per visible pair of every head (3.6 GFLOP)
    f = bench.backward_flops(S.workload("block_backward_f32"))
    assert abs(f["gemm"] - 43.5e9) <= 0.05e9 and abs(f["attention"] - 3.63e9) <= 0.01e9
    assert f["attention"] == f["attention_forward"] + f["attention_dq"] + f["attention_dkdv"]


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_dominant_class_breaks_near_ties_conservatively():
    """Within 5% of the largest summed time the class furthest below its roofline is
    reported; a clear leader is reported whatever its fraction."""
    import bench

    flops = {"per_launch": {"gate_up": 7.2e9, "down": 3.6e9, "attention": 1.2e9}}
    kern = {"gate_up": {"total_ms": 0.560, "launches": 30, "avg_us": 18.7},
            "down": {"total_ms": 0.549, "launches": 30, "avg_us": 18.3},
            "attention": {"total_ms": 0.340, "launches": 30, "avg_us": 11.3}}
    assert bench.dominant_class(kern, flops) == "down"
    kern["down"]["total_ms"] = 0.40
    assert bench.dominant_class(kern, flops) == "gate_up"
