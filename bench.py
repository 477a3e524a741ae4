"""Benchmark: SmolLM2-135M-shaped prefill (bf16, 30 layers, batch 4 x seq 512) on one
MI355X through the C ABI, plus the decode step (batch 64 over 2047 cached positions).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-graph] [--no-cpu]
                    [--profile-kernel NAME]

A step is one smol_model_prefill call: embedding, 30 blocks (RMSNorm, QKV+RoPE,
causal GQA attention, o_proj+residual, RMSNorm, gate/up+SwiGLU, down+residual),
final RMSNorm and the tied lm_head writing bf16 logits [4, 512, 49152]. Inputs and
weights are resident in HBM before the timed region. By default the step is
captured once into a HIP graph and replayed (every kernel still runs each step);
--no-graph times plain launches. Rank 0 prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E
F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA


def prefill_flops(s) -> dict:
    """Algorithmic FLOPs of one prefill (causal attention counts the visible triangle only)."""
    M, L, H, d = s.batch * s.seq, s.n_layers, s.hidden, s.head_dim
    per_layer = {
        "qkv_rope": 2 * M * H * (s.n_heads + 2 * s.n_kv_heads) * d,
        "o_proj": 2 * M * s.n_heads * d * H,
        "gate_up": 2 * M * H * 2 * s.intermediate,
        "down": 2 * M * s.intermediate * H,
        "attention": 2 * d * s.n_heads * s.seq * (s.seq + 1) * s.batch,
    }
    out = {k: v * L for k, v in per_layer.items()}
    out["lm_head"] = 2 * M * H * s.vocab
    out["per_launch"] = dict(per_layer, lm_head=out["lm_head"])
    out["total"] = sum(v for k, v in out.items() if k not in ("per_launch",))
    return out


def decode_bytes(s, P: int) -> dict:
    """Algorithmic HBM bytes of one decode step (bf16): every cached key/value read once,
    every weight read once, the new k/v written, logits written."""
    L, B, H, d, I, V = s.n_layers, s.batch, s.hidden, s.head_dim, s.intermediate, s.vocab
    layer_w = 2 * (H * (s.n_heads + 2 * s.n_kv_heads) * d + s.n_heads * d * H + 3 * H * I + 2 * H)
    kv_read = 2 * 2 * s.n_kv_heads * d * (P + 1) * B  # per layer: keys 0..P incl. the new one
    out = {
        "kv_read": kv_read * L,
        "weights": layer_w * L + 2 * V * H + 2 * H,
        "kv_append": 2 * 2 * s.n_kv_heads * d * B * L,
        "logits": 2 * B * V,
        "decode_attention_per_launch": kv_read,
        # the one-launch step (every layer up to the final norm): the cache, the layer
        # weights, the appended k/v, the embedding rows and the final norm weight
        "decode_step_per_launch": (kv_read + layer_w + 2 * 2 * s.n_kv_heads * d * B) * L + 2 * B * H + 2 * H,
    }
    out["total"] = out["kv_read"] + out["weights"] + out["kv_append"] + out["logits"]
    return out


def backward_flops(s) -> dict:
    """Algorithmic FLOPs of one block backward (forward recomputed): every linear layer
    three times (the forward product, the data gradient, the weight gradient), and per
    visible (query, key) pair of every head 12 d (S and P V forward; dV, dP, dQ, dK). By
    kernel: the forward S and P V; the dQ kernel dP and dQ (S recomputed); the dK/dV
    kernel dV and dK (S and dP recomputed), so the three add up to the 12 d."""
    M, H, I, d = s.batch * s.seq, s.hidden, s.intermediate, s.head_dim
    qkv = (s.n_heads + 2 * s.n_kv_heads) * d
    lin = 2 * M * H * (qkv + s.n_heads * d + 2 * I + I)
    pairs = s.batch * s.n_heads * s.seq * (s.seq + 1) // 2
    out = {"gemm": 3 * lin, "attention": 12 * d * pairs,
           "attention_forward": 4 * d * pairs, "attention_dq": 4 * d * pairs, "attention_dkdv": 4 * d * pairs}
    out["total"] = out["gemm"] + out["attention"]
    return out


def _time_steps(fn, steps, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def _rep_ms(fn, reps, torch, stream, before=None):
    """Per-rep durations (ms) from events recorded on `stream` around each call of fn;
    `before` runs (untimed) ahead of each rep."""
    out = []
    with torch.cuda.stream(stream):
        for _ in range(reps):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
    return out


def _pct(ms):
    a = np.asarray(ms)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.median(a)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "reps": len(ms)}


def ceilings(torch, dev):
    """Achieved ceilings on this GPU, as context for the roofline fractions: a plain
    device copy (bytes read + written per second) and a large bf16 GEMM through
    torch.matmul (hipBLASLt, used as a black box)."""
    n = 1 << 28  # 1 GiB of float32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    copy_gbps = 2 * 4 * n * 10 / (time.perf_counter() - t0) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        z = torch.matmul(x, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        z = torch.matmul(x, y)
    torch.cuda.synchronize()
    gemm_tflops = 2 * m ** 3 * 10 / (time.perf_counter() - t0) / 1e12
    del x, y, z
    return {"copy_gbps": round(copy_gbps, 1), "copy_frac_of_hbm_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
            "bf16_gemm_8192_tflops": round(gemm_tflops, 1),
            "bf16_gemm_frac_of_peak": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
            "how": "torch copy_ of 1 GiB float32; torch.matmul 8192^3 bf16 (hipBLASLt)"}


def _kernel_time(B, kernel, run_once, torch, max_launches=4096):
    """Summed duration (ms) and count of one kernel class's launches over one eager step,
    from the start/stop events the HIP runtime records at each of those dispatches
    (the library launches them with hipExtLaunchKernelGGL while timing is on)."""
    torch.cuda.synchronize()
    B.smol_timing_begin(kernel, max_launches)
    run_once()
    ms, n = B.smol_timing_end()
    return ms, n


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_prefill_b4s512_gemms.md")
TRAFFIC_DECODE_PROFILE = os.path.join(ROOT, "profiles", "traffic_decode_step_b64.md")
TRAFFIC_BACKWARD_PROFILE = os.path.join(ROOT, "profiles", "traffic_block_backward_b4s512.md")
TRAFFIC_OTHER_PROFILE = os.path.join(ROOT, "profiles", "traffic_prefill_smollm3_b2s4096.md")


def measured_traffic(key: str, path=None):
    """HBM bytes per launch of a kernel from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE passes scaled by a plain copy of known size), or None when the kernel
    sources have changed since the counters were taken. path None: the prefill GEMM
    summary, looked up when called (not when this module is imported)."""
    import hashlib
    if path is None:
        path = TRAFFIC_PROFILE
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("source-sha256: ", "source-files: ", key + ": ")))
    if key not in fields or "source-sha256" not in fields or "source-files" not in fields:
        return None
    h = hashlib.sha256()
    for f in fields["source-files"].split():
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return int(fields[key]) if h.hexdigest() == fields["source-sha256"].strip() else None


def other_prefill(B, torch, dev, name, md, reps, warmup):
    """One of the other prefill shapes (context, not the headline): graph replays of a
    whole prefill, median and p10/p90, MFMA fraction and per-class kernel durations.
    md: device weights of that shape's model."""
    from llama_decoder_only_amd import synthetic as S

    s = S.workload(name)
    cfg = B.Config.from_shape(s)
    ids = torch.from_numpy(S.token_ids(s, 0)).to(dev)
    logits = torch.empty(s.batch, s.seq, s.vocab, dtype=torch.bfloat16, device=dev)
    ws = B.workspace(cfg, B.SMOL_OP_PREFILL, s.batch, s.seq, dev)
    stream = torch.cuda.Stream()

    def step():
        B.smol_model_prefill(cfg, md, ids, logits, ws=ws, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ms = _rep_ms(lambda: g.replay(), reps, torch, stream)
    t = float(np.median(ms)) * 1e-3
    flops = prefill_flops(s)
    kern = {}
    with torch.cuda.stream(stream):
        for k in ("qkv_rope", "attention", "o_proj", "gate_up", "down", "lm_head"):
            kms, n = _kernel_time(B, k, step, torch)
            kern[k] = {"total_ms": kms, "launches": n, "avg_us": 1e3 * kms / max(n, 1)}
    del ws, logits
    rl = prefill_rooflines(kern, flops)
    dom = dominant_class({k: v for k, v in kern.items() if k in rl}, flops)
    return {"workload": f"{name}: {s.n_layers} layers, hidden {s.hidden}, {s.n_heads}/{s.n_kv_heads} heads x "
                        f"{s.head_dim}, intermediate {s.intermediate}, vocab {s.vocab}; batch {s.batch} x seq {s.seq}",
            "timing": "hip_graph (median of reps)", "ms_per_step": round(t * 1e3, 3),
            "tokens_per_s": round(s.batch * s.seq / t, 1), "rep_ms": _pct(ms),
            "algorithmic_gflop_per_step": round(flops["total"] / 1e9, 1),
            "mfma_frac": round(flops["total"] / t / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
            "roofline": dict(rl[dom], kernel=dom,
                             traffic=measured_traffic(f"{name}:{dom}-traffic-bytes-per-launch", TRAFFIC_OTHER_PROFILE)),
            "rooflines": rl}


# Classes whose summed time per step lies within this fraction of the largest count as
# tied for "dominant": the event timing and a rocprofv3 trace of the same run can rank
# two classes that close either way (the gate/up and down GEMMs of the headline prefill).
DOMINANT_TIE = 0.05


def dominant_class(kern, flops):
    """The kernel class with the most time per step; among classes within DOMINANT_TIE
    of it, the one furthest below its MFMA roofline (the conservative pick)."""
    cand = [k for k in kern if k in flops["per_launch"] and kern[k]["launches"] > 0]
    top = max(kern[k]["total_ms"] for k in cand)
    tied = [k for k in cand if kern[k]["total_ms"] >= (1.0 - DOMINANT_TIE) * top]
    return min(tied, key=lambda k: flops["per_launch"][k] / kern[k]["avg_us"])


def prefill_rooflines(kern, flops):
    """Per kernel class of a prefill: algorithmic FLOPs per launch over the class's average
    launch duration, against the bf16 MFMA peak."""
    out = {}
    for k, v in kern.items():
        if k not in flops["per_launch"] or v["launches"] == 0:
            continue
        ach = flops["per_launch"][k] / (v["avg_us"] * 1e-6) / 1e12
        out[k] = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(ach / BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(v["avg_us"], 2),
                  "launches": v["launches"], "total_ms": round(v["total_ms"], 4),
                  "algorithmic_flop_per_launch": flops["per_launch"][k]}
    return out


def _note(msg):
    """A progress line on stderr (stdout carries the one JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def other_prefills(B, torch, dev, md):
    """The long-context prefill (the same model as the headline, md) and the SmolLM3-3B
    shape (weights drawn on the GPU)."""
    from llama_decoder_only_amd import synthetic as S

    out = {"long_prefill": other_prefill(B, torch, dev, "long_prefill_bf16", md, reps=10, warmup=2)}
    _note("long prefill done")
    m5 = random_model(B, torch, dev, S.workload("smollm3_prefill_bf16"))
    out["smollm3_prefill"] = other_prefill(B, torch, dev, "smollm3_prefill_bf16", m5, reps=5, warmup=1)
    _note("SmolLM3-shaped prefill done")
    out["smollm3_prefill"]["data"] = "weights N(0, 0.02^2) drawn on the GPU (torch generator), norm weights 1"
    del m5
    torch.cuda.empty_cache()
    return out


def random_model(B, torch, dev, s, seed=1):
    """Device weights of shape s drawn on the GPU (torch's generator, N(0, std^2), norm
    weights 1): for timing only, where the values do not matter and drawing billions
    of them on the host would take minutes."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    H, I, d = s.hidden, s.intermediate, s.head_dim

    def w(*shape):
        return (torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * s.std).to(torch.bfloat16)

    ones = lambda: torch.ones(H, device=dev, dtype=torch.bfloat16)  # noqa: E731
    layers = [B.LayerWeights([ones(), w(s.n_heads * d, H), w(s.n_kv_heads * d, H), w(s.n_kv_heads * d, H),
                              w(H, s.n_heads * d), ones(), w(I, H), w(I, H), w(H, I)]) for _ in range(s.n_layers)]
    return B.ModelWeights(w(s.vocab, H), layers, ones())


def _oracle_cfg(O, s):
    return O.Config(hidden=s.hidden, n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, intermediate=s.intermediate,
                    n_layers=s.n_layers, vocab=s.vocab, max_pos=s.max_pos, rms_eps=s.rms_eps, rope_theta=s.rope_theta)


def _oracle_layer(O, layer):
    return O.LayerWeights(**{n: getattr(layer, n).f64 for n in layer.NAMES})


def _host_info():
    """CPU model, BLAS library and its thread count, as the oracle's numpy sees them."""
    from threadpoolctl import threadpool_info

    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    vendor = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas})) or "unknown"
    return model, vendor, int(threads)


def cpu_baseline(s, model, ids_np, budget_s=8.0):
    """The CPU oracle (numpy float64, as it stands) timed on the host, on bounded samples.

    Headline (the prefill workload of the metric): whole sequences of the batch 4 x seq
    512 prefill, one after another until about budget_s seconds have passed. `configs`
    gives the other workloads, each a stated sample: the float32 block and the 30-layer
    float32 model at batch 1 x seq 128 (whole); the seq-8192 prefill as one block over
    the whole sequence plus the head on 256 rows, scaled to 30 blocks and 8192 rows
    (extrapolated: the blocks cost the same); the decode step for 8 of its 64 sequences
    (2047 cached positions, scaled to 64; the cache values of one layer serve all 30);
    the SmolLM3-3B shape as one block over one sequence of 4096 plus the head on 128 rows,
    scaled to 36 blocks, 2 sequences and 8192 rows (extrapolated)."""
    import oracle.smol as O
    from llama_decoder_only_amd import synthetic as S

    cpu, blas, threads = _host_info()
    cfg = _oracle_cfg(O, s)
    om = O.ModelWeights(embed=model.embed.f64, layers=[_oracle_layer(O, l) for l in model.layers],
                        final_norm=model.final_norm.f64)
    t0 = time.perf_counter()
    done = 0
    while done < ids_np.shape[0]:
        O.model_prefill(ids_np[done:done + 1], om, cfg)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    out = {"value": done * s.seq / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} of {ids_np.shape[0]} sequences x {s.seq} tokens, full 30-layer forward and all "
                     f"logits, numpy float64, {dt:.1f} s; host has {os.cpu_count()} logical CPUs",
           "cpu_model": cpu, "blas": blas, "configs": {}}
    cf = out["configs"]

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # float32 block and 30-layer model, batch 1 x seq 128: whole
    s1 = S.workload("block_f32")
    l1 = _oracle_layer(O, S.layer_weights(s1, 0, 0))
    x1 = S.hidden_states(s1, 0).f64
    t = timed(lambda: O.block_forward(x1, l1, _oracle_cfg(O, s1)))
    cf["block_f32"] = {"tokens_per_s": round(s1.seq / t, 1), "seconds": round(t, 3), "sample": "whole (1 x 128)"}
    s1b = S.workload("model_f32")
    m1b = S.model_weights(s1b, 0)
    om1b = O.ModelWeights(embed=m1b.embed.f64, layers=[_oracle_layer(O, l) for l in m1b.layers],
                          final_norm=m1b.final_norm.f64)
    ids1b = S.token_ids(s1b, 0)
    t = timed(lambda: O.model_prefill(ids1b, om1b, _oracle_cfg(O, s1b)))
    cf["model_f32"] = {"tokens_per_s": round(s1b.seq / t, 1), "seconds": round(t, 3), "sample": "whole (1 x 128)"}
    del m1b, om1b
    # seq-8192 prefill: one block over the whole sequence, the head on 256 rows
    s3 = S.workload("long_prefill_bf16")
    ids3 = S.token_ids(s3, 0)
    x3 = O.embed(ids3, om.embed)
    tb = timed(lambda: O.block_forward(x3, om.layers[0], cfg, layer=0))
    th = timed(lambda: O.lm_head(x3[0, :256], om.final_norm, om.embed, cfg))
    t = tb * s3.n_layers + th * s3.seq / 256
    cf["long_prefill_bf16"] = {"tokens_per_s": round(s3.seq / t, 1), "seconds": round(t, 2), "extrapolated": True,
                               "sample": f"one block at 1 x 8192 ({tb:.1f} s) x 30 + the head on 256 rows "
                                         f"({th:.2f} s) x 32"}
    del x3
    # decode step: 8 of 64 sequences over 2047 cached positions
    s4 = S.workload("decode_bf16")
    nb = 8
    kc, vc = S.kv_cache_values(S.workload("decode_bf16", batch=nb), 0, 0, s4.cache_len)
    kc64, vc64 = kc.f64, vc.f64
    dids = S.token_ids(s4, 0, S.T_DECODE_IDS)[:nb, 0]
    t = timed(lambda: O.decode_step(dids, s4.cache_len, om, cfg, [kc64] * s4.n_layers, [vc64] * s4.n_layers))
    t *= s4.batch / nb
    cf["decode_bf16"] = {"tokens_per_s": round(s4.batch / t, 1), "ms_per_step": round(t * 1e3, 1),
                         "extrapolated": True,
                         "sample": f"{nb} of {s4.batch} sequences (2047 cached), scaled x {s4.batch // nb}; "
                                   "one layer's cache values serve all 30 layers"}
    del kc, vc, kc64, vc64
    # SmolLM3-3B shape: one block over one sequence of 4096, the head on 128 rows
    # (constant weights: drawing 3 G normals would take minutes, and the oracle's time
    # does not depend on the values)
    s5 = S.workload("smollm3_prefill_bf16")
    c5 = _oracle_cfg(O, s5)
    H5, I5, q5, k5 = s5.hidden, s5.intermediate, s5.n_heads * s5.head_dim, s5.n_kv_heads * s5.head_dim
    l5 = O.LayerWeights(attn_norm=np.ones(H5), wq=np.full((q5, H5), 0.02), wk=np.full((k5, H5), 0.02),
                        wv=np.full((k5, H5), -0.02), wo=np.full((H5, q5), 0.02), mlp_norm=np.ones(H5),
                        w_gate=np.full((I5, H5), 0.02), w_up=np.full((I5, H5), -0.02), w_down=np.full((H5, I5), 0.02))
    x5 = S.hidden_states(S.workload("smollm3_prefill_bf16", batch=1), 0).f64 * 0.02
    tb = timed(lambda: O.block_forward(x5, l5, c5, layer=0))
    del l5
    e5 = np.full((s5.vocab, s5.hidden), 0.02)
    th = timed(lambda: O.lm_head(x5[0, :128], np.ones(s5.hidden), e5, c5))
    del e5, x5
    t = tb * s5.n_layers * s5.batch + th * s5.batch * s5.seq / 128
    cf["smollm3_prefill_bf16"] = {"tokens_per_s": round(s5.batch * s5.seq / t, 2), "seconds": round(t, 1),
                                  "extrapolated": True,
                                  "sample": f"one block at 1 x 4096 ({tb:.1f} s) x 36 blocks x 2 sequences + the "
                                            f"head on 128 rows ({th:.2f} s) x 64; constant weights (the time "
                                            "does not depend on the values)"}
    return out


def backward_section(B, S, torch, dev, stream, args):
    """smol_block_backward on one SmolLM2-135M block, float32, batch 4 x seq 512: the
    whole call (graph-replayed, median over reps) and each kernel class's summed
    launch durations from the runtime's dispatch events."""
    sb = S.workload("block_backward_f32")
    cfg = B.Config.from_shape(sb)
    w = B.upload_layer(S.layer_weights(sb, 0, 0), dev)
    x, dy = B.to_device(S.hidden_states(sb, 0), dev), B.to_device(S.output_grad(sb, 0), dev)
    dx = torch.empty_like(x)
    g = B.LayerGrads.zeros_like(w)
    ws = torch.empty(B.smol_block_backward_workspace_size(cfg, sb.batch, sb.seq), dtype=torch.uint8, device=dev)

    def bstep():
        B.smol_block_backward(cfg, w, x, dy, dx, g, ws=ws, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(3):
            bstep()
    torch.cuda.synchronize()
    ref = dx.clone()
    fn, mode = bstep, "eager"
    if not args.no_graph:
        bg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bg, stream=stream):
            bstep()
        dx.zero_()
        bg.replay()
        torch.cuda.synchronize()
        if not torch.equal(dx, ref):
            raise RuntimeError("backward graph replay differs from the eager result")
        fn, mode = bg.replay, "hip_graph"
    reps = _rep_ms(fn, max(args.steps, 5), torch, stream)
    t_s = float(np.median(reps)) * 1e-3
    fl = backward_flops(sb)
    kern = {}
    for k in ("bw_gemm", "bw_attn_fwd", "bw_attn_dq", "bw_attn_dkdv", "bw_rows"):
        with torch.cuda.stream(stream):
            ms, n = _kernel_time(B, k, bstep, torch)
        kern[k] = {"us": round(ms * 1e3, 2), "launches": n}
    ach = {"bw_gemm": fl["gemm"], "bw_attn_fwd": fl["attention_forward"], "bw_attn_dq": fl["attention_dq"],
           "bw_attn_dkdv": fl["attention_dkdv"]}
    for k, f in ach.items():
        kern[k]["tflops"] = round(f / (kern[k]["us"] * 1e-6) / 1e12, 2) if kern[k]["us"] > 0 else None
    dom = max(ach, key=lambda k: kern[k]["us"])
    btraffic = measured_traffic("bw_gemm-traffic-bytes-per-call", TRAFFIC_BACKWARD_PROFILE)
    dom_tf = kern[dom]["tflops"] or 0.0
    del w, x, dy, dx, g, ws
    return {
        "workload": "backward of one SmolLM2-135M block (forward recomputed), float32, batch 4 x seq 512, "
                    "input and all nine weight gradients",
        "timing": mode + " (median of reps)",
        "ms_per_call": round(t_s * 1e3, 4),
        "rep_ms": _pct(reps),
        "tokens_per_s": round(sb.batch * sb.seq / t_s, 1),
        "algorithmic_gflop": round(fl["total"] / 1e9, 3),
        "tflops": round(fl["total"] / t_s / 1e12, 2),
        "mfma_f32_frac": round(fl["total"] / t_s / 1e12 / F32_PEAK_TFLOPS, 4),
        "kernels": kern,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": dom_tf, "peak": F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tf / F32_PEAK_TFLOPS, 4),
                     "traffic": btraffic if dom == "bw_gemm" else None,
                     "traffic_source": (os.path.relpath(TRAFFIC_BACKWARD_PROFILE, ROOT)
                                        if dom == "bw_gemm" and btraffic is not None else None),
                     "note": "summed over the class's launches in one call (traffic: with its K-split reductions)"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the long-context and SmolLM3-shaped prefills")
    ap.add_argument("--other-only", action="store_true",
                    help="time only the long-context and SmolLM3-shaped prefills (a profiling aid; no headline)")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (outside the timed region): "
                         "a known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the whole forward on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from llama_decoder_only_amd import binding as B
    from llama_decoder_only_amd import synthetic as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    torch.cuda.set_device(0)

    s = S.workload("prefill_bf16")
    cfg = B.Config.from_shape(s)
    model = S.model_weights(s, 0)
    md = B.upload_model(model, dev)
    if args.other_only:
        if args.copy_check:  # the byte counters' calibration copy, outside the timed work
            src = torch.ones(args.copy_check << 18, dtype=torch.float32, device=dev)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        print(json.dumps(other_prefills(B, torch, dev, md)), flush=True)
        return
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(dev)
    logits = torch.empty(s.batch, s.seq, s.vocab, dtype=torch.bfloat16, device=dev)
    ws = B.workspace(cfg, B.SMOL_OP_PREFILL, s.batch, s.seq, dev)
    stream = torch.cuda.Stream()

    def step():
        B.smol_model_prefill(cfg, md, ids, logits, ws=ws, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()
    eager_ref = logits.clone()
    if args.copy_check:
        src = torch.ones(args.copy_check << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    eager_s = _time_steps(lambda: step(), args.steps, torch)
    graph_s = None
    mode = "eager"
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        for _ in range(3):  # every replay reproduces the eager result
            logits.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(logits, eager_ref):
                raise RuntimeError("graph replay differs from the eager result")
        graph_s = _time_steps(lambda: g.replay(), args.steps, torch)
        mode = "hip_graph"
    step_s = graph_s if graph_s is not None else eager_s
    rep_ms = _rep_ms((lambda: g.replay()) if graph_s is not None else step, args.steps, torch, stream)
    # the same steps cold: MALL and L2 flushed by a 512 MiB write before each (back to
    # back, as timed above, a prefill finds part of the 268 MB of weights still in MALL)
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    cold_ms = _rep_ms((lambda: g.replay()) if graph_s is not None else step, args.steps, torch, stream,
                      before=lambda: flush.fill_(1.0))
    del flush

    flops = prefill_flops(s)
    tokens = s.batch * s.seq
    value = tokens / step_s

    # per-kernel-class durations from dispatch events (eager step on the same stream)
    kern = {}
    with torch.cuda.stream(stream):
        for name in ("qkv_rope", "attention", "o_proj", "gate_up", "down", "lm_head", "embed"):
            ms, n = _kernel_time(B, name, step, torch)
            kern[name] = {"total_ms": ms, "launches": n, "avg_us": 1e3 * ms / max(n, 1)}
    dominant = dominant_class(kern, flops)
    avg_s = kern[dominant]["avg_us"] * 1e-6
    ach = flops["per_launch"][dominant] / avg_s / 1e12
    traffic = measured_traffic(dominant + "-traffic-bytes-per-launch")
    rooflines = prefill_rooflines(kern, flops)
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "traffic_source": os.path.relpath(TRAFFIC_PROFILE, ROOT) if traffic is not None else None,
                "algorithmic_flop_per_launch": flops["per_launch"][dominant],
                "avg_launch_us": round(kern[dominant]["avg_us"], 2)}

    out = {
        "metric": "prefill tokens/s (SmolLM2-135M fwd, bf16, 1 GPU) + % MFMA peak; decode HBM GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "dtype_note": "the arithmetic: float16 MFMA operands (activations rounded to float16; bf16 weights and "
                      "cache values converted to float16 exactly) with float32 accumulation, float32 residual "
                      "stream and statistics; weights, embedding, KV cache and logits stored as bf16",
        "data": "synthetic: seeded N(0, (1/24)^2) weights, unit RMSNorm weights, uniform token ids",
        "config": {"workload": "SmolLM2-135M-shaped prefill: 30 layers, hidden 576, 9/3 heads x 64, "
                               "intermediate 1536, vocab 49152 tied head; batch 4 x seq 512, bf16 logits",
                   "global_batch": s.batch, "seq_len": s.seq, "parallelism": "single GPU", "timing": mode},
        "mfma_frac": round(flops["total"] / step_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "algorithmic_gflop_per_step": round(flops["total"] / 1e9, 2),
        "eager_ms_per_step": round(eager_s * 1e3, 4),
        "rep_ms": _pct(rep_ms),
        "cold": {"ms_per_step": round(float(np.median(cold_ms)), 4),
                 "tokens_per_s": round(tokens / (float(np.median(cold_ms)) * 1e-3), 1),
                 "rep_ms": _pct(cold_ms), "how": "MALL/L2 flushed by a 512 MiB write before each step"},
        "roofline": roofline,
        "rooflines": rooflines,
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
    }
    _note("headline prefill done")

    if not args.no_other:
        out.update(other_prefills(B, torch, dev, md))

    if not args.no_decode:
        sd = S.workload("decode_bf16")
        P, cap = sd.cache_len, sd.cache_len + 1
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        kc = torch.randn(sd.n_layers, sd.batch, sd.n_kv_heads, cap, sd.head_dim, generator=gen, device=dev,
                         dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn(kc.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dids = torch.from_numpy(S.token_ids(sd, 0, S.T_DECODE_IDS)[:, 0].copy()).to(dev)
        cl = torch.full((sd.batch,), P, dtype=torch.int32, device=dev)
        dlog = torch.empty(sd.batch, sd.vocab, dtype=torch.bfloat16, device=dev)
        dws = B.workspace(cfg, B.SMOL_OP_DECODE, sd.batch, cap, dev)

        def dstep():
            B.smol_decode_step(cfg, md, dids, cl, kc, vc, dlog, ws=dws, stream=stream)

        with torch.cuda.stream(stream):
            for _ in range(3):
                dstep()
        torch.cuda.synchronize()
        dref = dlog.clone()
        dmode = "eager"
        dfn = dstep
        if not args.no_graph:
            dg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(dg, stream=stream):
                dstep()
            for _ in range(3):
                dlog.zero_()
                dg.replay()
                torch.cuda.synchronize()
                if not torch.equal(dlog, dref):
                    raise RuntimeError("decode graph replay differs from the eager result")
            dfn = dg.replay
            dmode = "hip_graph"
        # warm: steps back to back; cold (the headline): MALL and L2 flushed by a 512 MiB
        # write before each step
        warm_s = _time_steps(dfn, args.decode_steps, torch)
        flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        cold_ms = _rep_ms(dfn, args.decode_steps, torch, stream, before=lambda: flush.fill_(1.0))
        del flush
        d_s = float(np.median(cold_ms)) * 1e-3
        db = decode_bytes(sd, P)
        with torch.cuda.stream(stream):
            ms, n = _kernel_time(B, "decode_step", dstep, torch)
        step_kernel = "decode_step"
        per_launch = db["decode_step_per_launch"]
        if n == 0:  # the shape went to the multi-kernel path: its attention dominates
            step_kernel = "decode_attention"
            per_launch = db["decode_attention_per_launch"]
            with torch.cuda.stream(stream):
                ms, n = _kernel_time(B, "decode_attention", dstep, torch)
        att_s = ms / max(n, 1) * 1e-3
        att_gbps = per_launch / att_s / 1e9
        dtraffic = measured_traffic(step_kernel + "-traffic-bytes-per-launch", TRAFFIC_DECODE_PROFILE)
        dkern = {}
        with torch.cuda.stream(stream):
            for k in ("embed", "qkv_rope", "decode_attention", "decode_combine", "o_proj", "gate_up", "down",
                      "decode_step", "lm_head"):
                kms, kn = _kernel_time(B, k, dstep, torch)
                if kn:
                    dkern[k] = round(1e3 * kms / kn, 2)
        out["decode"] = {
            "workload": "decode step: batch 64, 2047 cached positions (+1 new), 30 layers, bf16",
            "timing": dmode + ", cold: MALL/L2 flushed by a 512 MiB write before each step (median)",
            "ms_per_step": round(d_s * 1e3, 4),
            "rep_ms_cold": _pct(cold_ms),
            "warm_ms_per_step": round(warm_s * 1e3, 4),
            "warm_hbm_gbps": round(db["total"] / warm_s / 1e9, 1),
            "tokens_per_s": round(sd.batch / d_s, 1),
            "algorithmic_gb_per_step": round(db["total"] / 1e9, 4),
            "hbm_gbps": round(db["total"] / d_s / 1e9, 1),
            "hbm_frac": round(db["total"] / d_s / 1e9 / HBM_PEAK_GBPS, 4),
            "roofline": {"bound": "hbm", "kernel": step_kernel, "achieved": round(att_gbps, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
                         "traffic": dtraffic,
                         "traffic_source": os.path.relpath(TRAFFIC_DECODE_PROFILE, ROOT) if dtraffic is not None else None,
                         "algorithmic_bytes_per_launch": per_launch,
                         "avg_launch_us": round(att_s * 1e6, 2)},
            "kernels_us": dkern,
        }
        # next-token choice on the decode step's logits [64, 49152] (smol_sample), and the
        # decode step + greedy choice captured together, timed cold like the step
        nxt = torch.empty(sd.batch, dtype=torch.int32, device=dev)
        uni = torch.rand(sd.batch, generator=gen, device=dev, dtype=torch.float32)
        samp = {}
        for label, (t, k, p) in (("greedy", (0.0, 0, 1.0)), ("t0.8_topk50_topp0.9", (0.8, 50, 0.9)),
                                 ("t1.0_topp0.9", (1.0, 0, 0.9))):
            with torch.cuda.stream(stream):
                ms, n = _kernel_time(B, "sample", lambda: [B.smol_sample(dlog, nxt, t, k, p, uni, stream=stream)
                                                           for _ in range(5)], torch)
            samp[label] = round(1e3 * ms / max(n, 1), 2)

        def gstep():
            dstep()
            B.smol_sample(dlog, nxt, 0.0, 0, 1.0, uni, stream=stream)

        gfn = gstep
        if not args.no_graph:
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg, stream=stream):
                gstep()
            gfn = gg.replay
        flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        gen_ms = _rep_ms(gfn, args.decode_steps, torch, stream, before=lambda: flush.fill_(1.0))
        del flush
        g_s = float(np.median(gen_ms)) * 1e-3
        out["generate"] = {
            "workload": "one greedy generation step at the decode workload: decode step + smol_sample",
            "ms_per_token_step": round(g_s * 1e3, 4),
            "tokens_per_s": round(sd.batch / g_s, 1),
            "sample_us": samp,
        }
        del kc, vc
        _note("decode done")

    if not args.no_backward:
        out["backward"] = backward_section(B, S, torch, dev, stream, args)
        _note("backward done")

    if not args.no_decode:
        out["ceilings"] = ceilings(torch, dev)

    if not args.no_cpu:
        _note("CPU oracle baseline (about 10-30 s)")
        out["cpu_baseline"] = cpu_baseline(s, model, ids_np)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
