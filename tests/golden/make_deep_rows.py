"""Writes the CPU oracle's residual stream after the last block, at sampled rows of
two full-size prefills, for the GPU parity tests that compare logits deep in the
sequence at full depth (tests/test_gpu_deep.py).

    python tests/golden/make_deep_rows.py [long|smollm3|all]

* long:    the SmolLM2-135M-shaped prefill at batch 1 x seq 8192 (30 layers);
* smollm3: sequence 0 of the SmolLM3-3B-shaped prefill at batch 2 x seq 4096 (36
           layers, hidden 2048, 16/4 heads x 128, intermediate 11008, vocab 128256).

Only the oracle (oracle/smol.py, float64) and the seeded input generator
(llama_decoder_only_amd/synthetic.py) run here; nothing from the HIP path. The
blocks are streamed one at a time (the weights of one block are drawn, run through
O.block_forward at positions 0 .. T-1 with the block's index, and dropped), which is
the loop of O.model_prefill without holding every block in float64 at once. What is
stored: the rows, the residual stream x at those rows after the last block (the test
applies O.lm_head, the final norm and the tied head, with the regenerated embedding),
and fingerprints of the generated inputs (leading token ids and weight entries), so a
test can tell that it regenerated the same inputs.
"""

from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402

CASES = {
    # name: (workload, sequence index, rows)
    "long": ("long_prefill_bf16", 0,
             np.unique(np.concatenate([[0, 95, 96, 1000, 4095, 4096, 6000, 8190, 8191],
                                       np.random.default_rng(77).integers(0, 8192, 7)]))),
    "smollm3": ("smollm3_prefill_bf16", 0,
                np.unique(np.concatenate([[0, 127, 128, 2047, 4095],
                                          np.random.default_rng(78).integers(0, 4096, 5)]))),
}


def path_of(name: str) -> str:
    return os.path.join(HERE, f"deep_rows_{CASES[name][0]}.npz")


def oracle_config(s: S.Shape) -> O.Config:
    return O.Config(hidden=s.hidden, n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, intermediate=s.intermediate,
                    n_layers=s.n_layers, vocab=s.vocab, max_pos=s.max_pos, rms_eps=s.rms_eps,
                    rope_theta=s.rope_theta, no_rope_interval=s.no_rope_interval, sliding_window=s.sliding_window)


def fingerprint(s: S.Shape, ids: np.ndarray, first_layer: S.Layer, last_layer: S.Layer, embed: S.Tensor) -> dict:
    return {"ids_head": ids[0, :16].astype(np.int64), "embed_head": embed.f64[:2, :4].ravel(),
            "w_q0_head": first_layer.wq.f64[0, :4], "w_down_last_head": last_layer.w_down.f64[-1, -4:]}


def run(name: str) -> None:
    wname, seq_idx, rows = CASES[name]
    s = S.workload(wname)
    cfg = oracle_config(s)
    ids = S.token_ids(s, 0)
    t0 = time.time()
    embed = S.normal(s, 0, 0, S.T_EMBED, (s.vocab, s.hidden), s.std)
    x = O.embed(ids[seq_idx:seq_idx + 1], embed.f64)
    ex = ThreadPoolExecutor(1)  # draws block l + 1 while block l runs
    nxt = ex.submit(S.layer_weights, s, 0, 0)
    first = last = None
    for l in range(s.n_layers):
        layer = nxt.result()
        if l + 1 < s.n_layers:
            nxt = ex.submit(S.layer_weights, s, 0, l + 1)
        if l == 0:
            first = layer
        last = layer
        lw = O.LayerWeights(**{n: getattr(layer, n).f64 for n in S.Layer.NAMES})
        x = O.block_forward(x, lw, cfg, 0, layer=l)
        print(f"{name}: block {l + 1}/{s.n_layers} done, {time.time() - t0:.0f} s", flush=True)
    ex.shutdown()
    fp = fingerprint(s, ids, first, last, embed)
    np.savez(path_of(name), rows=rows, x=x[0, rows], seq_idx=np.int64(seq_idx), workload=np.array(wname),
             **{f"fp_{k}": v for k, v in fp.items()})
    print(f"wrote {path_of(name)} ({len(rows)} rows, {time.time() - t0:.0f} s)", flush=True)


if __name__ == "__main__":
    which = sys.argv[1] if len(sys.argv) > 1 else "all"
    for n in (CASES if which == "all" else [which]):
        run(n)
