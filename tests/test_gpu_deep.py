"""Full-depth parity at full size, deep in the sequence: the long-context prefill
(SmolLM2-135M shape, 30 layers, batch 1 x seq 8192) and the SmolLM3-3B-shaped prefill
(36 layers, batch 2 x seq 4096, vocab 128256), run through the C ABI in the launch
configuration bench.py times, with the seeded weights of synthetic.py.

The oracle's residual stream after the last block at sampled rows comes from
tests/golden/make_deep_rows.py (float64 oracle, streamed block by block; rows up to
the last position); the test regenerates the same inputs, checks their fingerprints,
applies the oracle's head (O.lm_head: final RMSNorm and the tied embedding) to those
rows and compares every logit of them with the GPU's (rel <= 2e-2). The same runs
also check what holds at any size: finite logits, two runs bit-identical, tokens
changed after a position leave every earlier row (and the other sequence) bit-identical.
Progress lines go to stdout (run pytest with -s to see them as they happen)."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import TOL_BF16, ocfg, omodel, rel, say, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _golden(workload):
    return np.load(os.path.join(GOLDEN, f"deep_rows_{workload}.npz"), allow_pickle=False)


def _check_fingerprint(g, ids, embed, first, last):
    assert np.array_equal(g["fp_ids_head"], ids[0, :16]), "token ids differ from the stored run"
    assert np.array_equal(g["fp_embed_head"], embed.f64[:2, :4].ravel()), "embedding differs"
    assert np.array_equal(g["fp_w_q0_head"], first.wq.f64[0, :4]), "block 0 weights differ"
    assert np.array_equal(g["fp_w_down_last_head"], last.w_down.f64[-1, -4:]), "last block weights differ"


def _prefill(s, md, ids):
    cfg = B.Config.from_shape(s)
    logits = torch.empty(ids.shape[0], ids.shape[1], s.vocab, dtype=cfg.torch_dtype, device=DEV)
    B.smol_model_prefill(cfg, md, ids, logits)
    torch.cuda.synchronize()
    return logits


def _upload_streamed(s):
    """Draw the blocks in worker threads (numpy releases the GIL while drawing) and
    upload each as it is ready; host memory holds a few blocks at a time."""
    embed = S.normal(s, 0, 0, S.T_EMBED, (s.vocab, s.hidden), s.std)
    layers, first, last = [], None, None
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        for l, layer in enumerate(ex.map(lambda i: S.layer_weights(s, 0, i), range(s.n_layers))):
            layers.append(B.upload_layer(layer))
            if l == 0:
                first = layer
            last = layer
            if (l + 1) % 6 == 0:
                say(f"blocks drawn and uploaded: {l + 1}/{s.n_layers}")
    final = S.norm_weight(s, 0, 0, S.T_FINAL_NORM)
    md = B.ModelWeights(B.to_device(embed), layers, B.to_device(final))
    return md, embed, final, first, last


def _compare_rows(g, s, got_rows, embed, final):
    want = O.lm_head(g["x"], final.f64, embed.f64, ocfg(s))
    r = rel(got_rows, want)
    top = np.argsort(want, axis=1)[:, -2:]
    gap = want[np.arange(len(want)), top[:, 1]] - want[np.arange(len(want)), top[:, 0]]
    agree = int(np.sum(np.argmax(got_rows, 1) == top[:, 1]))
    say(f"rows {g['rows'].tolist()}: rel = {r:.3e}; argmax agrees on {agree}/{len(want)} "
        f"(smallest oracle top-2 gap {gap.min():.3e})")
    return r


def test_long_prefill_full_depth_deep_rows():
    """Batch 1 x seq 8192, 30 layers: rows 0 .. 8191 (4096, 6000 and the last among them)
    against the stored oracle rows; the first 96 rows against a live oracle run of that
    prefix; determinism and causality."""
    s = S.workload("long_prefill_bf16")
    say("long prefill bf16 B=1 T=8192, 30 layers: drawing the model")
    g = _golden("long_prefill_bf16")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    _check_fingerprint(g, ids_np, model.embed, model.layers[0], model.layers[-1])
    md = B.upload_model(model)
    ids = torch.from_numpy(ids_np).to(DEV)
    a = _prefill(s, md, ids)
    assert torch.isfinite(a.float()).all()
    rows = g["rows"]
    r = _compare_rows(g, s, to_np(a[0, torch.from_numpy(rows).to(DEV)]), model.embed, model.final_norm)
    assert r <= TOL_BF16
    b = _prefill(s, md, ids)
    assert torch.equal(a, b), "prefill is not deterministic"
    del b
    ids2 = ids.clone()
    ids2[:, 5001:] = (ids2[:, 5001:] + 7) % s.vocab
    c = _prefill(s, md, ids2)
    assert torch.equal(a[:, :5001], c[:, :5001]), "rows before the perturbation changed"
    assert not torch.equal(a[:, 5001:], c[:, 5001:])
    del c
    P = 96
    want = O.model_prefill(ids_np[:, :P], omodel(model), ocfg(s))
    rp = rel(to_np(a[:, :P]), want)
    say(f"prefix rows 0..95: rel = {rp:.3e}")
    assert rp <= TOL_BF16
    del a


@pytest.mark.timeout(900)
def test_smollm3_prefill_full_depth_deep_rows():
    """Batch 2 x seq 4096, 36 layers, vocab 128256, synthetic.py weights N(0, 0.02^2):
    sampled rows of sequence 0 (0, 127, 128, 2047, 4095 and five others) against the
    stored oracle rows, all 128256 logits of each; determinism; causality and batch
    independence."""
    s = S.workload("smollm3_prefill_bf16")
    say("SmolLM3-shaped prefill bf16 B=2 T=4096, 36 layers: drawing the model")
    g = _golden("smollm3_prefill_bf16")
    ids_np = S.token_ids(s, 0)
    md, embed, final, first, last = _upload_streamed(s)
    _check_fingerprint(g, ids_np, embed, first, last)
    ids = torch.from_numpy(ids_np).to(DEV)
    a = _prefill(s, md, ids)
    assert torch.isfinite(a.float()).all()
    rows = g["rows"]
    assert int(g["seq_idx"]) == 0
    r = _compare_rows(g, s, to_np(a[0, torch.from_numpy(rows).to(DEV)]), embed, final)
    assert r <= TOL_BF16
    b = _prefill(s, md, ids)
    assert torch.equal(a, b), "prefill is not deterministic"
    del b
    ids2 = ids.clone()
    ids2[0, 3001:] = (ids2[0, 3001:] + 11) % s.vocab
    c = _prefill(s, md, ids2)
    assert torch.equal(a[0, :3001], c[0, :3001]), "rows before the perturbation changed"
    assert torch.equal(a[1], c[1]), "the other sequence changed"
    assert not torch.equal(a[0, 3001:], c[0, 3001:])
    del a, c, md
