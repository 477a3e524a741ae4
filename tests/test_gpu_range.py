"""Large activations against the float16 range of the MFMA operands (bf16 models).

The bf16 path feeds its normalised activations to the MFMAs as float16 (65504 at
most). The deferred RMSNorm operand xs = w * x_new * r_old (stored at 2^-8) grows
with a row's rms growth over one residual update, which trained models can make
large in one block. These tests plant such a jump: a block whose o_proj weights are
scaled up 10^4 times (the row rms grows ~10^3-10^5 times in one update, measured on
the oracle), with a few rows that enter near 10^3, and compare with the float64
oracle at the bf16 bar (rel <= 2e-2, rel = max|gpu - oracle| / max|oracle|)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import TOL_BF16, ocfg, olayer, omodel, rel, say, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"
BIG_ROWS = (3, 40, 41, 100)  # token rows (of each sequence) that enter near 10^3
WO_SCALE = 1.0e4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _jump_layer(s, layer):
    """The layer with W_o scaled by WO_SCALE (rounded to bf16 again)."""
    layer.wo = S.stored(layer.wo.f64 * WO_SCALE, s.dtype)
    return layer


def _growth(x, lw, cfg):
    """Per-row rms growth of the residual stream over the attention update (oracle)."""
    _, parts = O.block_forward(x, lw, cfg, return_parts=True)
    h = x + parts["attn"]
    return np.sqrt(np.mean(h * h, -1)) / np.sqrt(np.mean(x * x, -1))


def test_block_bf16_norm_jump():
    s = S.workload("prefill_bf16", n_layers=1, batch=2, seq=160, norm_jitter=0.1)
    say("block bf16 B=2 T=160 with W_o x 1e4 and rows near 1e3")
    layer = _jump_layer(s, S.layer_weights(s, 0, 0))
    x = S.hidden_states(s, 0).f64 / 24.0  # rms ~ 1/24, the scale of an embedding row
    x[:, list(BIG_ROWS)] *= 2.4e4        # rows near 10^3
    x = S.stored(x, "f32").f64
    lw = olayer(layer)
    g = _growth(x, lw, ocfg(s))
    say(f"rms growth over the attention update: max {g.max():.3e}, median {np.median(g):.3e}")
    assert g.max() >= 1e3
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    out = torch.empty_like(xd)
    B.smol_block_forward(B.Config.from_shape(s), B.upload_layer(layer), xd, out)
    torch.cuda.synchronize()
    got = to_np(out)
    want = O.block_forward(x, lw, ocfg(s))
    assert np.isfinite(got).all()
    r = rel(got, want)
    # rows that entered small are judged on their own scale as well
    small = [t for t in range(s.seq) if t not in BIG_ROWS]
    r_small = rel(got[:, small], want[:, small])
    say(f"rel = {r:.3e}, rows that entered small: {r_small:.3e}")
    assert r <= TOL_BF16 and r_small <= TOL_BF16


def test_prefill_bf16_norm_jump_and_large_embedding_rows():
    """Two layers (the first with the scaled W_o), embedding rows of the ids at BIG_ROWS
    scaled to ~10^3; all logits against the oracle, the columns of the large rows and
    the ordinary columns judged separately (each on its own scale)."""
    s = S.workload("prefill_bf16", n_layers=2, batch=2, seq=160, norm_jitter=0.1)
    say("prefill bf16 2 layers B=2 T=160 with W_o x 1e4 and embedding rows near 1e3")
    model = S.model_weights(s, 0)
    ids = S.token_ids(s, 0)
    big_ids = sorted(set(int(ids[b, t]) for b in range(s.batch) for t in BIG_ROWS))
    E = model.embed.f64
    E[big_ids] *= 2.4e4
    model.embed = S.stored(E, s.dtype)
    model.layers[0] = _jump_layer(s, model.layers[0])
    om = omodel(model)
    g = _growth(O.embed(ids, om.embed), om.layers[0], ocfg(s))
    say(f"rms growth over layer 0's attention update: max {g.max():.3e}")
    assert g.max() >= 1e3
    cfg = B.Config.from_shape(s)
    logits = torch.empty(s.batch, s.seq, s.vocab, dtype=cfg.torch_dtype, device=DEV)
    B.smol_model_prefill(cfg, B.upload_model(model), torch.from_numpy(ids).to(DEV), logits)
    torch.cuda.synchronize()
    got = to_np(logits)
    want = O.model_prefill(ids, om, ocfg(s))
    assert np.isfinite(got).all()
    other = np.setdiff1d(np.arange(s.vocab), big_ids)
    r_big = rel(got[..., big_ids], want[..., big_ids])
    r_other = rel(got[..., other], want[..., other])
    say(f"rel: large-row columns {r_big:.3e}, other columns {r_other:.3e}")
    assert r_big <= TOL_BF16 and r_other <= TOL_BF16


def test_block_bf16_huge_attention_scores_stay_finite():
    """W_q and W_k scaled 1024 times: q and k stay inside float16 / bf16, but the scores
    reach ~10^5 in log2 units, where a bf16 rounding of the softmax's running reference
    max could miss the true max by ~10^3 and overflow exp2. The reference enters the
    score MFMAs as an exact three-part bf16 split, so every output stays finite; the
    float64 oracle's answer is reported (near-tied keys may pick differently under bf16
    q at this scale, so it is not held to the bar)."""
    s = S.workload("prefill_bf16", n_layers=1, batch=1, seq=192)
    say("block bf16 B=1 T=192 with W_q, W_k x 1024")
    layer = S.layer_weights(s, 0, 0)
    layer.wq = S.stored(layer.wq.f64 * 1024.0, s.dtype)
    layer.wk = S.stored(layer.wk.f64 * 1024.0, s.dtype)
    x = S.stored(S.hidden_states(s, 0).f64, "f32").f64
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    out = torch.empty_like(xd)
    B.smol_block_forward(B.Config.from_shape(s), B.upload_layer(layer), xd, out)
    torch.cuda.synchronize()
    got = to_np(out)
    assert np.isfinite(got).all()
    want = O.block_forward(x, olayer(layer), ocfg(s))
    say(f"finite; rel against the oracle {rel(got, want):.3e} (reported only)")
