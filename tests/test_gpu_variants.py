"""GPU parity of the SmolLM3 variants (nnterp "SmolLM3": NoPE blocks, rope_theta
5e6, a sliding window on the NoPE blocks) against the float64 CPU oracle.

A SmolLM3-like small shape: hidden 512, 4 query heads over 1 kv head of 128 (the
3B's group of 4), NoPE on every second block, theta 5e6, a window shorter than the
sequence, so the windowed blocks skip whole rounds of keys."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import TOL_BF16, TOL_F32, ocfg, omodel, rel, say, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _shape(dtype, seq, window, batch=2):
    return S.Shape(hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, intermediate=1024, n_layers=4, vocab=1024,
                   max_pos=4096, rms_eps=1e-6, rope_theta=5e6, dtype=dtype, batch=batch, seq=seq, std=0.04,
                   workload_id=31, norm_jitter=0.1, no_rope_interval=2, sliding_window=window)


@pytest.mark.parametrize("dtype,seq,window", [("f32", 200, 48), ("f32", 700, 100), ("bf16", 700, 100),
                                              ("f32", 1500, 300)])
def test_variants_prefill(dtype, seq, window):
    s = _shape(dtype, seq, window)
    say(f"SmolLM3 variants prefill {dtype} T={seq} W={window}")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    assert cfg.no_rope_interval == 2 and cfg.sliding_window == window
    ids_np = S.token_ids(s, 0)
    logits = torch.empty(s.batch, seq, s.vocab, dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                         device=DEV)
    B.smol_model_prefill(cfg, md, torch.from_numpy(ids_np).to(DEV), logits)
    torch.cuda.synchronize()
    got = to_np(logits)
    rows = np.arange(seq) if seq <= 700 else np.r_[0:64, seq // 2:seq // 2 + 64, seq - 64:seq]
    want = O.model_prefill(ids_np, omodel(model), ocfg(s), logit_rows=[b * seq + t for b in range(2) for t in rows])
    want = want.reshape(2, len(rows), s.vocab)
    r = rel(got[:, rows], want)
    say(f"rel = {r:.3e}")
    assert r <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    # the variants change the result (a check that the flags reach the kernels)
    plain = B.Config(**{**cfg.__dict__, "no_rope_interval": 0, "sliding_window": 0})
    B.smol_model_prefill(plain, md, torch.from_numpy(ids_np).to(DEV), logits)
    torch.cuda.synchronize()
    assert rel(to_np(logits)[:, rows], want) > 10 * (TOL_F32 if dtype == "f32" else TOL_BF16)


@pytest.mark.parametrize("dtype,batch", [("f32", 2), ("bf16", 2), ("bf16", 128)])
def test_variants_decode(dtype, batch):
    """Decode at P = 300 over a prefilled cache: the NoPE blocks see keys 201 .. 300
    only (window 100), in a cache of two 256-key chunks whose first is partly outside
    (batch 2, and batch 128 with its 128 sequence / kv-head pairs)."""
    s = _shape(dtype, 301, 100, batch=batch)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    P, cap = 300, 512
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kc = torch.zeros(s.n_layers, batch, s.n_kv_heads, cap, s.head_dim, dtype=tdt, device=DEV)
    vc = torch.zeros_like(kc)
    B.smol_model_prefill(cfg, md, ids[:, :P].contiguous(), torch.empty(batch, P, s.vocab, dtype=tdt, device=DEV), kc,
                         vc)
    out = torch.empty(batch, s.vocab, dtype=tdt, device=DEV)
    cl = torch.full((batch,), P, dtype=torch.int32, device=DEV)
    B.smol_decode_step(cfg, md, ids[:, P].contiguous(), cl, kc, vc, out)
    torch.cuda.synchronize()
    om = omodel(model)
    _, cache = O.model_prefill(ids_np[:, :P], om, ocfg(s), keep_cache=True)
    want, _, _ = O.decode_step(ids_np[:, P], P, om, ocfg(s), [c[0] for c in cache], [c[1] for c in cache])
    r = rel(to_np(out), want)
    say(f"decode rel = {r:.3e}")
    assert r <= (TOL_F32 if dtype == "f32" else TOL_BF16)
