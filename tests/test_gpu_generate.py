"""GPU parity of next-token choice (smol_sample) and of the generation loop
(smol_generate) against the float64 CPU oracle (oracle/generate.py).

Integer decisions are compared exactly. Where the oracle finds a decision within
1e-5 of its boundary (the top-p cut, or u against a CDF step) the GPU, which sums
in float32 and in another order, may land on either side: there the token must be
one that a boundary within 1e-5 allows (kept by the filter with top_p + 1e-3, and
u inside its CDF interval widened by 1e-5)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.generate as G  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import ocfg, omodel, say  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"
AMBIGUOUS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _logit_rows(dtype, B_, V, seed):
    """Seeded logits with the spread of a trained head (N(0, 2^2)) and planted ties:
    rows 0-7 repeat their maximum at other indices, row 8 is constant, rows 9-11
    hold -inf entries, row 12 has one dominant token."""
    rng = np.random.default_rng([seed, 7])
    x = rng.normal(0.0, 2.0, (B_, V))
    for r in range(8):
        m = x[r].max()
        x[r, rng.integers(0, V, 3 + r)] = m
    x[8] = 0.25
    for r in range(9, 12):
        x[r, rng.integers(0, V, V // 3)] = -np.inf
    if B_ > 12:
        x[12, 77] = 40.0
    if dtype == "bf16":
        bits = S.f32_to_bf16_bits(x.astype(np.float32))
        vals = S.bf16_bits_to_f32(bits).astype(np.float64)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        vals = x.astype(np.float32).astype(np.float64)
        t = torch.from_numpy(x.astype(np.float32)).to(DEV)
    return t, vals


SETTINGS = [  # temperature, top_k, top_p
    (0.0, 0, 1.0),
    (1.0, 0, 1.0),
    (0.7, 50, 1.0),
    (1.0, 0, 0.9),
    (0.8, 40, 0.95),
    (1.3, 1000, 0.5),
    (1.0, 1, 1.0),
    (2.0, 0, 0.3),
    (0.5, 49151, 0.999),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_matches_oracle(dtype):
    Bn, V = 64, 49152
    logits, vals = _logit_rows(dtype, Bn, V, 1 if dtype == "bf16" else 2)
    rng = np.random.default_rng([3, 1])
    exact = near = 0
    for t, k, p in SETTINGS:
        say(f"sample {dtype} T={t} top_k={k} top_p={p}")
        u = rng.random(Bn).astype(np.float32)
        out = torch.empty(Bn, dtype=torch.int32, device=DEV)
        B.smol_sample(logits, out, t, k, p, torch.from_numpy(u).to(DEV))
        got = out.cpu().numpy()
        for b in range(Bn):
            c = G.next_token(vals[b], t, k, p, float(u[b]))
            j = int(got[b])
            if min(c.p_margin, c.u_margin) >= AMBIGUOUS:
                assert j == c.token, (t, k, p, b, j, c.token)
                exact += 1
                continue
            near += 1
            if c.p_margin < AMBIGUOUS:  # the nucleus cut itself is within rounding
                wide = G.next_token(vals[b], t, k, min(1.0, p + 1e-3), float(u[b]))
                assert wide.kept[j], (t, k, p, b, j)
            else:  # u within rounding of a CDF step: j's interval must reach u
                w = np.where(c.kept, np.exp((vals[b] - vals[b].max()) / t), 0.0)
                cdf = np.cumsum(w / w.sum())
                lo = cdf[j - 1] if j > 0 else 0.0
                assert c.kept[j] and lo - AMBIGUOUS <= u[b] <= cdf[j] + AMBIGUOUS, (t, k, p, b, j, c.token)
    say(f"rows compared exactly: {exact}, within rounding of a boundary: {near}")
    assert exact >= len(SETTINGS) * Bn // 2


def test_sample_rows_of_a_prefill_and_determinism():
    """Rows addressed inside [B, T, V] logits (offset and stride) give what the same
    rows copied out give, and repeated calls give the same ids."""
    Bn, T, V = 4, 3, 49152
    logits, _ = _logit_rows("bf16", Bn * T, V, 5)
    full = logits.view(Bn, T, V)
    last = full[:, -1].contiguous()
    u = torch.from_numpy(np.random.default_rng(9).random(Bn).astype(np.float32)).to(DEV)
    a = torch.empty(Bn, dtype=torch.int32, device=DEV)
    b = torch.empty_like(a)
    for t, k, p in SETTINGS:
        B.smol_sample(full, a, t, k, p, u, row_offset=(T - 1) * V, row_stride=T * V)
        B.smol_sample(last, b, t, k, p, u)
        assert torch.equal(a, b)
        B.smol_sample(last, b, t, k, p, u)
        assert torch.equal(a, b)


def _tiny_shape(dtype="f32", batch=3, seq=10):
    return S.Shape(hidden=128, n_heads=2, n_kv_heads=1, head_dim=64, intermediate=256, n_layers=2, vocab=512,
                   max_pos=64, rms_eps=1e-5, rope_theta=100000.0, dtype=dtype, batch=batch, seq=seq, std=0.08,
                   workload_id=21, norm_jitter=0.1)


def _caches(s, cap, dtype):
    kc = torch.zeros(s.n_layers, s.batch, s.n_kv_heads, cap, s.head_dim, dtype=dtype, device=DEV)
    return kc, torch.zeros_like(kc)


def test_generate_greedy_equals_recompute():
    """Greedy generation with the cache (one prefill, then decode steps) against the
    oracle's full recompute of the growing sequence at every step, token by token,
    until a step whose top-two logit gap is too small for float32 to be sure."""
    s = _tiny_shape()
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    prompt = S.token_ids(s, 0)
    n_new, cap = 12, 32
    kc, vc = _caches(s, cap, torch.float32)
    out = torch.empty(n_new, s.batch, dtype=torch.int32, device=DEV)
    say("generate greedy f32 B=3 T=10 +12")
    B.smol_generate(B.Config.from_shape(s), md, torch.from_numpy(prompt).to(DEV), n_new, kc, vc, out)
    got = out.cpu().numpy()
    want, gaps = G.greedy_generate(prompt, n_new, omodel(model), ocfg(s))
    compared = 0
    for b in range(s.batch):
        for j in range(n_new):
            if gaps[j, b] < 1e-3:
                break
            assert got[j, b] == want[j, b], (b, j)
            compared += 1
    say(f"tokens compared: {compared} of {n_new * s.batch}")
    assert compared >= n_new * s.batch // 2


def test_generate_equals_stepwise_calls():
    """smol_generate's loop equals the same steps made one call at a time (prefill,
    sample of its last row, then decode step + sample), sampling with top-k and
    top-p: the same kernels in the same order give bit-identical ids."""
    s = S.workload("prefill_bf16", batch=4, seq=32)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    prompt = torch.from_numpy(S.token_ids(s, 0)).to(DEV)
    n_new, cap, t, k, p = 6, 48, 0.8, 50, 0.9
    u = torch.from_numpy(np.random.default_rng(11).random((n_new, s.batch)).astype(np.float32)).to(DEV)
    kc, vc = _caches(s, cap, torch.bfloat16)
    out = torch.empty(n_new, s.batch, dtype=torch.int32, device=DEV)
    say("generate bf16 B=4 T=32 +6 (loop)")
    B.smol_generate(cfg, md, prompt, n_new, kc, vc, out, t, k, p, u)
    kc2, vc2 = _caches(s, cap, torch.bfloat16)
    logits = torch.empty(s.batch, s.seq, s.vocab, dtype=torch.bfloat16, device=DEV)
    B.smol_model_prefill(cfg, md, prompt, logits, kc2, vc2)
    ids = torch.empty(n_new, s.batch, dtype=torch.int32, device=DEV)
    B.smol_sample(logits, ids[0], t, k, p, u[0], row_offset=(s.seq - 1) * s.vocab, row_stride=s.seq * s.vocab)
    step_logits = torch.empty(s.batch, s.vocab, dtype=torch.bfloat16, device=DEV)
    for j in range(1, n_new):
        cl = torch.full((s.batch,), s.seq + j - 1, dtype=torch.int32, device=DEV)
        B.smol_decode_step(cfg, md, ids[j - 1].contiguous(), cl, kc2, vc2, step_logits)
        B.smol_sample(step_logits, ids[j], t, k, p, u[j])
    torch.cuda.synchronize()
    assert torch.equal(out, ids)
    assert torch.equal(kc[:, :, :, : s.seq + n_new - 1], kc2[:, :, :, : s.seq + n_new - 1])


def test_generate_graph_replays():
    """The whole generation captured as one HIP graph: every replay (with eager work
    and synchronisations between them) reproduces the eager ids."""
    s = _tiny_shape("bf16", batch=2, seq=6)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    prompt = torch.from_numpy(S.token_ids(s, 0)).to(DEV)
    n_new, cap = 9, 16
    u = torch.from_numpy(np.random.default_rng(13).random((n_new, s.batch)).astype(np.float32)).to(DEV)
    kc, vc = _caches(s, cap, torch.bfloat16)
    ws = torch.empty(B.smol_generate_workspace_size(cfg, s.batch, s.seq, n_new, cap), dtype=torch.uint8, device=DEV)
    eager = torch.empty(n_new, s.batch, dtype=torch.int32, device=DEV)
    B.smol_generate(cfg, md, prompt, n_new, kc, vc, eager, 1.0, 20, 0.95, u, ws=ws)
    torch.cuda.synchronize()
    out = torch.full_like(eager, -7)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        B.smol_generate(cfg, md, prompt, n_new, kc, vc, out, 1.0, 20, 0.95, u, ws=ws, stream=stream)  # warm-up
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            B.smol_generate(cfg, md, prompt, n_new, kc, vc, out, 1.0, 20, 0.95, u, ws=ws, stream=stream)
    for r in range(3):
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        _ = (kc.float().sum() + 1).item()  # eager work between replays
