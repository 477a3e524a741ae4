"""GPU parity of chunked prefill (T > 1 on top of a filled cache), padding masks in
prefill and decode, and generation from right-padded prompts of different lengths,
against the float64 CPU oracle (oracle/smol.py, oracle/generate.py).

Chunked prefill is defined by absolute position: a chunk's query at position p sees
every key up to p, cached or new. A padding mask adds -inf to the masked keys'
scores (Sualeh77 model.py, "4. Attention", attention_mask); a query left with no
key comes out NaN on both sides."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.generate as G  # noqa: E402
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


def _caches(s, cap, dtype):
    kc = torch.zeros(s.n_layers, s.batch, s.n_kv_heads, cap, s.head_dim, dtype=dtype, device=DEV)
    return kc, torch.zeros_like(kc)


def _logits(s, T):
    return torch.empty(s.batch, T, s.vocab, dtype=torch.float32 if s.dtype == "f32" else torch.bfloat16, device=DEV)


@pytest.mark.parametrize("dtype,P", [("f32", 77), ("bf16", 64), ("f32", 1)])
def test_chunked_prefill(dtype, P):
    """Prefill of P tokens into the cache, then the remaining T - P tokens as one chunk
    at pos0 = P: the chunk's logits equal the one-shot prefill's at those positions
    (and the oracle's)."""
    name = "model_f32" if dtype == "f32" else "prefill_bf16"
    s = S.workload(name, n_layers=3, batch=2, seq=200, norm_jitter=0.1)
    say(f"chunked prefill {dtype} P={P} T=200")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    cap = 256
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kc, vc = _caches(s, cap, tdt)
    B.smol_model_prefill_ex(cfg, md, ids[:, :P].contiguous(), _logits(s, P), 0, None, kc, vc)
    chunk = _logits(s, 200 - P)
    B.smol_model_prefill_ex(cfg, md, ids[:, P:].contiguous(), chunk, P, None, kc, vc)
    kc1, vc1 = _caches(s, cap, tdt)
    whole = _logits(s, 200)
    B.smol_model_prefill(cfg, md, ids, whole, kc1, vc1)
    torch.cuda.synchronize()
    got, one = to_np(chunk), to_np(whole)[:, P:]
    want = O.model_prefill(ids_np, omodel(model), ocfg(s))[:, P:]
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    r1, r2 = rel(got, want), rel(got, one)
    say(f"rel vs oracle {r1:.2e}, vs one-shot {r2:.2e}")
    assert r1 <= tol and r2 <= tol
    # the chunk wrote the same cache entries the one-shot prefill did
    assert rel(to_np(kc[:, :, :, :200].float()), to_np(kc1[:, :, :, :200].float())) <= tol


def _mask(rng, B_, L, p_keep=0.8):
    m = rng.random((B_, L)) < p_keep
    m[:, 0] = True  # every query sees at least key 0
    return m


@pytest.mark.parametrize("dtype,seq", [("f32", 70), ("f32", 333), ("bf16", 150)])
def test_prefill_key_mask(dtype, seq):
    name = "model_f32" if dtype == "f32" else "prefill_bf16"
    s = S.workload(name, n_layers=2, batch=3, seq=seq, norm_jitter=0.1)
    say(f"masked prefill {dtype} T={seq}")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    mask = _mask(np.random.default_rng([seq, 5]), 3, seq)
    out = _logits(s, seq)
    B.smol_model_prefill_ex(cfg, md, torch.from_numpy(ids_np).to(DEV), out, 0,
                            torch.from_numpy(mask.astype(np.uint8)).to(DEV))
    torch.cuda.synchronize()
    got = to_np(out)
    want = O.model_prefill(ids_np, omodel(model), ocfg(s), key_mask=mask)
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert np.isfinite(got).all() and r <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_prefill_key_mask_with_cache_and_fully_masked_query():
    """One layer, a cache and a chunk: sequence 0's query at position 0 sees no key
    (NaN there, finite elsewhere in the sequence), and a masked key inside the cache
    is skipped by the chunk's queries."""
    s = S.workload("model_f32", n_layers=1, batch=2, seq=90, norm_jitter=0.1)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    cap, P = 128, 40
    mask = _mask(np.random.default_rng(3), 2, cap)
    mask[0, 0] = False
    mask[0, 1] = True
    km = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    kc, vc = _caches(s, cap, torch.float32)
    first, second = _logits(s, P), _logits(s, 90 - P)
    B.smol_model_prefill_ex(cfg, md, ids[:, :P].contiguous(), first, 0, km, kc, vc)
    B.smol_model_prefill_ex(cfg, md, ids[:, P:].contiguous(), second, P, km, kc, vc)
    torch.cuda.synchronize()
    got = np.concatenate([to_np(first), to_np(second)], axis=1)
    want = O.model_prefill(ids_np, omodel(model), ocfg(s), key_mask=mask[:, :90])
    assert np.isnan(got[0, 0]).all() and np.isnan(want[0, 0]).all()
    assert np.isfinite(got[0, 1:]).all() and np.isfinite(got[1]).all()
    ok = np.isfinite(want)
    assert rel(got[ok], want[ok]) <= TOL_F32


@pytest.mark.parametrize("dtype,batch", [("f32", 3), ("bf16", 3), ("f32", 48), ("bf16", 48)])
def test_decode_key_mask(dtype, batch):
    """At batch 3 and at batch 48 (144 sequence / kv-head pairs, near the benchmarked
    decode's 192), over 531 keys: two key chunks of the bf16 kernel (512 + 19), three of
    the float one (256 + 256 + 19)."""
    name = "model_f32" if dtype == "f32" else "prefill_bf16"
    s = S.workload(name, n_layers=2, batch=batch, seq=531, norm_jitter=0.1)
    say(f"masked decode {dtype}")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    P, cap = 530, 560  # keys 0 .. 530
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kc, vc = _caches(s, cap, tdt)
    B.smol_model_prefill_ex(cfg, md, ids[:, :P].contiguous(), _logits(s, P), 0, None, kc, vc)
    mask = _mask(np.random.default_rng(8), batch, cap, 0.6)
    out = torch.empty(batch, s.vocab, dtype=tdt, device=DEV)
    cl = torch.full((batch,), P, dtype=torch.int32, device=DEV)
    B.smol_decode_step_ex(cfg, md, ids[:, P].contiguous(), cl, kc, vc, out,
                          torch.from_numpy(mask.astype(np.uint8)).to(DEV))
    torch.cuda.synchronize()
    om = omodel(model)
    _, cache = O.model_prefill(ids_np[:, :P], om, ocfg(s), keep_cache=True)
    want, _, _ = O.decode_step(ids_np[:, P], P, om, ocfg(s), [c[0] for c in cache], [c[1] for c in cache],
                               key_mask=mask)
    got = to_np(out)
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    # no mask at all equals the all-ones mask
    out2 = torch.empty_like(out)
    B.smol_decode_step_ex(cfg, md, ids[:, P].contiguous(), cl, kc, vc, out2,
                          torch.ones(batch, cap, dtype=torch.uint8, device=DEV))
    out3 = torch.empty_like(out)
    B.smol_decode_step(cfg, md, ids[:, P].contiguous(), cl, kc, vc, out3)
    torch.cuda.synchronize()
    assert torch.equal(out2, out3)


def test_decode_window_skips_whole_chunk():
    """bf16 at head_dim 64 (512-key chunks), NoPE with a 100-key window on the second block,
    decode at P = 700: that block's first chunk (keys 0 .. 511) lies wholly before the window
    and contributes an empty partial, the second holds keys 512 .. 700. Against the oracle."""
    s = S.workload("prefill_bf16", n_layers=2, batch=3, seq=701, norm_jitter=0.1, no_rope_interval=2,
                   sliding_window=100)
    say("windowed decode bf16 P=700")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    P, cap = 700, 1024
    kc, vc = _caches(s, cap, torch.bfloat16)
    B.smol_model_prefill_ex(cfg, md, ids[:, :P].contiguous(), _logits(s, P), 0, None, kc, vc)
    out = torch.empty(3, s.vocab, dtype=torch.bfloat16, device=DEV)
    cl = torch.full((3,), P, dtype=torch.int32, device=DEV)
    B.smol_decode_step(cfg, md, ids[:, P].contiguous(), cl, kc, vc, out)
    torch.cuda.synchronize()
    om = omodel(model)
    _, cache = O.model_prefill(ids_np[:, :P], om, ocfg(s), keep_cache=True)
    want, _, _ = O.decode_step(ids_np[:, P], P, om, ocfg(s), [c[0] for c in cache], [c[1] for c in cache])
    r = rel(to_np(out), want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16


def test_generate_ragged_prompts():
    """Right-padded prompts of lengths 12, 7 and 3 (padding ids random): greedy tokens
    equal the oracle's full recompute of each sequence's own unpadded prompt."""
    s = S.Shape(hidden=128, n_heads=2, n_kv_heads=1, head_dim=64, intermediate=256, n_layers=2, vocab=512,
                max_pos=64, rms_eps=1e-5, rope_theta=100000.0, dtype="f32", batch=3, seq=12, std=0.08,
                workload_id=22, norm_jitter=0.1)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    prompt = S.token_ids(s, 0)
    lens = np.array([12, 7, 3], np.int32)
    n_new, cap = 10, 32
    kc, vc = _caches(s, cap, torch.float32)
    out = torch.empty(n_new, 3, dtype=torch.int32, device=DEV)
    say("generate ragged prompts f32")
    B.smol_generate(B.Config.from_shape(s), md, torch.from_numpy(prompt).to(DEV), n_new, kc, vc, out,
                    prompt_lens=torch.from_numpy(lens).to(DEV))
    got = out.cpu().numpy()
    compared = 0
    for b in range(3):
        want, gaps = G.greedy_generate(prompt[b:b + 1, :lens[b]], n_new, omodel(model), ocfg(s))
        for j in range(n_new):
            if gaps[j, 0] < 1e-3:
                break
            assert got[j, b] == want[j, 0], (b, j)
            compared += 1
    say(f"tokens compared: {compared} of {3 * n_new}")
    assert compared >= 15


def test_long_prefill_key_mask_and_window():
    """Keys past 4096 (the long-sequence attention configuration: 64-query blocks, two key
    groups) under a key mask and, on the second block, NoPE with a sliding window: bf16, 2
    layers, batch 1 x seq 4200 (a ragged last key tile), 192 logit rows against the oracle."""
    T = 4200
    s = S.workload("prefill_bf16", n_layers=2, batch=1, seq=T, norm_jitter=0.1, no_rope_interval=2,
                   sliding_window=1000)
    say(f"masked + windowed prefill bf16 T={T}")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cfg = B.Config.from_shape(s)
    ids_np = S.token_ids(s, 0)
    mask = _mask(np.random.default_rng([T, 7]), 1, T)
    out = _logits(s, T)
    B.smol_model_prefill_ex(cfg, md, torch.from_numpy(ids_np).to(DEV), out, 0,
                            torch.from_numpy(mask.astype(np.uint8)).to(DEV))
    torch.cuda.synchronize()
    rows = np.r_[0:64, T // 2:T // 2 + 64, T - 64:T]
    got = to_np(out)[0, rows]
    want = O.model_prefill(ids_np, omodel(model), ocfg(s), logit_rows=list(rows), key_mask=mask)
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert np.isfinite(got).all() and r <= TOL_BF16
