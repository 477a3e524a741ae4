"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle on the
same seeded inputs. fp32: rel <= 1e-4 and bit-exact argmax; bf16: rel <= 2e-2,
where rel = max|gpu - oracle| / max|oracle| over the compared tensor."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import (TOL_BF16, TOL_F32, LazyCache, block_rows_oracle, ocfg, olayer,  # noqa: E402
                               omodel, rel, say, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _ids(s, seed=0):
    return torch.from_numpy(S.token_ids(s, seed)).to(DEV)


def _run_block(s, layer_dev, x_np, pos0=0, kc=None, vc=None):
    cfg = B.Config.from_shape(s)
    x = torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).to(DEV)
    out = torch.empty_like(x)
    B.smol_block_forward(cfg, layer_dev, x, out, pos0=pos0, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ one block


@pytest.mark.parametrize("name,batch,seq,jitter", [
    ("block_f32", 1, 128, 0.0),     # the single-block fp32 workload
    ("block_f32", 2, 100, 0.1),     # ragged tail (M = 200), non-unit norm weights
    ("block_f32", 3, 1, 0.1),       # one token
    ("block_f32", 1, 333, 0.0),     # several key tiles plus a ragged one
])
def test_block_f32(name, batch, seq, jitter):
    s = S.workload(name, batch=batch, seq=seq, norm_jitter=jitter)
    say(f"block f32 B={batch} T={seq}")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.data))
    want = O.block_forward(x.f64, olayer(layer), ocfg(s))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_F32


@pytest.mark.parametrize("batch,seq,jitter", [(2, 77, 0.1), (4, 512, 0.0)])
def test_block_bf16(batch, seq, jitter):
    s = S.workload("prefill_bf16", n_layers=1, batch=batch, seq=seq, norm_jitter=jitter)
    say(f"block bf16 B={batch} T={seq}")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.f64))
    want = O.block_forward(x.f64, olayer(layer), ocfg(s))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16


@pytest.mark.parametrize("dtype,hidden,heads,kv,inter,tol", [
    ("f32", 640, 10, 5, 1280, TOL_F32),     # generic hidden size (no unrolled RMSNorm), G = 2
    ("bf16", 640, 10, 5, 1280, TOL_BF16),
    ("f32", 512, 4, 1, 1024, TOL_F32),      # head_dim 128, G = 4
    ("bf16", 512, 4, 1, 1024, TOL_BF16),
])
def test_block_other_shapes(dtype, hidden, heads, kv, inter, tol):
    base = "block_f32" if dtype == "f32" else "prefill_bf16"
    s = S.workload(base, n_layers=1, batch=2, seq=150, hidden=hidden, n_heads=heads, n_kv_heads=kv,
                   head_dim=hidden // heads, intermediate=inter, norm_jitter=0.1)
    say(f"block {dtype} H={hidden} heads={heads}/{kv} d={hidden // heads}")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.f64))
    want = O.block_forward(x.f64, olayer(layer), ocfg(s))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= tol


def test_smollm3_shaped_two_layers_bf16():
    """The SmolLM3-3B shape (H 2048, 16/4 heads x 128, I 11008, vocab 128256, eps 1e-6) with 2 of its
    36 layers, batch 1 x seq 200, sampled logit rows against the oracle."""
    s = S.workload("smollm3_prefill_bf16", n_layers=2, batch=1, seq=200, norm_jitter=0.1)
    say("SmolLM3-shaped 2 layers bf16 B=1 T=200")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    got = _prefill(s, B.upload_model(model), torch.from_numpy(ids_np).to(DEV))
    rows = np.array([0, 1, 63, 64, 127, 128, 150, 199])
    want = O.model_prefill(ids_np, omodel(model), ocfg(s), logit_rows=rows)
    r = rel(to_np(got[0, torch.from_numpy(rows).to(DEV)]), want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16


def test_block_f32_with_cache_and_offset():
    """Chunked prefill: positions pos0.. with keys 0..pos0-1 already in the cache."""
    s = S.workload("block_f32", batch=2, seq=40, norm_jitter=0.1)
    pos0, cap = 70, 128
    say("block f32 with cache, pos0=70")
    layer = S.layer_weights(s, 0, 0)
    ld = B.upload_layer(layer)
    x = S.hidden_states(s, 0)
    past_k = np.random.default_rng(5).standard_normal((2, s.n_kv_heads, pos0, s.head_dim)).astype(np.float32)
    past_v = np.random.default_rng(6).standard_normal((2, s.n_kv_heads, pos0, s.head_dim)).astype(np.float32)
    kc = torch.zeros(2, s.n_kv_heads, cap, s.head_dim, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :pos0] = torch.from_numpy(past_k).to(DEV)
    vc[:, :, :pos0] = torch.from_numpy(past_v).to(DEV)
    got = to_np(_run_block(s, ld, x.data, pos0=pos0, kc=kc, vc=vc))
    cfg = ocfg(s)
    lw = olayer(layer)
    pos = np.arange(pos0, pos0 + s.seq)
    attn, k, v = O.attention_sublayer(x.f64, lw, cfg, pos, past_k, past_v, np.arange(pos0))
    h = x.f64 + attn
    want = h + O.mlp_sublayer(h, lw, cfg)
    assert rel(got, want) <= TOL_F32
    assert rel(to_np(kc[:, :, pos0:pos0 + s.seq]), k) <= TOL_F32
    assert rel(to_np(vc[:, :, pos0:pos0 + s.seq]), v) <= TOL_F32
    assert torch.all(kc[:, :, pos0 + s.seq:] == 0)


def test_block_f32_at_the_last_positions():
    """Positions 8092 .. 8191 (the end of max_pos) over a cache of 8092 random keys: the
    RoPE angles there are large (p * omega_0 ~ 8e3 rad), which float32 angle arithmetic
    gets wrong by ~1e-4 rad; the keys written to the cache and the block output must still
    match the oracle at 1e-4."""
    s = S.workload("block_f32", batch=2, seq=100, norm_jitter=0.1)
    pos0, cap = 8092, 8192
    say("block f32 with cache, pos0=8092")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    past_k = np.random.default_rng(7).standard_normal((2, s.n_kv_heads, pos0, s.head_dim)).astype(np.float32)
    past_v = np.random.default_rng(8).standard_normal((2, s.n_kv_heads, pos0, s.head_dim)).astype(np.float32)
    kc = torch.zeros(2, s.n_kv_heads, cap, s.head_dim, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :pos0] = torch.from_numpy(past_k).to(DEV)
    vc[:, :, :pos0] = torch.from_numpy(past_v).to(DEV)
    got = to_np(_run_block(s, B.upload_layer(layer), x.data, pos0=pos0, kc=kc, vc=vc))
    cfg, lw = ocfg(s), olayer(layer)
    attn, k, v = O.attention_sublayer(x.f64, lw, cfg, np.arange(pos0, cap), past_k, past_v, np.arange(pos0))
    h = x.f64 + attn
    want = h + O.mlp_sublayer(h, lw, cfg)
    rk, r = rel(to_np(kc[:, :, pos0:]), k), rel(got, want)
    say(f"cache k rel = {rk:.2e}, output rel = {r:.2e}")
    assert rk <= TOL_F32 and r <= TOL_F32


def test_gqa_equals_mha_with_repeated_kv():
    """9/3 heads equals 9/9 heads whose k/v projections repeat each kv head 3 times."""
    s = S.workload("block_f32", batch=2, seq=96)
    s9 = S.workload("block_f32", batch=2, seq=96, n_kv_heads=9)
    say("GQA vs MHA")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got3 = to_np(_run_block(s, B.upload_layer(layer), x.data))
    rep = lambda t: S.Tensor(np.repeat(t.data.reshape(3, 64, -1), 3, axis=0).reshape(576, -1).copy(), t.dtype)  # noqa
    l9 = S.Layer(**{n: getattr(layer, n) for n in S.Layer.NAMES})
    l9.wk, l9.wv = rep(layer.wk), rep(layer.wv)
    got9 = to_np(_run_block(s9, B.upload_layer(l9), x.data))
    assert rel(got3, got9) <= 1e-5


# ------------------------------------------------------------------ whole model


def _prefill(s, md, ids, kc=None, vc=None):
    cfg = B.Config.from_shape(s)
    logits = torch.empty(ids.shape[0], ids.shape[1], s.vocab, dtype=cfg.torch_dtype, device=DEV)
    B.smol_model_prefill(cfg, md, ids, logits, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    return logits


def test_model_f32_argmax_exact():
    """The 30-layer model in float32 (batch 1, seq 128): logits within 1e-4, argmax bit-exact."""
    s = S.workload("model_f32")
    say("model f32 30 layers B=1 T=128")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    got = to_np(_prefill(s, B.upload_model(model), torch.from_numpy(ids_np).to(DEV)))
    want = O.model_prefill(ids_np, omodel(model), ocfg(s))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_F32
    top2 = np.sort(want, axis=-1)[..., -2:]
    gap = top2[..., 1] - top2[..., 0]
    err = np.max(np.abs(got - want))
    close = gap <= 2 * err
    say(f"argmax near-ties (gap <= 2*max err): {int(close.sum())}")
    assert np.array_equal(np.argmax(got, -1)[~close], np.argmax(want, -1)[~close])
    assert np.array_equal(np.argmax(got, -1), np.argmax(want, -1))


@pytest.mark.parametrize("layers,batch,seq", [(3, 2, 130), (2, 1, 1)])
def test_model_bf16_small(layers, batch, seq):
    s = S.workload("prefill_bf16", n_layers=layers, batch=batch, seq=seq, norm_jitter=0.1)
    say(f"model bf16 L={layers} B={batch} T={seq}")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    got = to_np(_prefill(s, B.upload_model(model), torch.from_numpy(ids_np).to(DEV)))
    want = O.model_prefill(ids_np, omodel(model), ocfg(s))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16


def test_prefill_bf16_full_size_sampled():
    """The benchmarked prefill (30 layers, batch 4 x seq 512, bf16): sequence 0 against the oracle
    on 48 sampled rows; all four sequences are run in the launch configuration bench.py times."""
    s = S.workload("prefill_bf16")
    say("prefill bf16 B=4 T=512 full size")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    md = B.upload_model(model)
    got = _prefill(s, md, torch.from_numpy(ids_np).to(DEV))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 511], np.random.default_rng(0).integers(0, 512, 42)]))
    want = O.model_prefill(ids_np[:1], omodel(model), ocfg(s), logit_rows=rows)
    g = to_np(got[0, torch.from_numpy(rows).to(DEV)])
    r = rel(g, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16
    assert torch.isfinite(got.float()).all()


def test_long_block_bf16_sampled_rows():
    """One bf16 block at seq 8192: 40 sampled rows (every key tile of the last row) against the oracle."""
    s = S.workload("long_prefill_bf16", n_layers=1)
    say("block bf16 B=1 T=8192 sampled rows")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.f64))
    rows = np.unique(np.concatenate([[0, 63, 64, 4095, 8190, 8191], np.random.default_rng(1).integers(0, 8192, 34)]))
    want = block_rows_oracle(x.f64[0], olayer(layer), ocfg(s), rows)
    r = rel(got[0, rows], want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16


def test_block_long_sequences_f32_and_bf16():
    """Long single blocks: float32 at 1 x 2100 (the two-key-group attention over 66 query
    blocks; early, middle and last rows) at the float32 bar, and bf16 at 2 x 4100 (past
    4096 keys: 64-query blocks with two key groups; both sequences) at the bf16 bar."""
    s = S.workload("block_f32", batch=1, seq=2100, norm_jitter=0.1)
    say("block f32 B=1 T=2100")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.data))
    rows = np.unique(np.concatenate([[0, 31, 32, 1055, 1056, 1057, 2047, 2048, 2099],
                                     np.random.default_rng(3).integers(0, 2100, 23)]))
    want = block_rows_oracle(x.f64[0], olayer(layer), ocfg(s), rows)
    r = rel(got[0, rows], want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_F32
    s2 = S.workload("long_prefill_bf16", n_layers=1, batch=2, seq=4100, norm_jitter=0.1)
    say("block bf16 B=2 T=4100")
    layer2 = S.layer_weights(s2, 0, 0)
    x2 = S.hidden_states(s2, 0)
    got2 = to_np(_run_block(s2, B.upload_layer(layer2), x2.f64))
    rows2 = np.unique(np.concatenate([[0, 2047, 2048, 4095, 4096, 4099], np.random.default_rng(4).integers(0, 4100, 10)]))
    for b in range(2):
        want2 = block_rows_oracle(x2.f64[b], olayer(layer2), ocfg(s2), rows2)
        r2 = rel(got2[b, rows2], want2)
        say(f"sequence {b}: rel = {r2:.3e}")
        assert r2 <= TOL_BF16


def test_model_prefill_row_owned_head_ragged():
    """One block and the tied head at batch 2 x seq 4100 (M = 8200 rows, vocab 49152): the
    head's 9.4 MB of activations are more than one XCD's L2 keeps, so the lm_head runs
    256 x 256 tiles under row ownership (XCD 6 owns tiles 30..34 of 33), the last one ragged
    (8200 = 32 x 256 + 8). Every logit of sampled rows of both sequences, among them the eight
    rows of the ragged tile (sequence 1, positions 4092..4099), against the oracle."""
    s = S.workload("long_prefill_bf16", n_layers=1, batch=2, seq=4100, norm_jitter=0.1)
    say("model bf16 L=1 B=2 T=4100 (head over M = 8200)")
    model = S.model_weights(s, 0)
    ids_np = S.token_ids(s, 0)
    got = _prefill(s, B.upload_model(model), torch.from_numpy(ids_np).to(DEV))
    assert torch.isfinite(got.float()).all()
    rows = np.unique(np.concatenate([[0, 255, 256, 2047, 4091, 4092, 4095, 4096, 4099],
                                     np.random.default_rng(5).integers(0, 4100, 7)]))
    for b in range(2):
        want = O.model_prefill(ids_np[b:b + 1], omodel(model), ocfg(s), logit_rows=rows)
        r = rel(to_np(got[b, torch.from_numpy(rows).to(DEV)]), want)
        say(f"sequence {b}: rel = {r:.3e}")
        assert r <= TOL_BF16


def test_block_bf16_many_rows_last_tiles():
    """A bf16 block over M = 26 x 500 = 13000 rows: gate/up runs 256 x 256 tiles with each XCD
    owning a range of whole tiles, the last one ragged (13000 = 50 x 256 + 200). The last rows of
    the last sequence, and rows of a middle one, against the oracle."""
    s = S.workload("prefill_bf16", n_layers=1, batch=26, seq=500, norm_jitter=0.1)
    say("block bf16 B=26 T=500 (M = 13000)")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.f64))
    rows = np.r_[0:8, 240:260, 436:500]
    for b in (12, 25):
        want = block_rows_oracle(x.f64[b], olayer(layer), ocfg(s), rows)
        r = rel(got[b, rows], want)
        say(f"sequence {b}: rel = {r:.3e}")
        assert r <= TOL_BF16


def test_smollm3_block_full_size_sampled_rows():
    """One block of the SmolLM3-3B-shaped prefill at its full size (bf16, batch 2 x seq 4096, H
    2048, 16/4 heads x 128, I 11008): 24 sampled rows of each sequence (first and last key tiles
    among them) against the oracle's own steps."""
    s = S.workload("smollm3_prefill_bf16", n_layers=1, norm_jitter=0.1)
    say("SmolLM3-shaped block bf16 B=2 T=4096 sampled rows")
    layer = S.layer_weights(s, 0, 0)
    x = S.hidden_states(s, 0)
    got = to_np(_run_block(s, B.upload_layer(layer), x.f64))
    rows = np.unique(np.concatenate([[0, 127, 128, 2047, 4094, 4095], np.random.default_rng(5).integers(0, 4096, 18)]))
    for b in range(2):
        want = block_rows_oracle(x.f64[b], olayer(layer), ocfg(s), rows)
        r = rel(got[b, rows], want)
        say(f"sequence {b}: rel = {r:.3e}")
        assert r <= TOL_BF16


# ------------------------------------------------------------------ decode


def _decode(s, md, ids, cache_len, kc, vc):
    cfg = B.Config.from_shape(s)
    logits = torch.empty(ids.shape[0], s.vocab, dtype=cfg.torch_dtype, device=DEV)
    B.smol_decode_step(cfg, md, ids, cache_len, kc, vc, logits)
    torch.cuda.synchronize()
    return logits


def test_decode_f32_equals_prefill():
    """Decode at position P after a prefill of P tokens equals the prefill of P+1 tokens at P."""
    s = S.workload("model_f32", n_layers=3, batch=3, seq=51, norm_jitter=0.1)
    say("decode f32 vs prefill")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    ids_np = S.token_ids(s, 0)
    ids = torch.from_numpy(ids_np).to(DEV)
    P, cap = 50, 64
    kc = torch.zeros(s.n_layers, 3, s.n_kv_heads, cap, s.head_dim, device=DEV)
    vc = torch.zeros_like(kc)
    s_p = S.workload("model_f32", n_layers=3, batch=3, seq=P, norm_jitter=0.1)
    _prefill(s_p, md, ids[:, :P].contiguous(), kc, vc)
    cl = torch.full((3,), P, dtype=torch.int32, device=DEV)
    got = to_np(_decode(s, md, ids[:, P].contiguous(), cl, kc, vc))
    full = to_np(_prefill(s, md, ids))[:, P]
    assert rel(got, full) <= TOL_F32
    want = O.model_prefill(ids_np, omodel(model), ocfg(s))[:, P]
    assert rel(got, want) <= TOL_F32


def test_decode_bf16_full_size():
    """The benchmarked decode step: batch 64, 2047 cached positions (N(0,1) bf16), 30 layers."""
    s = S.workload("decode_bf16")
    say("decode bf16 B=64 P=2047 full size")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    P, cap = s.cache_len, 2048
    ks, vs = [], []
    kc = torch.empty(s.n_layers, s.batch, s.n_kv_heads, cap, s.head_dim, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for l in range(s.n_layers):
        k, v = S.kv_cache_values(s, 0, l, cap)
        ks.append(k)
        vs.append(v)
        kc[l] = B.to_device(k)
        vc[l] = B.to_device(v)
    ids_np = S.token_ids(s, 0, S.T_DECODE_IDS)[:, 0]
    ids = torch.from_numpy(ids_np.copy()).to(DEV)
    cl = torch.full((s.batch,), P, dtype=torch.int32, device=DEV)
    got = to_np(_decode(s, md, ids, cl, kc, vc))
    say("oracle decode")
    want, nk, nv = O.decode_step(ids_np, P, omodel(model), ocfg(s), LazyCache(ks, P), LazyCache(vs, P))
    r = rel(got, want)
    say(f"rel = {r:.3e}")
    assert r <= TOL_BF16
    for l in (0, 17, 29):
        assert rel(to_np(kc[l, :, :, P]), nk[l]) <= TOL_BF16
        assert rel(to_np(vc[l, :, :, P]), nv[l]) <= TOL_BF16
    assert torch.equal(kc[5, :, :, :P], B.to_device(ks[5])[:, :, :P])


def test_decode_bf16_ragged_lengths():
    """Batch 48 with a different cache length per sequence: around the 256-key split
    edges of the decode attention, at position 0, at the last slot of the cache, and
    one with no room left (NaN logits, no cache write). Each valid sequence against
    the oracle's decode of that sequence alone."""
    s = S.workload("decode_bf16", n_layers=2, batch=48)
    say("decode bf16 ragged cache lengths, B=48")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    cap = 600
    edge = [0, 1, 63, 64, 255, 256, 257, 300, 511, 512, 513, cap - 1]
    rng = np.random.default_rng(7)
    lens = edge + [int(x) for x in rng.integers(0, cap, size=s.batch - len(edge) - 1)] + [cap]
    ks, vs = [], []
    kc = torch.empty(s.n_layers, s.batch, s.n_kv_heads, cap, s.head_dim, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for l in range(s.n_layers):
        k, v = S.kv_cache_values(s, 0, l, cap)
        ks.append(k)
        vs.append(v)
        kc[l] = B.to_device(k)
        vc[l] = B.to_device(v)
    ids_np = S.token_ids(s, 0, S.T_DECODE_IDS)[:, 0]
    ids = torch.from_numpy(ids_np.copy()).to(DEV)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    got = to_np(_decode(s, md, ids, cl, kc, vc))
    om, oc = omodel(model), ocfg(s)
    worst = 0.0
    for b_, P in enumerate(lens[:-1]):
        kb = [k.f64[b_:b_ + 1, :, :P] for k in ks]
        vb = [v.f64[b_:b_ + 1, :, :P] for v in vs]
        want, nk, nv = O.decode_step(ids_np[b_:b_ + 1], P, om, oc, kb, vb)
        worst = max(worst, rel(got[b_:b_ + 1], want))
        assert rel(to_np(kc[1, b_, :, P]), nk[1][0]) <= TOL_BF16
    say(f"worst rel = {worst:.3e}")
    assert worst <= TOL_BF16
    assert np.isnan(got[-1]).all()
    assert torch.equal(kc[:, -1], torch.stack([B.to_device(k)[-1] for k in ks]))


@pytest.mark.parametrize("batch", [3, 48])
def test_decode_invalid_cache_len_gives_nan_and_no_write(batch):
    s = S.workload("model_f32", n_layers=2, batch=batch, seq=1)
    say(f"decode invalid cache_len, batch {batch}")
    md = B.upload_model(S.model_weights(s, 0))
    cap = 16
    kc = torch.zeros(2, batch, s.n_kv_heads, cap, s.head_dim, device=DEV)
    vc = torch.zeros_like(kc)
    cl = torch.full((batch,), 4, dtype=torch.int32, device=DEV)
    cl[1], cl[2] = cap, -1
    ids = torch.arange(1, batch + 1, dtype=torch.int32, device=DEV)
    out = _decode(s, md, ids, cl, kc, vc)
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[3:]).all()
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    assert torch.all(kc[:, 1:3] == 0) and torch.all(vc[:, 1:3] == 0)
    assert torch.any(kc[:, 0, :, 4] != 0)


def test_prefill_invalid_id_poisons_only_its_sequence():
    """An id outside [0, vocab) turns its sequence's logits NaN from that position on;
    the other sequences are bit-identical to a clean run."""
    s = S.workload("model_f32", n_layers=2, batch=2, seq=20)
    say("prefill invalid id")
    md = B.upload_model(S.model_weights(s, 0))
    ids = _ids(s)
    good = _prefill(s, md, ids)
    bad_ids = ids.clone()
    bad_ids[1, 5] = -3
    bad = _prefill(s, md, bad_ids)
    assert torch.equal(good[0], bad[0])
    assert torch.isnan(bad[1, 5:]).all()
