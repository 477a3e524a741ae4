"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, an invariant, a special case, a library routine (torch's SDPA and
rms_norm, transformers' LlamaForCausalLM built offline from a config) or a
brute-force evaluation. They call the oracle through its module so that
tests/test_oracle_pins.py can plant mistakes into it and check that some pin
catches each one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.smol as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_cfg(**kw):
    base = dict(hidden=24, n_heads=6, n_kv_heads=2, intermediate=20, n_layers=2, vocab=37, max_pos=64,
                rms_eps=1e-5, rope_theta=100000.0)
    base.update(kw)
    return O.Config(**base)


def _rand_layer(cfg, rng, std=0.2, norm_jitter=0.0):
    H, I, d = cfg.hidden, cfg.intermediate, cfg.head_dim
    n = lambda *s: rng.standard_normal(s) * std  # noqa: E731
    nw = lambda: 1.0 + norm_jitter * rng.standard_normal(H)  # noqa: E731
    return O.LayerWeights(
        attn_norm=nw(), wq=n(cfg.n_heads * d, H), wk=n(cfg.n_kv_heads * d, H), wv=n(cfg.n_kv_heads * d, H),
        wo=n(H, cfg.n_heads * d), mlp_norm=nw(), w_gate=n(I, H), w_up=n(I, H), w_down=n(H, I))


def _rand_model(cfg, rng, std=0.2, norm_jitter=0.0):
    return O.ModelWeights(
        embed=rng.standard_normal((cfg.vocab, cfg.hidden)) * std,
        layers=[_rand_layer(cfg, rng, std, norm_jitter) for _ in range(cfg.n_layers)],
        final_norm=1.0 + norm_jitter * rng.standard_normal(cfg.hidden))


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ RMSNorm


def pin_rmsnorm_closed_forms():
    """Constant row c*1 -> c / sqrt(c^2 + eps) * w; one-hot s*e_k -> s / sqrt(s^2/H + eps)."""
    H, eps = 576, 1e-5
    w = _rng(1).standard_normal(H)
    for c in (0.0, 1e-3, 0.5, -3.0, 40.0):
        got = O.rms_norm(np.full((2, H), c), w, eps)
        want = c / math.sqrt(c * c + eps) * w
        assert np.allclose(got, want[None], rtol=1e-13, atol=1e-15), c
    for s in (1e-2, 2.0, -7.5):
        x = np.zeros(H)
        x[17] = s
        got = O.rms_norm(x, np.ones(H), eps)
        want = np.zeros(H)
        want[17] = s / math.sqrt(s * s / H + eps)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-15), s


def pin_rmsnorm_vs_torch():
    """torch.nn.functional.rms_norm (a library routine) in float64."""
    import torch

    x = _rng(2).standard_normal((5, 96)) * 3
    w = _rng(3).standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-5).numpy()
    assert _rel(O.rms_norm(x, w, 1e-5), want) < 1e-13


# ------------------------------------------------------------------ RoPE


def pin_inv_freq_closed_form():
    """omega_0 = 1, omega_{d/4} = theta^(-1/2), constant ratio omega_{i+1}/omega_i = theta^(-2/d)."""
    for d, theta in ((64, 1e5), (128, 1e5), (64, 1e4)):
        w = O.rope_inv_freq(d, theta)
        assert w.shape == (d // 2,)
        assert w[0] == 1.0
        assert abs(w[d // 4] - 1.0 / math.sqrt(theta)) < 1e-15
        ratio = w[1:] / w[:-1]
        assert np.allclose(ratio, theta ** (-2.0 / d), rtol=1e-12)
    # printed-by-hand values for theta = 1e5, d = 64: omega_1 = 10^(-5/32)
    w = O.rope_inv_freq(64, 1e5)
    assert abs(w[1] - 10 ** (-5.0 / 32.0)) < 1e-15


def pin_rope_complex_form():
    """(z_i + i z_{i+d/2}) * exp(i p omega_i) is the same rotation (a distinct formulation)."""
    d, theta = 64, 1e5
    z = _rng(4).standard_normal((3, 7, d))
    pos = np.array([0, 1, 5, 100, 2047, 4096, 8191])
    got = O.rope_rotate(z, pos, theta)
    zc = z[..., : d // 2] + 1j * z[..., d // 2:]
    omega = theta ** (-np.arange(d // 2) * 2.0 / d)
    rc = zc * np.exp(1j * pos[:, None] * omega[None, :])
    want = np.concatenate([rc.real, rc.imag], axis=-1)
    assert _rel(got, want) < 1e-12


def pin_rope_invariants():
    """Norm preservation, R_0 = I, <R_m q, R_n k> = <R_{m-n} q, k>, and the pairing e_0 -> e_{d/2}."""
    d, theta = 64, 1e5
    rng = _rng(5)
    z = rng.standard_normal((9, d))
    pos = np.array([0, 3, 17, 255, 256, 1000, 4095, 8190, 8191])
    r = O.rope_rotate(z, pos, theta)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(z, axis=-1), rtol=1e-13)
    assert np.array_equal(O.rope_rotate(z, np.zeros(9, int), theta), z)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in ((5, 2), (8191, 0), (8191, 8000), (300, 299), (7, 7)):
        lhs = O.rope_rotate(q[None], [m], theta)[0] @ O.rope_rotate(k[None], [n], theta)[0]
        rhs = O.rope_rotate(q[None], [m - n], theta)[0] @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs)), (m, n)
    e0 = np.zeros(d)
    e0[0] = 1.0
    p = 3
    r0 = O.rope_rotate(e0[None], [p], theta)[0]
    want = np.zeros(d)
    want[0], want[d // 2] = math.cos(p), math.sin(p)
    assert np.allclose(r0, want, atol=1e-15)


# ------------------------------------------------------------------ attention


def pin_attention_vs_sdpa():
    """GQA with kv head h // group equals torch SDPA on repeat_interleave-expanded K/V (float64)."""
    import torch

    rng = _rng(6)
    B, nq, nkv, T, d = 2, 9, 3, 23, 16
    q = rng.standard_normal((B, nq, T, d))
    k = rng.standard_normal((B, nkv, T, d))
    v = rng.standard_normal((B, nkv, T, d))
    got = O.gqa_attention(q, k, v, np.arange(T), np.arange(T))
    kt = torch.from_numpy(k).repeat_interleave(nq // nkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(nq // nkv, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=True).numpy()
    assert _rel(got, want) < 1e-12


def pin_attention_special_cases():
    """Position 0 returns v_0 exactly; equal keys give the running mean of the visible v;
    a single query at position P over keys 0..P is an unmasked softmax."""
    rng = _rng(7)
    B, nq, nkv, T, d = 1, 6, 2, 11, 8
    q = rng.standard_normal((B, nq, T, d))
    k = rng.standard_normal((B, nkv, T, d))
    v = rng.standard_normal((B, nkv, T, d))
    o = O.gqa_attention(q, k, v, np.arange(T), np.arange(T))
    for h in range(nq):
        assert np.array_equal(o[0, h, 0], v[0, h // 3, 0])
    keq = np.broadcast_to(k[:, :, :1], k.shape)
    o2 = O.gqa_attention(q, keq, v, np.arange(T), np.arange(T))
    run_mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    for h in range(nq):
        assert np.allclose(o2[0, h], run_mean[0, h // 3], rtol=1e-12, atol=1e-14)
    P = T - 1
    o3 = O.gqa_attention(q[:, :, P:], k, v, np.array([P]), np.arange(T))
    for h in range(nq):
        s = k[0, h // 3] @ q[0, h, P] / math.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(o3[0, h, 0], p @ v[0, h // 3], rtol=1e-12)


def pin_causality():
    """Perturbing tokens after t leaves the logits at positions <= t bit-identical."""
    cfg = _tiny_cfg()
    rng = _rng(8)
    mw = _rand_model(cfg, rng)
    ids = rng.integers(0, cfg.vocab, size=(2, 13))
    base = O.model_prefill(ids, mw, cfg)
    t = 6
    ids2 = ids.copy()
    ids2[:, t + 1:] = (ids2[:, t + 1:] + 5) % cfg.vocab
    pert = O.model_prefill(ids2, mw, cfg)
    assert np.array_equal(base[:, : t + 1], pert[:, : t + 1])
    assert not np.allclose(base[:, t + 1:], pert[:, t + 1:])


# ------------------------------------------------------------------ MLP


def pin_silu_values():
    """silu(0) = 0, silu(1) = 1/(1+e^-1), silu(-1) = -1/(1+e); silu(z) -> z for large z."""
    got = O.silu(np.array([0.0, 1.0, -1.0, 40.0, -40.0]))
    assert got[0] == 0.0
    assert abs(got[1] - 0.7310585786300049) < 1e-15
    assert abs(got[2] + 0.2689414213699951) < 1e-15
    assert abs(got[3] - 40.0) < 1e-12 and abs(got[4]) < 1e-15


def pin_swiglu_special_case():
    """With one-hot gate/up rows the MLP reduces to scalars: down[:, j] * silu(u_a) * u_b."""
    H, I = 8, 3
    u = _rng(9).standard_normal((4, H))
    wg = np.zeros((I, H))
    wu = np.zeros((I, H))
    wg[1, 2] = 1.0
    wu[1, 5] = 1.0
    wd = _rng(10).standard_normal((H, I))
    got = O.swiglu_mlp(u, wg, wu, wd)
    want = np.outer(u[:, 2] / (1 + np.exp(-u[:, 2])) * u[:, 5], wd[:, 1])
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ whole model


def _hf_model(cfg, mw):
    """transformers' LlamaForCausalLM from an in-memory config with our weights, float64, eager attention."""
    import torch
    from transformers import LlamaConfig, LlamaForCausalLM

    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, rms_norm_eps=cfg.rms_eps,
                     rope_theta=cfg.rope_theta, max_position_embeddings=cfg.max_pos, tie_word_embeddings=True,
                     attention_bias=False, mlp_bias=False, hidden_act="silu")
    hc._attn_implementation = "eager"
    torch.manual_seed(0)
    m = LlamaForCausalLM(hc).double().eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))  # noqa: E731
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(mw.embed))
        m.model.norm.weight.copy_(t(mw.final_norm))
        for lw, L in zip(mw.layers, m.model.layers):
            L.input_layernorm.weight.copy_(t(lw.attn_norm))
            L.post_attention_layernorm.weight.copy_(t(lw.mlp_norm))
            L.self_attn.q_proj.weight.copy_(t(lw.wq))
            L.self_attn.k_proj.weight.copy_(t(lw.wk))
            L.self_attn.v_proj.weight.copy_(t(lw.wv))
            L.self_attn.o_proj.weight.copy_(t(lw.wo))
            L.mlp.gate_proj.weight.copy_(t(lw.w_gate))
            L.mlp.up_proj.weight.copy_(t(lw.w_up))
            L.mlp.down_proj.weight.copy_(t(lw.w_down))
    assert m.lm_head.weight.data_ptr() == m.model.embed_tokens.weight.data_ptr()
    inv = m.model.rotary_emb.inv_freq.double().numpy()
    assert np.allclose(inv, cfg.rope_theta ** (-np.arange(cfg.head_dim // 2) * 2.0 / cfg.head_dim), rtol=1e-6)
    return m


def pin_model_vs_transformers():
    """Logits of the oracle equal transformers' Llama on the same weights (rotate_half RoPE,
    GQA by repeat, causal mask, pre-norm residuals, tied head). transformers builds the RoPE
    angles in float32, so agreement is to ~1e-6 relative, far below any structural mistake."""
    import torch

    cfg = _tiny_cfg(hidden=48, n_heads=6, n_kv_heads=2, intermediate=40, n_layers=2, vocab=53)
    rng = _rng(11)
    mw = _rand_model(cfg, rng, std=0.3, norm_jitter=0.2)
    ids = rng.integers(0, cfg.vocab, size=(2, 29))
    want = _hf_model(cfg, mw)(torch.from_numpy(ids)).logits.detach().numpy()
    got = O.model_prefill(ids, mw, cfg)
    assert got.shape == want.shape
    assert _rel(got, want) < 2e-6, _rel(got, want)


def pin_block_vs_transformers_smollm2_shape():
    """One SmolLM2-135M-shaped block (H 576, 9/3 heads, d 64, I 1536) at seq 128 equals
    transformers' decoder layer (taken as the model minus embedding and head)."""
    import torch

    cfg = O.Config(n_layers=1, vocab=64)
    rng = _rng(12)
    lw = _rand_layer(cfg, rng, std=1.0 / 24.0, norm_jitter=0.1)
    mw = O.ModelWeights(embed=rng.standard_normal((cfg.vocab, cfg.hidden)), layers=[lw],
                        final_norm=np.ones(cfg.hidden))
    m = _hf_model(cfg, mw)
    x = rng.standard_normal((1, 128, cfg.hidden))
    pos = torch.arange(128)[None]
    xt = torch.from_numpy(x)
    cos_sin = m.model.rotary_emb(xt, pos)
    mask = torch.full((128, 128), -torch.inf, dtype=torch.float64).triu(1)[None, None]
    out = m.model.layers[0](xt, attention_mask=mask, position_ids=pos, position_embeddings=cos_sin)
    want = (out[0] if isinstance(out, tuple) else out).detach().numpy()
    got = O.block_forward(x, lw, cfg)
    assert _rel(got, want) < 2e-6, _rel(got, want)


def pin_param_count():
    """134,515,008 parameters for the SmolLM2-135M shape with tied embeddings, as printed
    in abi96062 model.py; the fixture also carries the config the count is for."""
    with open(os.path.join(GOLDEN, "smollm2_135m.json")) as f:
        g = json.load(f)
    cfg = O.Config(hidden=g["hidden_size"], n_heads=g["num_attention_heads"], n_kv_heads=g["num_key_value_heads"],
                   intermediate=g["intermediate_size"], n_layers=g["num_hidden_layers"], vocab=g["vocab_size"],
                   max_pos=g["max_position_embeddings"], rms_eps=g["rms_norm_eps"], rope_theta=g["rope_theta"])
    assert cfg.head_dim == g["head_dim"]
    assert O.param_count(cfg, tied=True) == g["param_count"]
    assert O.param_count(cfg, tied=False) == g["param_count"] + g["vocab_size"] * g["hidden_size"]


def pin_logits_shape():
    """Input (1, 10) gives logits (1, 10, vocab) (abi96062 model.py __main__), here on a narrow model."""
    with open(os.path.join(GOLDEN, "smollm2_135m.json")) as f:
        g = json.load(f)
    cfg = _tiny_cfg(vocab=g["vocab_size"], n_layers=1)
    rng = _rng(13)
    mw = _rand_model(cfg, rng)
    ids = rng.integers(0, cfg.vocab, size=tuple(g["example_input_shape"]))
    out = O.model_prefill(ids, mw, cfg)
    assert list(out.shape) == g["example_logits_shape"][:2] + [cfg.vocab]
    assert cfg.vocab == g["example_logits_shape"][2]


def pin_gqa_mapping_smollm3():
    """The SmolLM3 page's mapping (query head h reads kv head h // 4) holds for 16/4 heads:
    editing kv head j changes exactly query heads 4j .. 4j+3."""
    with open(os.path.join(GOLDEN, "smollm3_3b_shape.json")) as f:
        g = json.load(f)
    nq, nkv = g["num_attention_heads"], g["num_key_value_heads"]
    rng = _rng(14)
    T, d = 5, 8
    q = rng.standard_normal((1, nq, T, d))
    k = rng.standard_normal((1, nkv, T, d))
    v = rng.standard_normal((1, nkv, T, d))
    base = O.gqa_attention(q, k, v, np.arange(T), np.arange(T))
    for j in range(nkv):
        v2 = v.copy()
        v2[0, j] += 1.0
        out = O.gqa_attention(q, k, v2, np.arange(T), np.arange(T))
        changed = [h for h in range(nq) if not np.array_equal(out[0, h], base[0, h])]
        assert changed == [h for h in range(nq) if g["gqa_head_to_kv"][h] == j]


def pin_decode_equals_prefill():
    """Decode at position P over a cache from prefill(ids[:P]) equals prefill(ids[:P+1]) at P."""
    cfg = _tiny_cfg()
    rng = _rng(15)
    mw = _rand_model(cfg, rng)
    B, P = 3, 9
    ids = rng.integers(0, cfg.vocab, size=(B, P + 1))
    full = O.model_prefill(ids, mw, cfg)
    _, cache = O.model_prefill(ids[:, :P], mw, cfg, keep_cache=True)
    kc = [c[0] for c in cache]
    vc = [c[1] for c in cache]
    logits, nk, nv = O.decode_step(ids[:, P], P, mw, cfg, kc, vc)
    assert _rel(logits, full[:, P]) < 1e-12
    _, cache_full = O.model_prefill(ids, mw, cfg, keep_cache=True)
    for li in range(cfg.n_layers):
        assert np.allclose(nk[li], cache_full[li][0][:, :, P], rtol=1e-12)
        assert np.allclose(nv[li], cache_full[li][1][:, :, P], rtol=1e-12)


def _brute_force_logits(cfg, mw, ids, mask=None):  # noqa: C901
    """Scalar pure-Python evaluation of the whole forward (for tiny sizes only).
    mask[b][j] False: key j of sequence b gets weight 0 (its value still enters the
    sum times 0, as in probs @ v); a query with no unmasked key gets NaN."""
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    G = nq // nkv
    B, T = len(ids), len(ids[0])

    def norm(row, w):
        ms = sum(v * v for v in row) / H
        r = 1.0 / math.sqrt(ms + cfg.rms_eps)
        return [w[i] * row[i] * r for i in range(H)]

    def lin(row, W):
        return [sum(W[o][i] * row[i] for i in range(len(row))) for o in range(len(W))]

    def rot(vec, p):
        out = list(vec)
        for i in range(d // 2):
            a = p * cfg.rope_theta ** (-2.0 * i / d)
            c, s = math.cos(a), math.sin(a)
            out[i] = vec[i] * c - vec[i + d // 2] * s
            out[i + d // 2] = vec[i + d // 2] * c + vec[i] * s
        return out

    E = mw.embed.tolist()
    logits = []
    rope_every = getattr(cfg, "no_rope_interval", 0)
    win = getattr(cfg, "sliding_window", 0)
    for b in range(B):
        xs = [list(E[ids[b][t]]) for t in range(T)]
        for li, lw in enumerate(mw.layers):
            nope = rope_every > 0 and (li + 1) % rope_every == 0  # blocks rope_every-1, 2 rope_every-1, ...
            w_l = win if (nope and win > 0) else 0
            W = {n: getattr(lw, n).tolist() for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
            us = [norm(x, lw.attn_norm.tolist()) for x in xs]
            qs = [lin(u, W["wq"]) for u in us]
            ks = [lin(u, W["wk"]) for u in us]
            vs = [lin(u, W["wv"]) for u in us]
            for t in range(T):
                att = [0.0] * (nq * d)
                for h in range(nq):
                    g = h // G
                    qh = qs[t][h * d:(h + 1) * d] if nope else rot(qs[t][h * d:(h + 1) * d], t)
                    seen = [j for j in range(t + 1) if (mask is None or mask[b][j]) and (w_l == 0 or j > t - w_l)]
                    if not seen:
                        for e in range(d):
                            att[h * d + e] = float("nan")
                        continue
                    sc = {}
                    for j in seen:
                        kj = ks[j][g * d:(g + 1) * d] if nope else rot(ks[j][g * d:(g + 1) * d], j)
                        sc[j] = sum(qh[e] * kj[e] for e in range(d)) / math.sqrt(d)
                    mx = max(sc.values())
                    ex = {j: math.exp(s - mx) for j, s in sc.items()}
                    z = sum(ex.values())
                    for e in range(d):
                        att[h * d + e] = sum((ex[j] / z if j in ex else 0.0) * vs[j][g * d + e] for j in range(t + 1))
                xs[t] = [xs[t][i] + o for i, o in enumerate(lin(att, W["wo"]))]
            for t in range(T):
                w = norm(xs[t], lw.mlp_norm.tolist())
                gt = lin(w, W["w_gate"])
                up = lin(w, W["w_up"])
                y = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
                xs[t] = [xs[t][i] + o for i, o in enumerate(lin(y, W["w_down"]))]
        for t in range(T):
            z = norm(xs[t], mw.final_norm.tolist())
            logits.append([sum(E[v][i] * z[i] for i in range(H)) for v in range(cfg.vocab)])
    return np.array(logits).reshape(B, T, cfg.vocab)


def pin_brute_force_tiny():
    """numpy oracle vs a scalar pure-Python evaluation: H 12, 3 q heads / 1 kv head, d 4,
    I 8, 2 layers, vocab 16, T 5."""
    cfg = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                   rms_eps=1e-5, rope_theta=1e5)
    rng = _rng(16)
    mw = _rand_model(cfg, rng, std=0.5, norm_jitter=0.3)
    ids = rng.integers(0, cfg.vocab, size=(2, 5))
    want = _brute_force_logits(cfg, mw, ids.tolist())
    got = O.model_prefill(ids, mw, cfg)
    assert _rel(got, want) < 1e-12


def pin_padding_mask():
    """The pages' attention_mask adds 0 / -inf per key (Sualeh77 model.py, "4.
    Attention"): an all-True mask changes nothing; a scalar evaluation with masked
    keys agrees (a query whose every key is masked comes out NaN in both); a masked
    token's embedding cannot reach any other position's logits; masking keys is not
    masking queries."""
    cfg = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                   rms_eps=1e-5, rope_theta=1e5)
    rng = _rng(41)
    mw = _rand_model(cfg, rng, std=0.5, norm_jitter=0.3)
    ids = rng.integers(0, cfg.vocab, size=(2, 6))
    full = np.ones((2, 6), bool)
    assert np.array_equal(O.model_prefill(ids, mw, cfg, key_mask=full), O.model_prefill(ids, mw, cfg))
    mask = np.array([[True, False, True, False, True, True], [True, True, False, True, False, True]])
    want = _brute_force_logits(cfg, mw, ids.tolist(), mask.tolist())
    got = O.model_prefill(ids, mw, cfg, key_mask=mask)
    assert np.isfinite(got).all() and _rel(got, want) < 1e-12
    # a query with every key masked: NaN at that position of the block's output only
    x = O.embed(ids, mw.embed)
    none0 = mask.copy()
    none0[0, :2] = [False, True]  # query 0 of sequence 0 sees no key; query 1 sees key 1
    out = O.block_forward(x, mw.layers[0], cfg, key_mask=none0)
    assert np.isnan(out[0, 0]).all() and np.isfinite(out[0, 1:]).all() and np.isfinite(out[1]).all()
    bf = _brute_force_logits(cfg, O.ModelWeights(mw.embed, mw.layers[:1], mw.final_norm), ids.tolist(), none0.tolist())
    assert np.isnan(bf[0, 0]).all() and np.isfinite(bf[0, 1:]).all()
    ids2 = ids.copy()
    ids2[0, 3] = (ids2[0, 3] + 5) % cfg.vocab  # a masked token of sequence 0
    got2 = O.model_prefill(ids2, mw, cfg, key_mask=mask)
    keep = [t for t in range(6) if t != 3]
    a, b_ = got[0, keep], got2[0, keep]
    assert np.array_equal(np.isnan(a), np.isnan(b_)) and np.array_equal(a[~np.isnan(a)], b_[~np.isnan(b_)])


def pin_nope_blocks_and_window():
    """SmolLM3 variants (nnterp SmolLM3, "NoPE blocks" and the sliding-window
    section): every 4th block is NoPE, which on 36 blocks gives the page's list 3, 7,
    ..., 35; a NoPE block's queries and keys are the bare projections, so its output
    does not move when the whole sequence shifts position; a window at least the
    sequence long changes nothing; a window of 1 leaves each query its own value; and
    a scalar evaluation with a NoPE block and a window agrees. (A rotary block is
    shift-invariant too, since its scores depend on position offsets only; what tells
    the two apart is that its keys differ from the projections past position 0.)"""
    cfg4 = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=36, vocab=16, max_pos=256,
                    rms_eps=1e-5, rope_theta=5e6, no_rope_interval=4)
    assert [l for l in range(36) if not cfg4.rope_on(l)] == [3, 7, 11, 15, 19, 23, 27, 31, 35]
    rng = _rng(43)
    cfg1 = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=1, vocab=16, max_pos=256,
                    rms_eps=1e-5, rope_theta=5e6, no_rope_interval=1)
    lw = _rand_layer(cfg1, rng, std=0.5, norm_jitter=0.3)
    x = rng.normal(0, 1, (2, 7, 12))
    a = O.block_forward(x, lw, cfg1, pos0=0)
    assert np.array_equal(a, O.block_forward(x, lw, cfg1, pos0=123))
    _, parts = O.block_forward(x, lw, cfg1, return_parts=True)
    u = O.rms_norm(x, lw.attn_norm, cfg1.rms_eps)
    raw_k = (u @ lw.wk.T).reshape(2, 7, 1, 4).transpose(0, 2, 1, 3)
    assert np.array_equal(parts["k"], raw_k)
    rope = O.Config(**{**cfg1.__dict__, "no_rope_interval": 0})  # a rotary block rotates them
    _, parts_r = O.block_forward(x, lw, rope, return_parts=True)
    assert np.array_equal(parts_r["k"][:, :, 0], raw_k[:, :, 0]) and not np.allclose(parts_r["k"][:, :, 1:], raw_k[:, :, 1:])
    wide = O.Config(**{**cfg1.__dict__, "sliding_window": 7})
    assert np.array_equal(O.block_forward(x, lw, wide), a)
    one = O.Config(**{**cfg1.__dict__, "sliding_window": 1})
    attn, k, v = O.attention_sublayer(x, lw, one, np.arange(7))
    want = np.repeat(v, 3, axis=1).transpose(0, 2, 1, 3).reshape(2, 7, 12) @ lw.wo.T
    assert _rel(attn, want) < 1e-12
    cfg2 = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                    rms_eps=1e-5, rope_theta=5e6, no_rope_interval=2, sliding_window=2)
    mw = _rand_model(cfg2, rng, std=0.5, norm_jitter=0.3)
    ids = rng.integers(0, cfg2.vocab, size=(2, 6))
    assert _rel(O.model_prefill(ids, mw, cfg2), _brute_force_logits(cfg2, mw, ids.tolist())) < 1e-12


# ---------------------------------------------------------------- next-token choice
# (oracle/generate.py; Sualeh77 model.py "7. Top-level", generate; abi96062 model.py,
# SmolLM2Model.generate)

import oracle.generate as G  # noqa: E402


def _kept(logits, t=1.0, k=0, p=1.0):
    return set(np.nonzero(G.next_token(np.asarray(logits, np.float64), t, k, p, 0.5).kept)[0].tolist())


def pin_greedy_ties_and_nan():
    """Greedy is the argmax, lowest index among equal maxima; NaN rows give -1."""
    assert G.next_token([1.0, 3.0, 3.0, 2.0], 0.0).token == 1
    assert G.next_token([-np.inf, np.inf, np.inf], 0.0).token == 1
    assert G.next_token([0.0, np.nan, 1.0], 0.0).token == -1
    assert G.next_token([0.0, np.nan, 1.0], 1.0, u=0.3).token == -1
    assert G.next_token([0.0, np.inf, 1.0], 1.0, u=0.3).token == -1  # softmax undefined


def pin_top_k_keeps_ties():
    """Tokens below the k-th largest logit go; ties with it stay."""
    l = [5.0, 4.0, 4.0, 1.0, 0.0]
    assert _kept(l, k=1) == {0}
    assert _kept(l, k=2) == {0, 1, 2}
    assert _kept(l, k=3) == {0, 1, 2}
    assert _kept(l, k=4) == {0, 1, 2, 3}
    assert _kept(l, k=0) == _kept(l, k=5) == {0, 1, 2, 3, 4}


def pin_top_p_hand_values():
    """Probabilities 0.5, 0.3, 0.2 (cumulative 0.5, 0.8, 1.0): the nucleus keeps every
    token up to and including the first whose cumulative probability exceeds p,
    whatever the tokens' order in the vocabulary; equal logits rank by index."""
    lp = np.log([0.5, 0.3, 0.2])
    assert _kept(lp, p=0.45) == {0}
    assert _kept(lp, p=0.6) == {0, 1}
    assert _kept(lp, p=0.9) == {0, 1, 2}
    perm = np.log([0.2, 0.5, 0.3])  # same distribution, other token order
    assert _kept(perm, p=0.6) == {1, 2}
    # logits 1, 2, 2, 0: probabilities e^2/Z twice (0.3995 each), e/Z, 1/Z
    tie = [1.0, 2.0, 2.0, 0.0]
    assert _kept(tie, p=0.3) == {1}
    assert _kept(tie, p=0.5) == {1, 2}
    assert _kept(tie, p=0.85) == {0, 1, 2}


def pin_top_p_after_top_k():
    """Top-p works on the distribution that top-k left (renormalised): probabilities
    0.4, 0.3, 0.2, 0.1 with k = 2 become 4/7, 3/7, so p = 0.5 keeps one token; without
    top-k (cumulative 0.4, 0.7) the same p keeps two."""
    lp = np.log([0.4, 0.3, 0.2, 0.1])
    assert _kept(lp, k=2, p=0.5) == {0}
    assert _kept(lp, p=0.5) == {0, 1}


def pin_inverse_cdf_stratified():
    """With stratified uniforms u_i = (i + 1/2) / N the draw counts are N times the
    probabilities exactly: 0.1, 0.2, 0.3, 0.4 at temperature 1, and p^2 / sum p^2
    (= 1/30, 4/30, 9/30, 16/30) at temperature 1/2."""
    lp = np.log([0.1, 0.2, 0.3, 0.4])
    for t, n, want in ((1.0, 1000, [100, 200, 300, 400]), (0.5, 300, [10, 40, 90, 160])):
        counts = np.zeros(4, int)
        for i in range(n):
            counts[G.next_token(lp, t, u=(i + 0.5) / n).token] += 1
        assert counts.tolist() == want, (t, counts)


def pin_inverse_cdf_steps():
    """The draw is the first index whose cumulative probability exceeds u: with two
    equal probabilities u = 0.5 picks index 1, u = 0 the first kept index and u just
    below 1 the last kept index."""
    assert G.next_token([0.0, 0.0], 1.0, u=0.5).token == 1
    assert G.next_token([0.0, 0.0], 1.0, u=0.0).token == 0
    l = [0.0, -np.inf, 3.0, 1.0, -np.inf]
    assert G.next_token(l, 1.0, u=0.0).token == 0
    assert G.next_token(l, 1.0, u=1.0 - 1e-12).token == 3
    assert G.next_token(l, 1.0, top_k=1, u=0.0).token == 2


def _brute_choice(l, t, k, p, u):
    """The same choice by enumeration: sorted order by explicit comparisons, the
    nucleus as the shortest sorted prefix whose mass exceeds p, the draw by a running
    sum. Tiny V only."""
    V = len(l)
    order = sorted(range(V), key=lambda i: (-l[i], i))
    kept = set(range(V))
    if 0 < k < V:
        kth = order[k - 1]
        kept = {i for i in range(V) if l[i] >= l[kth]}
    w = {i: math.exp((l[i] - max(l)) / t) for i in kept}
    if p < 1.0:
        ranked = [i for i in order if i in kept]
        z = sum(w[i] for i in ranked)
        for n in range(1, len(ranked) + 1):
            if sum(w[i] for i in ranked[:n]) / z > p:
                break
        kept = set(ranked[:n])
    z = sum(w[i] for i in kept)
    acc = 0.0
    for i in range(V):
        if i in kept:
            acc += w[i] / z
            if acc > u:
                return i
    return max(kept)


def pin_choice_brute_force():
    rng = _rng(31)
    for trial in range(300):
        V = int(rng.integers(2, 7))
        l = np.round(rng.normal(0, 1.5, V), 1)  # rounding makes ties common
        t = float(rng.choice([0.3, 1.0, 2.5]))
        k = int(rng.integers(0, V + 1))
        p = float(rng.choice([1.0, 0.95, 0.7, 0.35]))
        u = float(rng.random())
        c = G.next_token(l, t, k, p, u)
        if min(c.p_margin, c.u_margin) < 1e-9:
            continue  # a cut within rounding of a boundary: either side is correct
        assert c.token == _brute_choice(l.tolist(), t, k, p, u), (trial, l, t, k, p, u)


def pin_greedy_generate_brute_force():
    """The greedy loop by full recompute (abi96062 model.py, SmolLM2Model.generate at
    temperature 0: the whole sequence again each step, the last position's argmax
    appended) against the scalar brute-force forward with an argmax written out by
    comparisons (lowest index among equal maxima): two prompt lengths, three steps,
    every sequence's token at every step, and the top-2 gaps the loop reports."""
    cfg = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                   rms_eps=1e-5, rope_theta=1e5)
    rng = _rng(57)
    mw = _rand_model(cfg, rng, std=0.6, norm_jitter=0.3)
    for T in (2, 5):
        prompt = rng.integers(0, cfg.vocab, size=(2, T))
        out, gaps = G.greedy_generate(prompt, 3, mw, cfg)
        seqs = [list(map(int, row)) for row in prompt]
        for j in range(3):
            logits = _brute_force_logits(cfg, mw, seqs)  # [B, len, V]
            for b in range(2):
                last = logits[b, len(seqs[b]) - 1]
                best = 0
                for v in range(1, cfg.vocab):
                    if last[v] > last[best]:
                        best = v
                srt = sorted(last)
                assert out[j, b] == best, (T, j, b)
                assert abs(gaps[j, b] - (srt[-1] - srt[-2])) < 1e-9
            for b in range(2):
                seqs[b].append(int(out[j, b]))


def pin_masked_decode_equals_masked_prefill():
    """A decode step under a padding mask (Sualeh77 model.py, "4. Attention": the
    attention_mask also applies on the cache branch) equals the masked prefill of one
    more token at that position and the scalar brute force; the cache it starts from
    is the masked prefill's, and the appended k', v equal the masked prefill's."""
    cfg = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                   rms_eps=1e-5, rope_theta=1e5)
    rng = _rng(59)
    mw = _rand_model(cfg, rng, std=0.6, norm_jitter=0.3)
    B, P = 2, 6
    ids = rng.integers(0, cfg.vocab, size=(B, P + 1))
    mask = np.array([[True, False, True, True, False, True, True], [True, True, False, False, True, False, True]])
    _, cache = O.model_prefill(ids[:, :P], mw, cfg, keep_cache=True, key_mask=mask[:, :P])
    logits, nk, nv = O.decode_step(ids[:, P], P, mw, cfg, [c[0] for c in cache], [c[1] for c in cache],
                                   key_mask=mask)
    full, cache_full = O.model_prefill(ids, mw, cfg, keep_cache=True, key_mask=mask)
    brute = _brute_force_logits(cfg, mw, ids.tolist(), mask.tolist())
    assert np.isfinite(logits).all()
    assert _rel(logits, full[:, P]) < 1e-12 and _rel(logits, brute[:, P]) < 1e-12
    for li in range(cfg.n_layers):
        assert np.allclose(nk[li], cache_full[li][0][:, :, P], rtol=1e-12)
        assert np.allclose(nv[li], cache_full[li][1][:, :, P], rtol=1e-12)
    unmasked, _, _ = O.decode_step(ids[:, P], P, mw, cfg, [c[0] for c in cache], [c[1] for c in cache])
    assert _rel(unmasked, logits) > 1e-3  # the mask matters on the cache branch


# ---------------------------------------------------------------- block backward
# (oracle/backward.py: the chain rule through the block of oracle/smol.py)

import oracle.backward as BW  # noqa: E402

GRAD_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def _block_loss(x, lw, cfg, dy, pos0, layer, mask):
    return float(np.sum(dy * O.block_forward(x, lw, cfg, pos0=pos0, key_mask=mask, layer=layer)))


def _finite_difference_check(cfg, lw, x, dy, pos0=0, layer=0, mask=None, seed=0, n_elem=10):
    """Central differences of L = sum(dy * block_forward(...)) in float64: for every
    gradient, n_elem single entries and one random direction over the whole tensor.
    With step 1e-5 the truncation and rounding errors are ~1e-9 relative."""
    g = BW.block_backward(x, lw, cfg, dy, pos0=pos0, layer=layer, key_mask=mask)
    rng = _rng(seed)
    h = 1e-5
    tensors = {"x": x, **{n: getattr(lw, n) for n in GRAD_NAMES}}
    for name, base in tensors.items():
        assert g[name].shape == np.shape(base), (name, g[name].shape, np.shape(base))

        def loss_at(delta):
            if name == "x":
                return _block_loss(x + delta, lw, cfg, dy, pos0, layer, mask)
            lw2 = O.LayerWeights(**{**lw.__dict__, name: getattr(lw, name) + delta})
            return _block_loss(x, lw2, cfg, dy, pos0, layer, mask)

        scale = max(np.max(np.abs(g[name])), 1e-12)
        flat_idx = rng.choice(np.size(base), size=min(n_elem, np.size(base)), replace=False)
        for fi in flat_idx:
            e = np.zeros(np.shape(base))
            e.flat[fi] = h
            fd = (loss_at(e) - loss_at(-e)) / (2 * h)
            assert abs(fd - g[name].flat[fi]) <= 1e-6 * scale, (name, int(fi), fd, g[name].flat[fi])
        r = rng.standard_normal(np.shape(base))
        fd = (loss_at(h * r) - loss_at(-h * r)) / (2 * h)
        an = float(np.sum(g[name] * r))
        assert abs(fd - an) <= 1e-6 * max(abs(fd), scale), (name, "direction", fd, an)


def pin_backward_finite_differences():
    """The block's gradients (input and all nine weights) against central finite
    differences of the forward oracle: rotary block at positions 3.., grouped heads
    (6 query heads over 2 kv heads), unit-scale activations."""
    cfg = _tiny_cfg()
    rng = _rng(51)
    lw = _rand_layer(cfg, rng, std=0.3, norm_jitter=0.3)
    x = rng.standard_normal((2, 5, cfg.hidden))
    dy = rng.standard_normal((2, 5, cfg.hidden))
    _finite_difference_check(cfg, lw, x, dy, pos0=3, seed=1)


def pin_backward_variants_finite_differences():
    """The same check on a NoPE block with a sliding window of 2 and a padding mask
    (nnterp SmolLM3 variants; Sualeh77 model.py, "4. Attention", attention_mask):
    masked and out-of-window keys receive no gradient through the scores; one kv
    head shared by 3 query heads."""
    cfg = O.Config(hidden=12, n_heads=3, n_kv_heads=1, intermediate=8, n_layers=2, vocab=16, max_pos=32,
                   rms_eps=1e-5, rope_theta=5e6, no_rope_interval=2, sliding_window=2)
    rng = _rng(52)
    lw = _rand_layer(cfg, rng, std=0.5, norm_jitter=0.3)
    x = rng.standard_normal((2, 6, cfg.hidden))
    dy = rng.standard_normal((2, 6, cfg.hidden))
    mask = np.array([[True, True, True, False, True, True, False, True],
                     [True, False, True, True, False, True, True, True]])  # no two masked keys in a row
    assert not cfg.rope_on(1) and cfg.window(1) == 2
    _finite_difference_check(cfg, lw, x, dy, pos0=2, layer=1, mask=mask, seed=2)
    _finite_difference_check(cfg, lw, x, dy, pos0=0, layer=0, mask=mask, seed=3)  # rotary block, no window


def pin_backward_vs_transformers_autograd():
    """The gradients equal torch autograd through transformers' Llama decoder layer
    (float64 weights; its RoPE angles are built in float32, hence ~1e-6 relative) at
    a SmolLM2-like head layout (9 query heads over 3 kv heads of 8)."""
    import torch

    cfg = O.Config(hidden=72, n_heads=9, n_kv_heads=3, intermediate=64, n_layers=1, vocab=32, max_pos=64,
                   rms_eps=1e-5, rope_theta=1e5)
    rng = _rng(53)
    lw = _rand_layer(cfg, rng, std=0.15, norm_jitter=0.2)
    mw = O.ModelWeights(embed=rng.standard_normal((cfg.vocab, cfg.hidden)), layers=[lw],
                        final_norm=np.ones(cfg.hidden))
    m = _hf_model(cfg, mw)
    T, pos0 = 11, 4
    x = rng.standard_normal((2, T, cfg.hidden))
    dy = rng.standard_normal((2, T, cfg.hidden))
    xt = torch.from_numpy(x).requires_grad_(True)
    pos = torch.arange(pos0, pos0 + T)[None]
    cos_sin = m.model.rotary_emb(xt, pos)
    mask = torch.full((T, T), -torch.inf, dtype=torch.float64).triu(1)[None, None]
    L = m.model.layers[0]
    L.zero_grad()
    out = L(xt, attention_mask=mask, position_ids=pos, position_embeddings=cos_sin)
    out = out[0] if isinstance(out, tuple) else out
    (out * torch.from_numpy(dy)).sum().backward()
    g = BW.block_backward(x, lw, cfg, dy, pos0=pos0)
    hf = {"x": xt.grad, "attn_norm": L.input_layernorm.weight.grad, "wq": L.self_attn.q_proj.weight.grad,
          "wk": L.self_attn.k_proj.weight.grad, "wv": L.self_attn.v_proj.weight.grad,
          "wo": L.self_attn.o_proj.weight.grad, "mlp_norm": L.post_attention_layernorm.weight.grad,
          "w_gate": L.mlp.gate_proj.weight.grad, "w_up": L.mlp.up_proj.weight.grad,
          "w_down": L.mlp.down_proj.weight.grad}
    for name, want in hf.items():
        assert _rel(g[name], want.detach().numpy()) < 1e-5, (name, _rel(g[name], want.detach().numpy()))


def pin_backward_special_cases():
    """Closed forms: with w_down = 0 and wo = 0 the block is the identity, so dx = dy
    and only w_down and wo get gradients (the sublayers' other weights sit behind a
    zero map); the w_down gradient is then dy^T silu(gate) * up of the normed input;
    with dy = 0 every gradient is 0."""
    cfg = _tiny_cfg()
    rng = _rng(54)
    lw = _rand_layer(cfg, rng, std=0.3, norm_jitter=0.3)
    lw0 = O.LayerWeights(**{**lw.__dict__, "w_down": np.zeros_like(lw.w_down), "wo": np.zeros_like(lw.wo)})
    x = rng.standard_normal((2, 4, cfg.hidden))
    dy = rng.standard_normal((2, 4, cfg.hidden))
    g = BW.block_backward(x, lw0, cfg, dy)
    assert np.array_equal(g["x"], dy)
    for n in ("attn_norm", "wq", "wk", "wv", "mlp_norm", "w_gate", "w_up"):
        assert not np.any(g[n]), n
    w = O.rms_norm(x, lw.mlp_norm, cfg.rms_eps).reshape(-1, cfg.hidden)
    y = O.silu(w @ lw.w_gate.T) * (w @ lw.w_up.T)
    assert _rel(g["w_down"], dy.reshape(-1, cfg.hidden).T @ y) < 1e-12
    assert np.any(g["wo"])
    z = BW.block_backward(x, lw, cfg, np.zeros_like(dy))
    assert all(not np.any(v) for v in z.values())


ALL_PINS = [
    pin_rmsnorm_closed_forms,
    pin_rmsnorm_vs_torch,
    pin_inv_freq_closed_form,
    pin_rope_complex_form,
    pin_rope_invariants,
    pin_attention_vs_sdpa,
    pin_attention_special_cases,
    pin_causality,
    pin_silu_values,
    pin_swiglu_special_case,
    pin_model_vs_transformers,
    pin_block_vs_transformers_smollm2_shape,
    pin_param_count,
    pin_logits_shape,
    pin_gqa_mapping_smollm3,
    pin_decode_equals_prefill,
    pin_brute_force_tiny,
    pin_padding_mask,
    pin_nope_blocks_and_window,
    pin_greedy_ties_and_nan,
    pin_top_k_keeps_ties,
    pin_top_p_hand_values,
    pin_top_p_after_top_k,
    pin_inverse_cdf_stratified,
    pin_inverse_cdf_steps,
    pin_choice_brute_force,
    pin_greedy_generate_brute_force,
    pin_masked_decode_equals_masked_prefill,
    pin_backward_finite_differences,
    pin_backward_variants_finite_differences,
    pin_backward_vs_transformers_autograd,
    pin_backward_special_cases,
]

SAMPLER_PINS = [p for p in ALL_PINS if p.__name__ in (
    "pin_greedy_ties_and_nan", "pin_top_k_keeps_ties", "pin_top_p_hand_values", "pin_top_p_after_top_k",
    "pin_inverse_cdf_stratified", "pin_inverse_cdf_steps", "pin_choice_brute_force",
    "pin_greedy_generate_brute_force")]

BACKWARD_PINS = [p for p in ALL_PINS if p.__name__.startswith("pin_backward")]
