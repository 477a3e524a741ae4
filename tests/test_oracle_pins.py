"""The CPU oracle against its pins, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle.smol as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
# Each entry replaces one oracle function with a plausibly wrong variant; at least one
# pin must fail on it. The mistakes are planted in the oracle, on the CPU.

F64 = np.float64


def _rms_eps_outside(x, w, eps):
    x = np.asarray(x, F64)
    return np.asarray(w, F64) * x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)


def _rms_sum_not_mean(x, w, eps):
    x = np.asarray(x, F64)
    return np.asarray(w, F64) * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _rms_weight_dropped(x, w, eps):
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _inv_freq_half_exponent(d, theta):
    return float(theta) ** (-np.arange(d // 2, dtype=F64) / d)


def _rope_interleaved(z, positions, theta):
    z = np.asarray(z, F64)
    d = z.shape[-1]
    ang = np.asarray(positions, F64)[..., None] * O.rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = z[..., 0::2], z[..., 1::2]
    out = np.empty_like(z)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _rope_sign_flipped(z, positions, theta):
    z = np.asarray(z, F64)
    d = z.shape[-1]
    ang = np.asarray(positions, F64)[..., None] * O.rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = z[..., : d // 2], z[..., d // 2:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def _make_attention(mapping="div", scale="sqrt", strict=False, mask="keys", window_off=0):
    def attn(q, k, v, q_pos, k_pos, key_mask=None, window=0):
        q, k, v = (np.asarray(a, F64) for a in (q, k, v))
        B, nq, T, d = q.shape
        nkv = k.shape[1]
        G = nq // nkv
        qp, kp = np.asarray(q_pos), np.asarray(k_pos)
        vis = (kp[None, :] < qp[:, None]) if strict else (kp[None, :] <= qp[:, None])
        if window > 0:
            vis = vis & (kp[None, :] > qp[:, None] - window - window_off)
        sc = 1.0 / np.sqrt(d) if scale == "sqrt" else 1.0 / d
        out = np.empty((B, nq, T, d))
        for b in range(B):
            vb = vis
            if key_mask is not None and mask == "keys":
                vb = vis & np.asarray(key_mask[b], bool)[None, :]
            elif key_mask is not None and mask == "queries":  # the mask applied to query rows
                vb = vis & np.asarray(key_mask[b], bool)[-T:][:, None]
            for h in range(nq):
                g = h // G if mapping == "div" else h % nkv
                s = np.where(vb, (q[b, h] @ k[b, g].T) * sc, -np.inf)
                with np.errstate(invalid="ignore"):
                    out[b, h] = O.softmax(s) @ v[b, g]
        return out
    return attn


def _swiglu_swapped(u, wg, wu, wd):
    g = u @ np.asarray(wg, F64).T
    up = u @ np.asarray(wu, F64).T
    return (O.silu(up) * g) @ np.asarray(wd, F64).T


def _silu_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, F64)))


def _block_no_mlp_residual(x, lw, cfg, pos0=0, return_parts=False, key_mask=None, layer=0):
    x = np.asarray(x, F64)
    positions = np.arange(pos0, pos0 + x.shape[1])
    attn, k, v = O.attention_sublayer(x, lw, cfg, positions, key_mask=key_mask, layer=layer)
    h = x + attn
    mlp = O.mlp_sublayer(h, lw, cfg)
    out = mlp + attn  # the first residual's x is dropped
    if return_parts:
        return out, {"attn": attn, "mlp": mlp, "k": k, "v": v}
    return out


def _mlp_reads_stream_not_norm(h, lw, cfg):
    return O.swiglu_mlp(np.asarray(h, F64), lw.w_gate, lw.w_up, lw.w_down)


_orig_attention_sublayer = O.attention_sublayer


def _attention_rotates_v(x, lw, cfg, positions, past_k=None, past_v=None, past_pos=None, key_mask=None, layer=0):
    out, k, v = _orig_attention_sublayer(x, lw, cfg, positions, past_k, past_v, past_pos, key_mask, layer)
    vr = O.rope_rotate(v, np.asarray(positions), cfg.rope_theta)
    # recompute the output with rotated values
    B, T, H = np.asarray(x).shape
    d = cfg.head_dim
    u = O.rms_norm(x, lw.attn_norm, cfg.rms_eps)
    q = (u @ np.asarray(lw.wq, F64).T).reshape(B, T, cfg.n_heads, d).transpose(0, 2, 1, 3)
    if cfg.rope_on(layer):
        q = O.rope_rotate(q, np.asarray(positions), cfg.rope_theta)
    if past_k is not None:
        k_all = np.concatenate([past_k, k], 2)
        v_all = np.concatenate([past_v, vr], 2)
        kp = np.concatenate([past_pos, positions])
    else:
        k_all, v_all, kp = k, vr, positions
    km = None if key_mask is None else np.asarray(key_mask, bool)[:, np.asarray(kp)]
    o = O.gqa_attention(q, k_all, v_all, positions, kp, km, cfg.window(layer)).transpose(0, 2, 1, 3).reshape(B, T, -1)
    return o @ np.asarray(lw.wo, F64).T, k, vr


def _attention_wo_transposed(x, lw, cfg, positions, past_k=None, past_v=None, past_pos=None, key_mask=None, layer=0):
    import copy
    lw2 = copy.copy(lw)
    lw2.wo = np.asarray(lw.wo).T
    return _orig_attention_sublayer(x, lw2, cfg, positions, past_k, past_v, past_pos, key_mask, layer)


def _lm_head_no_final_norm(x, final_norm, E, cfg):
    return np.asarray(x, F64) @ np.asarray(E, F64).T


_orig_decode_step = O.decode_step


def _decode_step_ignores_mask(ids, cache_len, mw, cfg, k_cache, v_cache, key_mask=None):
    return _orig_decode_step(ids, cache_len, mw, cfg, k_cache, v_cache)


MISTAKES = {
    "rmsnorm eps outside the root": ("rms_norm", _rms_eps_outside),
    "rmsnorm sum instead of mean": ("rms_norm", _rms_sum_not_mean),
    "rmsnorm weight dropped": ("rms_norm", _rms_weight_dropped),
    "inv_freq exponent halved": ("rope_inv_freq", _inv_freq_half_exponent),
    "rope interleaved pairs": ("rope_rotate", _rope_interleaved),
    "rope sign flipped": ("rope_rotate", _rope_sign_flipped),
    "gqa head h % n_kv": ("gqa_attention", _make_attention(mapping="mod")),
    "attention scale 1/d": ("gqa_attention", _make_attention(scale="d")),
    "causal mask excludes the diagonal": ("gqa_attention", _make_attention(strict=True)),
    "padding mask ignored": ("gqa_attention", _make_attention(mask="ignored")),
    "padding mask applied to queries": ("gqa_attention", _make_attention(mask="queries")),
    "sliding window one key too wide": ("gqa_attention", _make_attention(window_off=1)),
    "NoPE on blocks 0, 4, 8, ...": ("Config.rope_on", lambda self, layer: not (self.no_rope_interval > 0 and layer % self.no_rope_interval == 0)),
    "swiglu gate and up swapped": ("swiglu_mlp", _swiglu_swapped),
    "silu is the sigmoid": ("silu", _silu_sigmoid),
    "block drops the residual x": ("block_forward", _block_no_mlp_residual),
    "mlp reads the stream, not its norm": ("mlp_sublayer", _mlp_reads_stream_not_norm),
    "rope applied to v": ("attention_sublayer", _attention_rotates_v),
    "o_proj transposed": ("attention_sublayer", _attention_wo_transposed),
    "final norm dropped": ("lm_head", _lm_head_no_final_norm),
    "decode step ignores the padding mask": ("decode_step", _decode_step_ignores_mask),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = MISTAKES[name]
    if attr.startswith("Config."):
        monkeypatch.setattr(O.Config, attr.split(".", 1)[1], bad)
    else:
        monkeypatch.setattr(O, attr, bad)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught: {name}"


# ---------------------------------------------------------------- planted mistakes in the sampler
import oracle.generate as G  # noqa: E402


def _top_k_exactly_k(logits, k):
    V = logits.shape[0]
    if k <= 0 or k >= V:
        return np.ones(V, dtype=bool)
    keep = np.zeros(V, dtype=bool)
    keep[np.argsort(-logits, kind="stable")[:k]] = True
    return keep


def _top_p_without_crossing_token(logits, weights, keep, p):
    if p >= 1.0:
        return keep, np.inf
    idx = np.nonzero(keep)[0]
    order = idx[np.lexsort((idx, -logits[idx]))]
    cum = np.cumsum(weights[order] / weights[order].sum())
    new = np.zeros_like(keep)
    new[order[cum <= p]] = True
    new[order[0]] = True
    return new, np.inf


def _top_p_before_top_k(logits, weights, keep, p):
    # the nucleus measured with the probabilities of every token, not of the top-k survivors
    return _top_p_plain(logits, np.exp(logits - logits.max()), keep, p)


def _top_p_plain(logits, full, keep, p):
    if p >= 1.0:
        return keep, np.inf
    idx = np.nonzero(keep)[0]
    order = idx[np.lexsort((idx, -logits[idx]))]
    cum = np.cumsum(full[order] / full.sum())
    over = np.nonzero(cum > p)[0]
    s = int(over[0]) if over.size else len(order) - 1
    new = np.zeros_like(keep)
    new[order[: s + 1]] = True
    return new, np.inf


def _top_p_ties_by_descending_index(logits, weights, keep, p):
    if p >= 1.0:
        return keep, np.inf
    idx = np.nonzero(keep)[0]
    order = idx[np.lexsort((-idx, -logits[idx]))]
    cum = np.cumsum(weights[order] / weights[order].sum())
    over = np.nonzero(cum > p)[0]
    s = int(over[0]) if over.size else len(order) - 1
    new = np.zeros_like(keep)
    new[order[: s + 1]] = True
    return new, np.inf


def _make_next_token(side="right", temp_mul=False, greedy_last=False):
    def next_token(logits, temperature, top_k=0, top_p=1.0, u=0.0):
        l = np.asarray(logits, dtype=np.float64)
        if np.isnan(l).any():
            return G.Choice(-1, None, np.inf, np.inf)
        if temperature == 0:
            j = len(l) - 1 - int(np.argmax(l[::-1])) if greedy_last else int(np.argmax(l))
            return G.Choice(j, None, np.inf, np.inf)
        if not np.isfinite(l.max()):
            return G.Choice(-1, None, np.inf, np.inf)
        keep = G.top_k_keep(l, top_k)
        z = l * temperature if temp_mul else l / temperature
        w = np.where(keep, np.exp(z - z.max()), 0.0)
        keep, pm = G.top_p_keep(l, w, keep, top_p)
        w = np.where(keep, w, 0.0)
        cdf = np.cumsum(w / w.sum())
        j = min(int(np.searchsorted(cdf, u, side=side)), len(l) - 1)
        return G.Choice(j, keep, pm, np.inf)
    return next_token


def _make_greedy_generate(row_off=1, append_first=False):
    """The recompute loop with a slip: logits read from position T - row_off, or the
    previous token appended before the step's forward instead of after it."""
    def greedy_generate(prompt, max_new, mw, cfg):
        ids = np.asarray(prompt, dtype=np.int64)
        B = ids.shape[0]
        out = np.zeros((max_new, B), dtype=np.int64)
        gaps = np.zeros((max_new, B))
        prev = ids[:, -1].copy()
        for j in range(max_new):
            if append_first:
                ids = np.concatenate([ids, prev[:, None]], axis=1)
            T = ids.shape[1]
            row = O.model_prefill(ids, mw, cfg, logit_rows=[b * T + T - row_off for b in range(B)])
            for b in range(B):
                out[j, b] = G.next_token(row[b], 0.0).token
                top2 = np.sort(row[b])[-2:]
                gaps[j, b] = top2[1] - top2[0]
            prev = out[j].copy()
            if not append_first:
                ids = np.concatenate([ids, out[j][:, None]], axis=1)
        return out, gaps
    return greedy_generate


GEN_MISTAKES = {
    "top-k keeps exactly k tokens (drops ties)": ("top_k_keep", _top_k_exactly_k),
    "top-p drops the token that crosses p": ("top_p_keep", _top_p_without_crossing_token),
    "top-p measured before top-k renormalises": ("top_p_keep", _top_p_before_top_k),
    "top-p ranks equal logits by descending index": ("top_p_keep", _top_p_ties_by_descending_index),
    "draw takes the first cdf >= u": ("next_token", _make_next_token(side="left")),
    "temperature multiplies the logits": ("next_token", _make_next_token(temp_mul=True)),
    "greedy takes the last maximum": ("next_token", _make_next_token(greedy_last=True)),
    "greedy loop reads the second-to-last position": ("greedy_generate", _make_greedy_generate(row_off=2)),
    "greedy loop appends the token before the step": ("greedy_generate", _make_greedy_generate(append_first=True)),
}


@pytest.mark.parametrize("name", sorted(GEN_MISTAKES))
def test_sampler_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = GEN_MISTAKES[name]
    monkeypatch.setattr(G, attr, bad)
    failed = []
    for pin in P.SAMPLER_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught: {name}"


# ---------------------------------------------------------------- planted mistakes in the backward
import oracle.backward as BW  # noqa: E402


def _rms_backward_no_mean(du, n, r, w):
    return r * (du * w), np.sum((du * n).reshape(-1, n.shape[-1]), axis=0)


def _rms_backward_no_r(du, n, r, w):
    dn = du * w
    return dn - n * np.mean(dn * n, axis=-1, keepdims=True), np.sum((du * n).reshape(-1, n.shape[-1]), axis=0)


def _rotate_forward_only(z, positions, theta, sign):
    return O.rope_rotate(z, positions, theta)


def _make_attention_backward(row_sum=True, dk_scale=True, dv_transposed=False):
    def attention_backward(P, do, q, k, v, scale):
        dv = (P @ do) if dv_transposed else (P.T @ do)
        dp = do @ v.T
        ds = P * (dp - np.sum(dp * P, axis=-1, keepdims=True)) if row_sum else P * dp
        return (ds @ k) * scale, (ds.T @ q) * (scale if dk_scale else 1.0), dv
    return attention_backward


def _silu_grad_sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


BW_MISTAKES = {
    "rmsnorm backward drops the mean term": ("_rms_backward", _rms_backward_no_mean),
    "rmsnorm backward drops the 1/rms factor": ("_rms_backward", _rms_backward_no_r),
    "rotary carried back by +angle": ("_rotate", _rotate_forward_only),
    "softmax backward without the row sum": ("_attention_backward", _make_attention_backward(row_sum=False)),
    "dk without the 1/sqrt(d) scale": ("_attention_backward", _make_attention_backward(dk_scale=False)),
    "dv from P, not its transpose": ("_attention_backward", _make_attention_backward(dv_transposed=True)),
    "silu derivative taken as the sigmoid": ("_silu_grad", _silu_grad_sigmoid),
}


@pytest.mark.parametrize("name", sorted(BW_MISTAKES))
def test_backward_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = BW_MISTAKES[name]
    monkeypatch.setattr(BW, attr, bad)
    failed = []
    for pin in P.BACKWARD_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught: {name}"
