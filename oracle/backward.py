"""Plain CPU oracle for the backward pass of one decoder block.

TEST INFRASTRUCTURE ONLY (see oracle/smol.py): nothing on the product path may
import, call or run this module.

The block is the one of oracle/smol.py (nnterp SmolLM3, "The block, in order";
abi96062 components.py, TransformerBlock / RMSNorm / GroupedQueryAttention /
SwiGLU_FFN; Sualeh77 model.py, "2." to "6."). The pages train it (Sualeh77's model
is trained on TinyShakespeare; abi96062 model.py initialises it for training) but
print no gradient formula, so this module is the chain rule applied to the forward
definition, step by step in reverse, in float64. It is pinned by central finite
differences of the forward (tests/oracle_pins.py), not by anything it shares with
the forward.

block_backward returns the gradients of L = sum(dy * block(x)) with respect to x
and to each of the block's nine weight tensors.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .smol import Config, LayerWeights, rope_inv_freq, silu

F64 = np.float64


def _rms_forward(x, w, eps):
    """u = w * n with n = x * r, r = 1 / sqrt(mean(x^2) + eps); returns (u, n, r)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x * r
    return w * n, n, r


def _rms_backward(du, n, r, w):
    """From du to (dx, dw) for u = w * n, n = x * r (r depends on the whole row):
    dn = du * w; dx = r * (dn - n * mean(dn * n)); dw = sum over rows of du * n."""
    dn = du * w
    dx = r * (dn - n * np.mean(dn * n, axis=-1, keepdims=True))
    dw = np.sum((du * n).reshape(-1, n.shape[-1]), axis=0)
    return dx, dw


def _rotate(z, positions, theta, sign):
    """The RoPE rotation of pairs (i, i + d/2) by sign * position * omega_i; sign -1
    is its transpose (the rotation is orthogonal), which carries gradients back."""
    d = z.shape[-1]
    ang = sign * np.asarray(positions, F64)[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = z[..., : d // 2], z[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _silu_grad(g):
    """d silu(g) / dg = s (1 + g (1 - s)) with s the logistic sigmoid of g."""
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def _attention_backward(P, do, q, k, v, scale):
    """One (sequence, query head) of o = softmax(scale * q k^T + mask) v, carried back:
    with p the probabilities, dv = p^T do, dp = do v^T, ds = p * (dp - rowsum(dp * p))
    (the softmax Jacobian), dq = scale * ds k, dk = scale * ds^T q. Masked entries
    have p = 0, so they pass nothing back. Returns (dq, dk, dv) of this head; a kv
    head shared by a group of query heads sums the group's dk and dv."""
    dv = P.T @ do
    dp = do @ v.T
    ds = P * (dp - np.sum(dp * P, axis=-1, keepdims=True))
    return (ds @ k) * scale, (ds.T @ q) * scale, dv


def block_backward(x, lw: LayerWeights, cfg: Config, dy, pos0: int = 0, layer: int = 0,
                   key_mask: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dy * block_forward(x)) for x [B, T, H] at positions pos0.. .

    Returns {"x": dx, "attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
    "w_up", "w_down": gradients shaped like the weights}."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    B, T, H = x.shape
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    W = {k: np.asarray(getattr(lw, k), F64) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
                                                      "w_up", "w_down")}
    pos = np.arange(pos0, pos0 + T)
    rope = cfg.rope_on(layer)
    win = cfg.window(layer)

    # ---- forward, keeping what the backward needs
    u, n1, r1 = _rms_forward(x, W["attn_norm"], cfg.rms_eps)
    q0 = (u @ W["wq"].T).reshape(B, T, nq, d).transpose(0, 2, 1, 3)   # [B, nq, T, d]
    k0 = (u @ W["wk"].T).reshape(B, T, nkv, d).transpose(0, 2, 1, 3)  # [B, nkv, T, d]
    v = (u @ W["wv"].T).reshape(B, T, nkv, d).transpose(0, 2, 1, 3)
    q = _rotate(q0, pos, cfg.rope_theta, 1.0) if rope else q0
    k = _rotate(k0, pos, cfg.rope_theta, 1.0) if rope else k0
    vis = pos[None, :] <= pos[:, None]  # [T (query), T (key)]
    if win > 0:
        vis &= pos[None, :] > pos[:, None] - win
    scale = 1.0 / np.sqrt(d)
    P = np.empty((B, nq, T, T), F64)
    O = np.empty((B, nq, T, d), F64)
    for b in range(B):
        vb = vis if key_mask is None else vis & np.asarray(key_mask[b], bool)[None, pos]
        for hh in range(nq):
            g = hh // G
            s = np.where(vb, (q[b, hh] @ k[b, g].T) * scale, -np.inf)
            m = s.max(axis=-1, keepdims=True)
            e = np.exp(s - m)
            P[b, hh] = e / e.sum(axis=-1, keepdims=True)
            O[b, hh] = P[b, hh] @ v[b, g]
    o = O.transpose(0, 2, 1, 3).reshape(B, T, nq * d)
    h = x + o @ W["wo"].T
    wv_, n2, r2 = _rms_forward(h, W["mlp_norm"], cfg.rms_eps)
    gt = wv_ @ W["w_gate"].T
    up = wv_ @ W["w_up"].T
    sg = silu(gt)
    yy = sg * up

    # ---- backward, in reverse order
    grads: Dict[str, np.ndarray] = {}
    M = B * T
    flat = lambda a: a.reshape(M, a.shape[-1])  # noqa: E731
    dh = dy.copy()                                  # out = h + ...
    grads["w_down"] = flat(dy).T @ flat(yy)        # out = ... + y Wd^T
    dyy = dy @ W["w_down"]
    dgt = dyy * up * _silu_grad(gt)
    dup = dyy * sg
    grads["w_gate"] = flat(dgt).T @ flat(wv_)
    grads["w_up"] = flat(dup).T @ flat(wv_)
    dwv = dgt @ W["w_gate"] + dup @ W["w_up"]
    dh2, grads["mlp_norm"] = _rms_backward(dwv, n2, r2, W["mlp_norm"])
    dh = dh + dh2
    dx = dh.copy()                                  # h = x + ...
    grads["wo"] = flat(dh).T @ flat(o)
    do = (dh @ W["wo"]).reshape(B, T, nq, d).transpose(0, 2, 1, 3)  # [B, nq, T, d]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for hh in range(nq):
            g = hh // G
            dq[b, hh], dkh, dvh = _attention_backward(P[b, hh], do[b, hh], q[b, hh], k[b, g], v[b, g], scale)
            dk[b, g] += dkh
            dv[b, g] += dvh
    dq0 = _rotate(dq, pos, cfg.rope_theta, -1.0) if rope else dq
    dk0 = _rotate(dk, pos, cfg.rope_theta, -1.0) if rope else dk
    dq0f = dq0.transpose(0, 2, 1, 3).reshape(B, T, nq * d)
    dk0f = dk0.transpose(0, 2, 1, 3).reshape(B, T, nkv * d)
    dvf = dv.transpose(0, 2, 1, 3).reshape(B, T, nkv * d)
    grads["wq"] = flat(dq0f).T @ flat(u)
    grads["wk"] = flat(dk0f).T @ flat(u)
    grads["wv"] = flat(dvf).T @ flat(u)
    du = dq0f @ W["wq"] + dk0f @ W["wk"] + dvf @ W["wv"]
    dx1, grads["attn_norm"] = _rms_backward(du, n1, r1, W["attn_norm"])
    grads["x"] = dx + dx1
    return grads
