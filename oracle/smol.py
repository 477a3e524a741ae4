"""Plain CPU oracle for the forward pass of a LLaMA-style pre-norm decoder stack.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it. It shares no code with the HIP library and imports
nothing from the package; callers hand it plain numpy arrays.

Every function is the plain definition of its step, written out in float64 with
numpy (``@`` is the only library primitive used for the contractions). The
sources are five web pages about SmolLM2-135M / SmolLM3; each function names the
page and section it follows:

* "model.py" of the Sualeh77 SmolLM2 HF Space (sections "1. Config" to "8. Quick
  self-test"), here called *Sualeh77 model.py*;
* "SmolLM3" of the nnterp encyclopedia, here *nnterp SmolLM3*;
* "block.py" of tohio/slm-125m-instruct, here *tohio block.py*;
* "model.py" and "components.py" of abi96062/smolLM2-135-implementation, here
  *abi96062 model.py* / *abi96062 components.py*.

Readings taken where the pages are silent or disagree (each also pinned by a
test in tests/test_oracle_pins.py):

* inverse frequencies are theta^(-2i/d) for i < d/2 (the two pages' forms agree);
* RoPE rotates the pair (i, i + d/2) of every q and k head, never v, with angles
  from integer positions (never positions rounded to the model dtype);
* query head h reads key/value head h // (n_heads / n_kv_heads);
* a query at absolute position p sees every key with position <= p;
* RMSNorm adds eps to the mean square inside the root, then scales by w.

parity pinned: every function below is pinned by at least one closed form,
invariant, special case, library routine or brute-force check in
tests/test_oracle_pins.py; the absolute logits of a random-weight model have no
printed value on the pages and are pinned only through those.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

F64 = np.float64


@dataclass(frozen=True)
class Config:
    """Model shape. SmolLM2-135M values from the HF LlamaConfig printed in
    Sualeh77 model.py, section "1. Config"."""

    hidden: int = 576
    n_heads: int = 9
    n_kv_heads: int = 3
    intermediate: int = 1536
    n_layers: int = 30
    vocab: int = 49152
    max_pos: int = 8192
    rms_eps: float = 1e-5
    rope_theta: float = 100000.0
    # SmolLM3 variants (nnterp SmolLM3, "NoPE blocks" and "A sliding window the 3B
    # checkpoints leave off"): with no_rope_interval k > 0, block l applies no rotary
    # when (l + 1) % k == 0; with sliding_window W > 0 those blocks attend only to
    # the W most recent positions (their own included).
    no_rope_interval: int = 0
    sliding_window: int = 0

    def rope_on(self, layer: int) -> bool:
        k = self.no_rope_interval
        return not (k > 0 and (layer + 1) % k == 0)

    def window(self, layer: int) -> int:
        return self.sliding_window if (self.sliding_window > 0 and not self.rope_on(layer)) else 0

    @property
    def head_dim(self) -> int:
        # Sualeh77 model.py, "1. Config": head_dim = hidden // heads (576 / 9 = 64)
        return self.hidden // self.n_heads

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads


@dataclass
class LayerWeights:
    """One block's weights, every matrix [out, in] as nn.Linear stores it
    (abi96062 components.py, GroupedQueryAttention / SwiGLU_FFN)."""

    attn_norm: np.ndarray  # [H]
    wq: np.ndarray  # [n_heads*d, H]
    wk: np.ndarray  # [n_kv*d, H]
    wv: np.ndarray  # [n_kv*d, H]
    wo: np.ndarray  # [H, n_heads*d]
    mlp_norm: np.ndarray  # [H]
    w_gate: np.ndarray  # [I, H]
    w_up: np.ndarray  # [I, H]
    w_down: np.ndarray  # [H, I]


@dataclass
class ModelWeights:
    embed: np.ndarray  # [V, H]; also the lm_head (tied)
    layers: List[LayerWeights] = field(default_factory=list)
    final_norm: Optional[np.ndarray] = None  # [H]


# ---------------------------------------------------------------- parameters


def param_shapes(cfg: Config, tied: bool = True) -> List[tuple]:
    """Every parameter tensor's shape, counted once (abi96062 model.py,
    get_num_params: the tied embedding / lm_head is one parameter)."""
    d = cfg.head_dim
    shapes = [(cfg.vocab, cfg.hidden)]
    for _ in range(cfg.n_layers):
        shapes += [
            (cfg.hidden,),  # input_layernorm
            (cfg.n_heads * d, cfg.hidden),
            (cfg.n_kv_heads * d, cfg.hidden),
            (cfg.n_kv_heads * d, cfg.hidden),
            (cfg.hidden, cfg.n_heads * d),
            (cfg.hidden,),  # post_attention_layernorm
            (cfg.intermediate, cfg.hidden),
            (cfg.intermediate, cfg.hidden),
            (cfg.hidden, cfg.intermediate),
        ]
    shapes.append((cfg.hidden,))  # final norm
    if not tied:
        shapes.append((cfg.vocab, cfg.hidden))
    return shapes


def param_count(cfg: Config, tied: bool = True) -> int:
    return int(sum(int(np.prod(s)) for s in param_shapes(cfg, tied)))


# ---------------------------------------------------------------- primitives


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: w * x / sqrt(mean(x^2) + eps).

    abi96062 components.py, RMSNorm (docstring formula and forward);
    Sualeh77 model.py, "2. RMSNorm"."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(w, F64) * (x / np.sqrt(ms + eps))


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i = 0 .. d/2-1.

    abi96062 components.py, RotaryEmbedding.__init__ (arange(0, d, 2) / d);
    Sualeh77 model.py, "3. RoPE", rope_freqs (arange(d/2) / (d/2), the same)."""
    i = np.arange(head_dim // 2, dtype=F64)
    return float(theta) ** (-(2.0 * i) / head_dim)


def rope_rotate(z: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate the last axis of z (length d) at the given integer positions.

    z has shape [..., T, d]; positions has shape [T] (or broadcasts to z[..., 0]).
    The pair (i, i + d/2) is rotated by angle p * omega_i:
        z'_i       = z_i cos - z_{i+d/2} sin
        z'_{i+d/2} = z_{i+d/2} cos + z_i sin
    Sualeh77 model.py, "3. RoPE", apply_rope (split-halves form);
    abi96062 components.py, rotate_half / apply_rotary_pos_emb (the same map);
    rope_interleaved is false in the SmolLM2 config."""
    z = np.asarray(z, F64)
    d = z.shape[-1]
    half = d // 2
    pos = np.asarray(positions, F64)
    ang = pos[..., None] * rope_inv_freq(d, theta)  # [..., T, d/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = z[..., :half], z[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Max-subtracted softmax; -inf entries get probability 0."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def gqa_attention(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    q_pos: np.ndarray,
    k_pos: np.ndarray,
    key_mask: Optional[np.ndarray] = None,
    window: int = 0,
) -> np.ndarray:
    """Causal grouped-query attention by its definition.

    q: [B, n_heads, T, d]; k, v: [B, n_kv, S, d]; q_pos: [T]; k_pos: [S]
    (absolute positions). Query head h uses kv head h // (n_heads / n_kv).
    For each query at position p the scores s_j = q . k_j / sqrt(d) over keys
    with k_pos_j <= p go through softmax and weight v_j. Returns [B, n_heads, T, d].

    Sualeh77 model.py, "4. Attention" (scores / sqrt(d), triu(1) mask, softmax,
    probs @ v; with a cache a single new token sees every cached key; an optional
    padding mask is added to the scores as 0 / -inf per key);
    abi96062 components.py, GroupedQueryAttention (repeat_interleave + causal SDPA);
    nnterp SmolLM3, "Grouped-query attention" (head h reads kv head h // group,
    scale head_dim ** -0.5).

    key_mask: optional bool [B, S], False = key j of sequence b gets -inf added to
    its score for every query and head. window W > 0: a query at position p sees
    only keys with p - W < position <= p. A query left with no visible key gets the
    softmax of all -inf, NaN."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    B, nq, T, d = q.shape
    nkv = k.shape[1]
    group = nq // nkv
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]  # [T, S]
    if window > 0:
        visible &= np.asarray(k_pos)[None, :] > np.asarray(q_pos)[:, None] - window
    out = np.empty((B, nq, T, d), F64)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        vis = visible if key_mask is None else visible & np.asarray(key_mask[b], bool)[None, :]
        for h in range(nq):
            g = h // group
            s = (q[b, h] @ k[b, g].T) * scale  # [T, S]
            s = np.where(vis, s, -np.inf)
            with np.errstate(invalid="ignore"):
                out[b, h] = softmax(s, axis=-1) @ v[b, g]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z)."""
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(u: np.ndarray, w_gate, w_up, w_down) -> np.ndarray:
    """down(silu(gate(u)) * up(u)).

    abi96062 components.py, SwiGLU_FFN (docstring formula and forward);
    Sualeh77 model.py, "5. MLP (SwiGLU)" (fused fc1 with gate = first half)."""
    g = u @ np.asarray(w_gate, F64).T
    up = u @ np.asarray(w_up, F64).T
    return (silu(g) * up) @ np.asarray(w_down, F64).T


# ---------------------------------------------------------------- the block


def attention_sublayer(x, lw: LayerWeights, cfg: Config, positions, past_k=None, past_v=None, past_pos=None,
                       key_mask=None, layer: int = 0):
    """self_attn(input_layernorm(x)) for x [B, T, H].

    Returns (attn_out [B,T,H], k_rot [B,n_kv,T,d], v [B,n_kv,T,d]); the cache
    holds keys after RoPE and before any head repetition (Sualeh77 model.py,
    "4. Attention", the stored k_cache / v_cache). key_mask: optional bool
    [B, >= last position + 1] over absolute key positions (False: masked). layer:
    the block's index, which decides the rotary and the window (Config)."""
    x = np.asarray(x, F64)
    B, T, H = x.shape
    d = cfg.head_dim
    u = rms_norm(x, lw.attn_norm, cfg.rms_eps)
    q = (u @ np.asarray(lw.wq, F64).T).reshape(B, T, cfg.n_heads, d).transpose(0, 2, 1, 3)
    k = (u @ np.asarray(lw.wk, F64).T).reshape(B, T, cfg.n_kv_heads, d).transpose(0, 2, 1, 3)
    v = (u @ np.asarray(lw.wv, F64).T).reshape(B, T, cfg.n_kv_heads, d).transpose(0, 2, 1, 3)
    positions = np.asarray(positions)
    if cfg.rope_on(layer):  # a NoPE block keeps q and k as projected (nnterp SmolLM3)
        q = rope_rotate(q, positions, cfg.rope_theta)
        k = rope_rotate(k, positions, cfg.rope_theta)
    if past_k is not None:
        k_all = np.concatenate([np.asarray(past_k, F64), k], axis=2)
        v_all = np.concatenate([np.asarray(past_v, F64), v], axis=2)
        k_pos = np.concatenate([np.asarray(past_pos), positions])
    else:
        k_all, v_all, k_pos = k, v, positions
    km = None if key_mask is None else np.asarray(key_mask, bool)[:, np.asarray(k_pos)]
    o = gqa_attention(q, k_all, v_all, positions, k_pos, km, cfg.window(layer))  # [B, nq, T, d]
    o = o.transpose(0, 2, 1, 3).reshape(B, T, cfg.n_heads * d)  # column h*d + e
    return o @ np.asarray(lw.wo, F64).T, k, v


def mlp_sublayer(h, lw: LayerWeights, cfg: Config):
    """mlp(post_attention_layernorm(h))."""
    w = rms_norm(h, lw.mlp_norm, cfg.rms_eps)
    return swiglu_mlp(w, lw.w_gate, lw.w_up, lw.w_down)


def block_forward(x, lw: LayerWeights, cfg: Config, pos0: int = 0, return_parts: bool = False, key_mask=None,
                  layer: int = 0):
    """Pre-norm block: h = x + attn(norm1(x)); out = h + mlp(norm2(h)).

    nnterp SmolLM3, "The block, in order"; tohio block.py, SLMDecoderBlock.forward;
    abi96062 components.py, TransformerBlock.forward; Sualeh77 model.py,
    "6. Transformer Block". Positions are pos0 .. pos0+T-1; key_mask as in
    attention_sublayer.
    Returns out (and, with return_parts, a dict with attn, mlp, k, v)."""
    x = np.asarray(x, F64)
    T = x.shape[1]
    positions = np.arange(pos0, pos0 + T)
    attn, k, v = attention_sublayer(x, lw, cfg, positions, key_mask=key_mask, layer=layer)
    h = x + attn
    mlp = mlp_sublayer(h, lw, cfg)
    out = h + mlp
    if return_parts:
        return out, {"attn": attn, "mlp": mlp, "k": k, "v": v}
    return out


# ---------------------------------------------------------------- the model


def embed(ids: np.ndarray, E: np.ndarray) -> np.ndarray:
    """x[b, t, :] = E[ids[b, t], :] (abi96062 model.py, SmolLM2Model.forward)."""
    return np.asarray(E, F64)[np.asarray(ids)]


def lm_head(x: np.ndarray, final_norm, E, cfg: Config) -> np.ndarray:
    """logits = RMSNorm(x; f) E^T, with lm_head tied to the embedding
    (abi96062 model.py, weight tying; nnterp SmolLM3, "The readout ...")."""
    z = rms_norm(x, final_norm, cfg.rms_eps)
    return z @ np.asarray(E, F64).T


def model_prefill(ids, mw: ModelWeights, cfg: Config, logit_rows: Optional[Sequence[int]] = None, keep_cache: bool = False,
                  key_mask=None):
    """embed -> n_layers blocks -> final norm -> tied lm_head, positions 0..T-1.

    abi96062 model.py, SmolLM2Model.forward; Sualeh77 model.py, "7. Top-level".
    logit_rows, if given, selects the flattened rows (b*T + t) whose logits are
    returned (the head is row-wise, so this only skips outputs).
    key_mask: optional bool [B, T] padding mask over key positions (False: the key
    gets -inf added to its scores; Sualeh77 model.py, "4. Attention",
    attention_mask).
    Returns logits [B, T, V] (or [len(rows), V]) and, with keep_cache, the list of
    per-layer (k_rot, v) each [B, n_kv, T, d]."""
    ids = np.asarray(ids)
    B, T = ids.shape
    if T > cfg.max_pos:
        raise ValueError("sequence longer than max_position_embeddings")
    x = embed(ids, mw.embed)
    cache = []
    for li, lw in enumerate(mw.layers):
        x, parts = block_forward(x, lw, cfg, 0, return_parts=True, key_mask=key_mask, layer=li)
        if keep_cache:
            cache.append((parts["k"], parts["v"]))
    xf = x.reshape(B * T, cfg.hidden)
    if logit_rows is not None:
        xf = xf[np.asarray(logit_rows)]
        logits = lm_head(xf, mw.final_norm, mw.embed, cfg)
    else:
        logits = lm_head(xf, mw.final_norm, mw.embed, cfg).reshape(B, T, cfg.vocab)
    return (logits, cache) if keep_cache else logits


def decode_step(ids, cache_len: int, mw: ModelWeights, cfg: Config, k_cache, v_cache, key_mask=None):
    """One new token per sequence at position P = cache_len.

    k_cache / v_cache: per layer arrays [B, n_kv, >=P, d] holding keys after RoPE
    and values for positions 0..P-1. The new token's q, k are rotated at P, its
    k', v appended, and it attends over keys 0..P (Sualeh77 model.py, "7. Top-level"
    forward with past_key_values, and generate); key_mask, optional bool [B, >= P+1]
    over key positions, masks keys as in gqa_attention.
    Returns (logits [B, V], new_k [L][B, n_kv, d], new_v [L][B, n_kv, d])."""
    ids = np.asarray(ids).reshape(-1, 1)
    B = ids.shape[0]
    P = int(cache_len)
    if P + 1 > cfg.max_pos:
        raise ValueError("cache_len + 1 exceeds max_position_embeddings")
    x = embed(ids, mw.embed)  # [B, 1, H]
    positions = np.array([P])
    new_k, new_v = [], []
    for li, lw in enumerate(mw.layers):
        pk = np.asarray(k_cache[li])[:, :, :P]
        pv = np.asarray(v_cache[li])[:, :, :P]
        attn, k, v = attention_sublayer(x, lw, cfg, positions, pk, pv, np.arange(P), key_mask=key_mask, layer=li)
        h = x + attn
        x = h + mlp_sublayer(h, lw, cfg)
        new_k.append(k[:, :, 0])
        new_v.append(v[:, :, 0])
    logits = lm_head(x[:, 0], mw.final_norm, mw.embed, cfg)
    return logits, new_k, new_v
