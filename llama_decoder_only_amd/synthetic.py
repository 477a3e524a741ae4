"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module only draws random numbers and rounds them to the storage format; it
holds none of the forward pass's arithmetic, so both the HIP path and the CPU
oracle can consume its arrays without sharing any computation.

Every tensor comes from its own stream
``Generator(PCG64(SeedSequence([seed, workload_id, layer, tensor_id])))``:
normals are drawn in float64, scaled by the std, rounded to float32 (round to
nearest even) and, for bfloat16 workloads, rounded again to bfloat16 (round to
nearest even). The oracle gets the exact stored values upcast to float64.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

# tensor ids of the seed tree
T_EMBED, T_WQ, T_WK, T_WV, T_WO, T_WG, T_WU, T_WD = 0, 1, 2, 3, 4, 5, 6, 7
T_ATTN_NORM, T_MLP_NORM, T_FINAL_NORM = 8, 9, 10
T_HIDDEN, T_IDS, T_KCACHE, T_VCACHE, T_DECODE_IDS, T_DY = 100, 101, 102, 103, 104, 105


@dataclass(frozen=True)
class Shape:
    """Dimensions of a LLaMA-style decoder plus the workload around it."""

    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    n_layers: int
    vocab: int
    max_pos: int
    rms_eps: float
    rope_theta: float
    dtype: str  # "f32" or "bf16"
    batch: int
    seq: int
    std: float
    workload_id: int
    cache_len: int = 0  # decode: positions already in the cache
    norm_jitter: float = 0.0  # >0: RMSNorm weights 1 + N(0, jitter^2) instead of 1
    no_rope_interval: int = 0  # SmolLM3 variants: NoPE on blocks (l + 1) % k == 0
    sliding_window: int = 0    # and a window on those blocks


SMOLLM2 = dict(hidden=576, n_heads=9, n_kv_heads=3, head_dim=64, intermediate=1536, n_layers=30,
               vocab=49152, max_pos=8192, rms_eps=1e-5, rope_theta=100000.0)
SMOLLM3_SHAPE = dict(hidden=2048, n_heads=16, n_kv_heads=4, head_dim=128, intermediate=11008, n_layers=36,
                     vocab=128256, max_pos=65536, rms_eps=1e-6, rope_theta=100000.0)
INIT_STD = 1.0 / 24.0  # the SmolLM2 config's initializer_range

WORKLOADS: Dict[str, Shape] = {
    # one block in float32 at batch 1, seq 128
    "block_f32": Shape(**{**SMOLLM2, "n_layers": 1}, dtype="f32", batch=1, seq=128, std=INIT_STD, workload_id=1),
    # the whole 30-layer model in float32 at the same size (bit-exact argmax check)
    "model_f32": Shape(**SMOLLM2, dtype="f32", batch=1, seq=128, std=INIT_STD, workload_id=11),
    # SmolLM2-135M prefill, bfloat16, batch 4 x seq 512
    "prefill_bf16": Shape(**SMOLLM2, dtype="bf16", batch=4, seq=512, std=INIT_STD, workload_id=2),
    # long-context prefill, bfloat16, batch 1 x seq 8192
    "long_prefill_bf16": Shape(**SMOLLM2, dtype="bf16", batch=1, seq=8192, std=INIT_STD, workload_id=3),
    # decode: batch 64, 2047 cached positions, one new token each
    "decode_bf16": Shape(**SMOLLM2, dtype="bf16", batch=64, seq=1, std=INIT_STD, workload_id=4, cache_len=2047),
    # backward of one SmolLM2-135M block in float32 at the prefill's batch 4 x seq 512
    "block_backward_f32": Shape(**{**SMOLLM2, "n_layers": 1}, dtype="f32", batch=4, seq=512, std=INIT_STD,
                                workload_id=6, norm_jitter=0.1),
    # SmolLM3-3B-shaped prefill, bfloat16, batch 2 x seq 4096
    "smollm3_prefill_bf16": Shape(**SMOLLM3_SHAPE, dtype="bf16", batch=2, seq=4096, std=0.02, workload_id=5),
}


def workload(name: str, **overrides) -> Shape:
    return replace(WORKLOADS[name], **overrides)


# ------------------------------------------------------------------ storage


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """A stored tensor: ``data`` is what the device receives (float32 values or
    bfloat16 bit patterns as uint16); ``f64`` gives the exact values in float64."""

    data: np.ndarray
    dtype: str

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    @property
    def shape(self):
        return self.data.shape


def _rng(s: Shape, seed: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, s.workload_id, layer, tensor_id])))


def _store(x64: np.ndarray, dtype: str) -> Tensor:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x32), "bf16")
    return Tensor(x32, "f32")


def stored(x64: np.ndarray, dtype: str) -> Tensor:
    """Values rounded to a storage format ("f32" or "bf16"), e.g. a test's edited copy
    of a drawn tensor."""
    return _store(np.asarray(x64, np.float64), dtype)


def normal(s: Shape, seed: int, layer: int, tensor_id: int, shape, std: float) -> Tensor:
    x = _rng(s, seed, layer, tensor_id).standard_normal(size=shape) * std
    return _store(x, s.dtype)


def norm_weight(s: Shape, seed: int, layer: int, tensor_id: int) -> Tensor:
    if s.norm_jitter > 0:
        x = 1.0 + _rng(s, seed, layer, tensor_id).standard_normal(size=(s.hidden,)) * s.norm_jitter
    else:
        x = np.ones(s.hidden)
    return _store(x, s.dtype)


# ------------------------------------------------------------------ weights


@dataclass
class Layer:
    attn_norm: Tensor
    wq: Tensor
    wk: Tensor
    wv: Tensor
    wo: Tensor
    mlp_norm: Tensor
    w_gate: Tensor
    w_up: Tensor
    w_down: Tensor

    NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")

    def tensors(self) -> List[Tensor]:
        return [getattr(self, n) for n in self.NAMES]


def layer_weights(s: Shape, seed: int, layer: int) -> Layer:
    H, I, d = s.hidden, s.intermediate, s.head_dim
    nq, nkv = s.n_heads * d, s.n_kv_heads * d
    return Layer(
        attn_norm=norm_weight(s, seed, layer, T_ATTN_NORM),
        wq=normal(s, seed, layer, T_WQ, (nq, H), s.std),
        wk=normal(s, seed, layer, T_WK, (nkv, H), s.std),
        wv=normal(s, seed, layer, T_WV, (nkv, H), s.std),
        wo=normal(s, seed, layer, T_WO, (H, nq), s.std),
        mlp_norm=norm_weight(s, seed, layer, T_MLP_NORM),
        w_gate=normal(s, seed, layer, T_WG, (I, H), s.std),
        w_up=normal(s, seed, layer, T_WU, (I, H), s.std),
        w_down=normal(s, seed, layer, T_WD, (H, I), s.std),
    )


@dataclass
class Model:
    embed: Tensor
    layers: List[Layer] = field(default_factory=list)
    final_norm: Optional[Tensor] = None


def model_weights(s: Shape, seed: int = 0) -> Model:
    return Model(
        embed=normal(s, seed, 0, T_EMBED, (s.vocab, s.hidden), s.std),
        layers=[layer_weights(s, seed, i) for i in range(s.n_layers)],
        final_norm=norm_weight(s, seed, 0, T_FINAL_NORM),
    )


# ------------------------------------------------------------------ activations


def hidden_states(s: Shape, seed: int = 0) -> Tensor:
    """Block input [B, T, H] ~ N(0, 1)."""
    return normal(s, seed, 0, T_HIDDEN, (s.batch, s.seq, s.hidden), 1.0)


def output_grad(s: Shape, seed: int = 0) -> Tensor:
    """Gradient arriving at a block's output [B, T, H] ~ N(0, 1), float32."""
    x = _rng(s, seed, 0, T_DY).standard_normal(size=(s.batch, s.seq, s.hidden))
    return _store(x, "f32")


def token_ids(s: Shape, seed: int = 0, tensor_id: int = T_IDS) -> np.ndarray:
    """Token ids uniform in [0, vocab), int32 [B, T]."""
    return _rng(s, seed, 0, tensor_id).integers(0, s.vocab, size=(s.batch, s.seq), dtype=np.int32)


def kv_cache_values(s: Shape, seed: int, layer: int, cap: int) -> tuple:
    """Cache contents ~ N(0, 1) for one layer: (K, V) each [B, n_kv, cap, d]; the
    first cache_len positions are the meaningful ones."""
    shape = (s.batch, s.n_kv_heads, cap, s.head_dim)
    return (normal(s, seed, layer, T_KCACHE, shape, 1.0), normal(s, seed, layer, T_VCACHE, shape, 1.0))
