"""Python binding of libsmol (include/smol.h): same names, argument marshalling only.

torch provides device memory and the stream; every step of the forward pass runs
in the library's HIP kernels. torch is imported before the library is opened so
that the process has one HIP runtime (torch's libamdhip64.so.7), which the
library then binds to by soname. There is no fallback: if libsmol.so is missing
or no GPU is present, the calls raise.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, asdict
from typing import List, Optional, Sequence

import numpy as np
import torch

# The in-tree library; SMOL_LIB_PATH names another build of the same sources (the
# host-sanitizer copy that build.py --sanitize-host writes, for the CPU ABI tests).
LIB_PATH = os.environ.get("SMOL_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmol.so")

SMOL_OK, SMOL_ERR_INVALID_ARG, SMOL_ERR_UNSUPPORTED, SMOL_ERR_WORKSPACE, SMOL_ERR_HIP = range(5)
SMOL_F32, SMOL_BF16 = 0, 1
SMOL_OP_BLOCK, SMOL_OP_PREFILL, SMOL_OP_DECODE = 0, 1, 2
KERNELS = ["embed", "rmsnorm", "qkv_rope", "attention", "o_proj", "gate_up", "down", "lm_head",
           "decode_attention", "decode_combine", "sample",
           "bw_gemm", "bw_attn_fwd", "bw_attn_dq", "bw_attn_dkdv", "bw_rows", "decode_step"]
EXPORTED = ["smol_workspace_size", "smol_block_forward", "smol_model_prefill", "smol_decode_step",
            "smol_model_prefill_ex", "smol_decode_step_ex", "smol_decode_step_static",
            "smol_sample", "smol_generate_workspace_size", "smol_generate",
            "smol_block_backward_workspace_size", "smol_block_backward",
            "smol_status_string", "smol_last_error", "smol_timing_begin", "smol_timing_end"]


class smol_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate",
                                              "n_layers", "vocab", "max_pos")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("no_rope_interval", ctypes.c_int32), ("sliding_window", ctypes.c_int32)]


LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


class smol_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class smol_layer_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class smol_model_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("layers", ctypes.POINTER(smol_layer_weights)),
                ("final_norm", ctypes.c_void_p)]


class SmolError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Open libsmol.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        cfgp = ctypes.POINTER(smol_config)
        L.smol_workspace_size.argtypes = [cfgp, i32, i32, i32, ctypes.POINTER(sz)]
        L.smol_block_forward.argtypes = [cfgp, ctypes.POINTER(smol_layer_weights), vp, vp, i32, i32, i32, vp, vp,
                                         i32, vp, sz, vp]
        L.smol_model_prefill.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, i32, i32, vp, vp, vp, i32,
                                         vp, sz, vp]
        L.smol_decode_step.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, vp, i32, vp, vp, i32, vp, vp,
                                       sz, vp]
        f32, i64 = ctypes.c_float, ctypes.c_int64
        L.smol_sample.argtypes = [vp, i32, i32, i32, i64, f32, i32, f32, vp, vp, vp]
        L.smol_generate_workspace_size.argtypes = [cfgp, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.smol_generate.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, vp, i32, i32, i32, f32, i32, f32,
                                    vp, vp, vp, vp, i32, vp, sz, vp]
        L.smol_model_prefill_ex.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, i32, i32, i32, vp, vp, vp,
                                            vp, i32, vp, sz, vp]
        L.smol_decode_step_ex.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, vp, i32, vp, vp, vp, i32,
                                          vp, vp, sz, vp]
        L.smol_decode_step_static.argtypes = [cfgp, ctypes.POINTER(smol_model_weights), vp, vp, i32, vp, vp, i32,
                                              vp, vp]
        L.smol_block_backward_workspace_size.argtypes = [cfgp, i32, i32, ctypes.POINTER(sz)]
        L.smol_block_backward.argtypes = [cfgp, ctypes.POINTER(smol_layer_weights), i32, vp, vp, i32, i32, i32, vp,
                                          vp, ctypes.POINTER(smol_layer_grads), i32, vp, sz, vp]
        L.smol_status_string.argtypes = [i32]
        L.smol_status_string.restype = ctypes.c_char_p
        L.smol_last_error.argtypes = []
        L.smol_last_error.restype = ctypes.c_char_p
        L.smol_timing_begin.argtypes = [i32, i32]
        L.smol_timing_end.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]
        for name in EXPORTED:
            if name not in ("smol_status_string", "smol_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ config


@dataclass(frozen=True)
class Config:
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
    dtype: str  # "f32" | "bf16"
    no_rope_interval: int = 0  # SmolLM3 NoPE blocks: (l + 1) % k == 0 has no rotary
    sliding_window: int = 0    # window of those blocks (0: none)

    @classmethod
    def from_shape(cls, s) -> "Config":
        """From a synthetic.Shape (or anything with the same attribute names)."""
        return cls(**{k: getattr(s, k) for k in cls.__dataclass_fields__ if hasattr(s, k)})

    def c(self) -> smol_config:
        d = asdict(self)
        d["dtype"] = SMOL_BF16 if self.dtype == "bf16" else SMOL_F32
        return smol_config(**d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# ------------------------------------------------------------------ marshalling


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int):
    if status != SMOL_OK:
        raise SmolError(status, f"{smol_status_string(status)}: {smol_last_error()}")


def smol_status_string(status: int) -> str:
    return lib().smol_status_string(status).decode()


def smol_last_error() -> str:
    return lib().smol_last_error().decode()


def smol_workspace_size(cfg: Config, op: int, batch: int, seq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().smol_workspace_size(ctypes.byref(cfg.c()), op, batch, seq, ctypes.byref(n)))
    return int(n.value)


def workspace(cfg: Config, op: int, batch: int, seq: int, device="cuda") -> torch.Tensor:
    """Device scratch of the size the library asks for (torch's allocator aligns to 512 B)."""
    return torch.empty(max(smol_workspace_size(cfg, op, batch, seq), 1), dtype=torch.uint8, device=device)


class LayerWeights:
    """One block's device weights plus the C struct pointing at them."""

    def __init__(self, tensors: Sequence[torch.Tensor]):
        self.tensors = list(tensors)
        self.c = smol_layer_weights(*[_ptr(t) for t in self.tensors])


class ModelWeights:
    """Device weights of the whole model plus the C structs pointing at them."""

    def __init__(self, embed: torch.Tensor, layers: List[LayerWeights], final_norm: torch.Tensor):
        self.embed, self.layers, self.final_norm = embed, layers, final_norm
        self._arr = (smol_layer_weights * len(layers))(*[lw.c for lw in layers])
        self.c = smol_model_weights(_ptr(embed), self._arr, _ptr(final_norm))


def to_device(t, device="cuda") -> torch.Tensor:
    """A synthetic.Tensor (float32 values or bfloat16 bit patterns) as a device tensor."""
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)


def upload_layer(layer, device="cuda") -> LayerWeights:
    return LayerWeights([to_device(t, device) for t in layer.tensors()])


def upload_model(model, device="cuda") -> ModelWeights:
    return ModelWeights(to_device(model.embed, device), [upload_layer(l, device) for l in model.layers],
                        to_device(model.final_norm, device))


# ------------------------------------------------------------------ entry points


def smol_block_forward(cfg: Config, w: LayerWeights, x_in: torch.Tensor, x_out: torch.Tensor, pos0: int = 0,
                       k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """x_in, x_out: float32 [B, T, H]; caches [B, n_kv, cap, d] in cfg's dtype or None."""
    B, T, _ = x_in.shape
    if ws is None:
        ws = workspace(cfg, SMOL_OP_BLOCK, B, T, x_in.device)
    cap = k_cache.shape[2] if k_cache is not None else 0
    _check(lib().smol_block_forward(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(x_in), _ptr(x_out), B, T, pos0,
                                    _ptr(k_cache), _ptr(v_cache), cap, _ptr(ws), ws.numel(), _stream(stream)))
    return x_out


def smol_model_prefill(cfg: Config, w: ModelWeights, ids: torch.Tensor, logits: torch.Tensor,
                       k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ids int32 [B, T]; logits [B, T, V] in cfg's dtype; caches [L, B, n_kv, cap, d] or None."""
    B, T = ids.shape
    if ws is None:
        ws = workspace(cfg, SMOL_OP_PREFILL, B, T, ids.device)
    cap = k_cache.shape[3] if k_cache is not None else 0
    _check(lib().smol_model_prefill(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(ids), B, T, _ptr(logits),
                                    _ptr(k_cache), _ptr(v_cache), cap, _ptr(ws), ws.numel(), _stream(stream)))
    return logits


def smol_decode_step(cfg: Config, w: ModelWeights, ids: torch.Tensor, cache_len: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, logits: torch.Tensor,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ids, cache_len int32 [B]; caches [L, B, n_kv, cap, d]; logits [B, V]."""
    B = ids.shape[0]
    cap = k_cache.shape[3]
    if ws is None:
        ws = workspace(cfg, SMOL_OP_DECODE, B, cap, ids.device)
    _check(lib().smol_decode_step(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(ids), _ptr(cache_len), B,
                                  _ptr(k_cache), _ptr(v_cache), cap, _ptr(logits), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return logits


def smol_decode_step_static(cfg: Config, w: ModelWeights, ids: torch.Tensor, cache_len: torch.Tensor,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, logits: torch.Tensor,
                            stream=None) -> torch.Tensor:
    """As smol_decode_step, on the library's fixed scratch (no workspace, no allocation)."""
    B = ids.shape[0]
    cap = k_cache.shape[3]
    _check(lib().smol_decode_step_static(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(ids), _ptr(cache_len), B,
                                         _ptr(k_cache), _ptr(v_cache), cap, _ptr(logits), _stream(stream)))
    return logits


def smol_sample(logits: torch.Tensor, next_ids: torch.Tensor, temperature: float = 0.0, top_k: int = 0,
                top_p: float = 1.0, uniforms: Optional[torch.Tensor] = None, row_offset: int = 0,
                row_stride: Optional[int] = None, stream=None) -> torch.Tensor:
    """logits [B, V] (or any rows: row b at element row_offset + b * row_stride), float32 or
    bfloat16; next_ids int32 [B] (written); uniforms float32 [B] in [0, 1) when sampling."""
    B = next_ids.shape[0]
    V = logits.shape[-1]
    if row_stride is None:
        row_stride = V
    if row_offset + (B - 1) * row_stride + V > logits.numel():
        raise ValueError("rows run past the logits tensor")
    dt = SMOL_BF16 if logits.dtype == torch.bfloat16 else SMOL_F32
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be float32 or bfloat16")
    base = _ptr(logits) + row_offset * logits.element_size()
    _check(lib().smol_sample(base, dt, B, V, row_stride, float(temperature), int(top_k), float(top_p), _ptr(uniforms),
                             _ptr(next_ids), _stream(stream)))
    return next_ids


def smol_generate_workspace_size(cfg: Config, batch: int, prompt_len: int, max_new: int, cache_cap: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().smol_generate_workspace_size(ctypes.byref(cfg.c()), batch, prompt_len, max_new, cache_cap,
                                              ctypes.byref(n)))
    return int(n.value)


def smol_generate(cfg: Config, w: ModelWeights, prompt_ids: torch.Tensor, max_new: int, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, out_ids: torch.Tensor, temperature: float = 0.0, top_k: int = 0,
                  top_p: float = 1.0, uniforms: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  stream=None, prompt_lens: Optional[torch.Tensor] = None) -> torch.Tensor:
    """prompt_ids int32 [B, T] (right-padded); prompt_lens int32 [B] or None; caches
    [L, B, n_kv, cap, d]; out_ids int32 [max_new, B] (written); uniforms float32
    [max_new, B] when temperature > 0."""
    B, T = prompt_ids.shape
    cap = k_cache.shape[3]
    if ws is None:
        ws = torch.empty(smol_generate_workspace_size(cfg, B, T, max_new, cap), dtype=torch.uint8,
                         device=prompt_ids.device)
    _check(lib().smol_generate(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(prompt_ids), _ptr(prompt_lens), B, T,
                               max_new,
                               float(temperature), int(top_k), float(top_p), _ptr(uniforms), _ptr(out_ids),
                               _ptr(k_cache), _ptr(v_cache), cap, _ptr(ws), ws.numel(), _stream(stream)))
    return out_ids


def trim_at_eos(out_ids: np.ndarray, eos_id: int) -> np.ndarray:
    """Tokens [max_new, B] cut after the first step at which every sequence's new token
    is eos_id (the stopping rule of Sualeh77 model.py, "7. Top-level", generate)."""
    for j in range(out_ids.shape[0]):
        if (out_ids[j] == eos_id).all():
            return out_ids[: j + 1]
    return out_ids


def smol_model_prefill_ex(cfg: Config, w: ModelWeights, ids: torch.Tensor, logits: torch.Tensor, pos0: int = 0,
                          key_mask: Optional[torch.Tensor] = None, k_cache: Optional[torch.Tensor] = None,
                          v_cache: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """ids int32 [B, T] at positions pos0 ..; key_mask uint8 [B, cap] (with caches) or [B, T]."""
    B, T = ids.shape
    if ws is None:
        ws = workspace(cfg, SMOL_OP_PREFILL, B, T, ids.device)
    cap = k_cache.shape[3] if k_cache is not None else 0
    if key_mask is not None and (key_mask.dtype != torch.uint8 or tuple(key_mask.shape) != (B, cap if k_cache is not None else T)):
        raise ValueError("key_mask must be uint8 [B, cache_cap] (with caches) or [B, seq]")
    _check(lib().smol_model_prefill_ex(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(ids), B, T, pos0,
                                       _ptr(key_mask), _ptr(logits), _ptr(k_cache), _ptr(v_cache), cap, _ptr(ws),
                                       ws.numel(), _stream(stream)))
    return logits


def smol_decode_step_ex(cfg: Config, w: ModelWeights, ids: torch.Tensor, cache_len: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, logits: torch.Tensor,
                        key_mask: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """As smol_decode_step, with key_mask uint8 [B, cap] (or None)."""
    B = ids.shape[0]
    cap = k_cache.shape[3]
    if key_mask is not None and (key_mask.dtype != torch.uint8 or tuple(key_mask.shape) != (B, cap)):
        raise ValueError("key_mask must be uint8 [B, cache_cap]")
    if ws is None:
        ws = workspace(cfg, SMOL_OP_DECODE, B, cap, ids.device)
    _check(lib().smol_decode_step_ex(ctypes.byref(cfg.c()), ctypes.byref(w.c), _ptr(ids), _ptr(cache_len), B,
                                     _ptr(key_mask), _ptr(k_cache), _ptr(v_cache), cap, _ptr(logits), _ptr(ws),
                                     ws.numel(), _stream(stream)))
    return logits


def smol_block_backward_workspace_size(cfg: Config, batch: int, seq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().smol_block_backward_workspace_size(ctypes.byref(cfg.c()), batch, seq, ctypes.byref(n)))
    return int(n.value)


class LayerGrads:
    """Float32 gradient buffers shaped like one block's weights, plus the C struct."""

    def __init__(self, tensors: Sequence[torch.Tensor]):
        self.tensors = list(tensors)
        for t in self.tensors:
            if t.dtype != torch.float32:
                raise ValueError("gradients are float32")
        self.c = smol_layer_grads(*[_ptr(t) for t in self.tensors])

    @classmethod
    def zeros_like(cls, w: LayerWeights) -> "LayerGrads":
        return cls([torch.zeros(t.shape, dtype=torch.float32, device=t.device) for t in w.tensors])

    def as_dict(self):
        return dict(zip(LAYER_FIELDS, self.tensors))


def smol_block_backward(cfg: Config, w: LayerWeights, x: torch.Tensor, dy: torch.Tensor, dx: torch.Tensor,
                        grads: LayerGrads, layer: int = 0, pos0: int = 0, key_mask: Optional[torch.Tensor] = None,
                        accumulate: bool = False, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """x, dy, dx float32 [B, T, H] (dx written); grads: LayerGrads (written, or added to
    with accumulate); key_mask uint8 [B, T] or None."""
    B, T, _ = x.shape
    if key_mask is not None and (key_mask.dtype != torch.uint8 or tuple(key_mask.shape) != (B, T)):
        raise ValueError("key_mask must be uint8 [B, seq]")
    if ws is None:
        ws = torch.empty(smol_block_backward_workspace_size(cfg, B, T), dtype=torch.uint8, device=x.device)
    _check(lib().smol_block_backward(ctypes.byref(cfg.c()), ctypes.byref(w.c), layer, _ptr(x), _ptr(dy), B, T, pos0,
                                     _ptr(key_mask), _ptr(dx), ctypes.byref(grads.c), int(bool(accumulate)),
                                     _ptr(ws), ws.numel(), _stream(stream)))
    return dx


def smol_timing_begin(kernel: str, max_launches: int):
    _check(lib().smol_timing_begin(KERNELS.index(kernel), max_launches))


def smol_timing_end():
    """Returns (summed milliseconds, launches timed)."""
    ms, n = ctypes.c_float(0), ctypes.c_int(0)
    _check(lib().smol_timing_end(ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
