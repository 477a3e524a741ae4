"""The C ABI on the CPU: the library loads, exports every symbol include/smol.h
declares, sizes workspaces, and rejects bad arguments before touching the GPU.

No call here reaches a kernel: each one fails a host-side check first (fake,
never-dereferenced pointers stand in for device buffers)."""

import ctypes
import os
import re

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "smol.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smol_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    declared = _declared_symbols()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(B.EXPORTED) == declared


def test_status_strings():
    assert B.smol_status_string(0) == "ok"
    assert "workspace" in B.smol_status_string(3)
    assert B.smol_status_string(99) == "unknown status"


def _cfg(**kw):
    c = B.Config.from_shape(S.workload("prefill_bf16"))
    d = {k: getattr(c, k) for k in c.__dataclass_fields__}
    d.update(kw)
    return B.Config(**d)


def _ws(cfg, op, b, t):
    n = ctypes.c_size_t(0)
    st = B.lib().smol_workspace_size(ctypes.byref(cfg.c()), op, b, t, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    cfg = _cfg()
    st, n1 = _ws(cfg, B.SMOL_OP_PREFILL, 4, 512)
    assert st == 0 and n1 > 4 * 512 * 576 * 4
    st, n2 = _ws(cfg, B.SMOL_OP_PREFILL, 8, 512)
    assert st == 0 and n2 > n1
    st, n3 = _ws(cfg, B.SMOL_OP_DECODE, 64, 2048)
    assert st == 0 and n3 > 0
    st, _ = _ws(cfg, 7, 1, 1)
    assert st == B.SMOL_ERR_INVALID_ARG
    st, _ = _ws(cfg, B.SMOL_OP_BLOCK, 0, 1)
    assert st == B.SMOL_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=577), B.SMOL_ERR_INVALID_ARG),              # hidden != heads * head_dim
    (dict(n_kv_heads=2), B.SMOL_ERR_INVALID_ARG),            # 9 % 2 != 0
    (dict(n_kv_heads=1), B.SMOL_ERR_UNSUPPORTED),            # 9 q heads per kv head
    (dict(head_dim=32, n_heads=18, n_kv_heads=6), B.SMOL_ERR_UNSUPPORTED),
    (dict(intermediate=1500), B.SMOL_ERR_UNSUPPORTED),
    (dict(vocab=49153), B.SMOL_ERR_UNSUPPORTED),
    (dict(rms_eps=-1.0), B.SMOL_ERR_INVALID_ARG),
    (dict(rope_theta=0.0), B.SMOL_ERR_INVALID_ARG),
    (dict(n_layers=0), B.SMOL_ERR_INVALID_ARG),
])
def test_config_checks(kw, status):
    st, _ = _ws(_cfg(**kw), B.SMOL_OP_PREFILL, 1, 8)
    assert st == status, B.smol_last_error()
    assert B.smol_last_error() != ""


def _layer_struct(null=None):
    return B.smol_layer_weights(*[None if n == null else FAKE for n in B.LAYER_FIELDS])


def _block(cfg, w, x_in=FAKE, x_out=FAKE, batch=1, seq=8, pos0=0, kc=None, vc=None, cap=0, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = _ws(cfg, B.SMOL_OP_BLOCK, max(batch, 1), max(seq, 1))[1]
    return B.lib().smol_block_forward(ctypes.byref(cfg.c()), ctypes.byref(w), x_in, x_out, batch, seq, pos0, kc, vc,
                                      cap, ws, ws_bytes, None)


def test_block_forward_rejects():
    cfg = _cfg()
    w = _layer_struct()
    assert _block(cfg, _layer_struct(null="wk")) == B.SMOL_ERR_INVALID_ARG and "wk" in B.smol_last_error()
    assert _block(cfg, w, x_in=None) == B.SMOL_ERR_INVALID_ARG
    assert _block(cfg, w, batch=0) == B.SMOL_ERR_INVALID_ARG
    assert _block(cfg, w, seq=8193) == B.SMOL_ERR_INVALID_ARG and "max_pos" in B.smol_last_error()
    assert _block(cfg, w, pos0=8190, seq=8) == B.SMOL_ERR_INVALID_ARG
    assert _block(cfg, w, pos0=-1) == B.SMOL_ERR_INVALID_ARG
    assert _block(cfg, w, kc=FAKE, vc=None, cap=16) == B.SMOL_ERR_INVALID_ARG
    assert _block(cfg, w, kc=FAKE, vc=FAKE, cap=4, seq=8) == B.SMOL_ERR_INVALID_ARG and "cache_cap" in B.smol_last_error()
    need = _ws(cfg, B.SMOL_OP_BLOCK, 1, 8)[1]
    assert _block(cfg, w, ws_bytes=need - 1) == B.SMOL_ERR_WORKSPACE
    assert _block(cfg, w, ws=FAKE + 8) == B.SMOL_ERR_INVALID_ARG and "aligned" in B.smol_last_error()
    assert _block(cfg, w, ws=None) == B.SMOL_ERR_INVALID_ARG
    # rows move in 16-byte vectors: every buffer of rows must be 16-byte aligned
    assert _block(cfg, w, x_in=FAKE + 8) == B.SMOL_ERR_INVALID_ARG and "x_in" in B.smol_last_error()
    assert _block(cfg, w, x_out=FAKE + 4) == B.SMOL_ERR_INVALID_ARG and "x_out" in B.smol_last_error()
    assert _block(cfg, w, kc=FAKE + 2, vc=FAKE, cap=16) == B.SMOL_ERR_INVALID_ARG
    assert "k_cache" in B.smol_last_error() and "aligned" in B.smol_last_error()
    odd = B.smol_layer_weights(*[FAKE + 8 if n == "w_up" else FAKE for n in B.LAYER_FIELDS])
    assert _block(cfg, odd) == B.SMOL_ERR_INVALID_ARG and "w_up must be 16-byte aligned" in B.smol_last_error()
    assert B.lib().smol_block_forward(None, ctypes.byref(w), FAKE, FAKE, 1, 8, 0, None, None, 0, FAKE, need,
                                      None) == B.SMOL_ERR_INVALID_ARG


def _model_struct(cfg, null_layer=None):
    layers = (B.smol_layer_weights * cfg.n_layers)(
        *[_layer_struct(null="w_down" if i == null_layer else None) for i in range(cfg.n_layers)])
    m = B.smol_model_weights(FAKE, layers, FAKE)
    return m, layers


def test_model_prefill_rejects():
    cfg = _cfg()
    m, keep = _model_struct(cfg)
    need = _ws(cfg, B.SMOL_OP_PREFILL, 2, 16)[1]
    call = lambda **k: B.lib().smol_model_prefill(  # noqa: E731
        ctypes.byref(cfg.c()), ctypes.byref(k.get("m", m)), k.get("ids", FAKE), k.get("b", 2), k.get("t", 16),
        k.get("logits", FAKE), k.get("kc"), k.get("vc"), k.get("cap", 0), FAKE, k.get("ws_bytes", need), None)
    assert call(ids=None) == B.SMOL_ERR_INVALID_ARG
    assert call(logits=None) == B.SMOL_ERR_INVALID_ARG
    assert call(t=0) == B.SMOL_ERR_INVALID_ARG
    assert call(t=9000) == B.SMOL_ERR_INVALID_ARG
    assert call(kc=FAKE, vc=FAKE, cap=8) == B.SMOL_ERR_INVALID_ARG
    assert call(ws_bytes=need // 2) == B.SMOL_ERR_WORKSPACE
    m2, keep2 = _model_struct(cfg, null_layer=17)
    assert call(m=m2) == B.SMOL_ERR_INVALID_ARG and "layer 17" in B.smol_last_error()
    m3 = B.smol_model_weights(None, keep, FAKE)
    assert call(m=m3) == B.SMOL_ERR_INVALID_ARG and "embed" in B.smol_last_error()
    m4 = B.smol_model_weights(FAKE + 8, keep, FAKE)
    assert call(m=m4) == B.SMOL_ERR_INVALID_ARG and "embed must be 16-byte aligned" in B.smol_last_error()
    m5 = B.smol_model_weights(FAKE, keep, FAKE + 2)
    assert call(m=m5) == B.SMOL_ERR_INVALID_ARG and "final_norm" in B.smol_last_error()
    assert call(logits=FAKE + 2) == B.SMOL_ERR_INVALID_ARG and "logits" in B.smol_last_error()
    assert call(kc=FAKE, vc=FAKE + 8, cap=64) == B.SMOL_ERR_INVALID_ARG and "v_cache" in B.smol_last_error()


def test_decode_step_rejects():
    cfg = _cfg()
    m, keep = _model_struct(cfg)
    need = _ws(cfg, B.SMOL_OP_DECODE, 64, 2048)[1]
    call = lambda **k: B.lib().smol_decode_step(  # noqa: E731
        ctypes.byref(cfg.c()), ctypes.byref(m), k.get("ids", FAKE), k.get("cl", FAKE), k.get("b", 64),
        k.get("kc", FAKE), k.get("vc", FAKE), k.get("cap", 2048), FAKE, FAKE, k.get("ws_bytes", need), None)
    assert call(cl=None) == B.SMOL_ERR_INVALID_ARG
    assert call(kc=None) == B.SMOL_ERR_INVALID_ARG
    assert call(b=0) == B.SMOL_ERR_INVALID_ARG
    assert call(cap=0) == B.SMOL_ERR_INVALID_ARG
    assert call(ws_bytes=need - 256) == B.SMOL_ERR_WORKSPACE
    assert call(kc=FAKE + 8) == B.SMOL_ERR_INVALID_ARG and "k_cache" in B.smol_last_error()


def test_decode_step_static_rejects():
    """The no-workspace decode step checks its arguments like smol_decode_step and turns
    a request larger than its fixed scratch into SMOL_ERR_WORKSPACE, before any GPU call."""
    cfg = _cfg()
    m, keep = _model_struct(cfg)
    call = lambda **k: B.lib().smol_decode_step_static(  # noqa: E731
        ctypes.byref(cfg.c()), ctypes.byref(m), k.get("ids", FAKE), k.get("cl", FAKE), k.get("b", 64),
        k.get("kc", FAKE), k.get("vc", FAKE), k.get("cap", 2048), k.get("logits", FAKE), None)
    assert call(ids=None) == B.SMOL_ERR_INVALID_ARG
    assert call(cl=None) == B.SMOL_ERR_INVALID_ARG
    assert call(logits=None) == B.SMOL_ERR_INVALID_ARG
    assert call(kc=None) == B.SMOL_ERR_INVALID_ARG
    assert call(b=0) == B.SMOL_ERR_INVALID_ARG
    assert call(cap=0) == B.SMOL_ERR_INVALID_ARG
    assert call(logits=FAKE + 2) == B.SMOL_ERR_INVALID_ARG and "logits" in B.smol_last_error()
    big = 1 << 14  # batch whose decode workspace passes the fixed scratch
    assert _ws(cfg, B.SMOL_OP_DECODE, big, 2048)[1] > (32 << 20)
    assert call(b=big) == B.SMOL_ERR_WORKSPACE and "scratch" in B.smol_last_error()


def test_sample_rejects():
    L = B.lib()
    call = lambda **k: L.smol_sample(  # noqa: E731
        k.get("logits", FAKE), k.get("dt", B.SMOL_BF16), k.get("b", 4), k.get("v", 49152), k.get("stride", 49152),
        k.get("t", 1.0), k.get("k", 0), k.get("p", 1.0), k.get("u", FAKE), k.get("out", FAKE), None)
    assert call(logits=None) == B.SMOL_ERR_INVALID_ARG
    assert call(out=None) == B.SMOL_ERR_INVALID_ARG
    assert call(dt=7) == B.SMOL_ERR_INVALID_ARG
    assert call(b=0) == B.SMOL_ERR_INVALID_ARG
    assert call(v=0) == B.SMOL_ERR_INVALID_ARG
    assert call(stride=100) == B.SMOL_ERR_INVALID_ARG and "row_stride" in B.smol_last_error()
    assert call(t=-1.0) == B.SMOL_ERR_INVALID_ARG
    assert call(t=float("nan")) == B.SMOL_ERR_INVALID_ARG
    assert call(t=float("inf")) == B.SMOL_ERR_INVALID_ARG
    assert call(p=float("nan")) == B.SMOL_ERR_INVALID_ARG
    assert call(k=-1) == B.SMOL_ERR_INVALID_ARG
    assert call(u=None) == B.SMOL_ERR_INVALID_ARG and "uniforms" in B.smol_last_error()


def test_generate_rejects():
    cfg = _cfg()
    m, keep = _model_struct(cfg)
    L = B.lib()
    n = ctypes.c_size_t(0)
    assert L.smol_generate_workspace_size(ctypes.byref(cfg.c()), 4, 16, 8, 64, ctypes.byref(n)) == 0
    need = n.value
    assert need >= _ws(cfg, B.SMOL_OP_PREFILL, 4, 16)[1] and need >= _ws(cfg, B.SMOL_OP_DECODE, 4, 64)[1]
    assert L.smol_generate_workspace_size(ctypes.byref(cfg.c()), 4, 0, 8, 64, ctypes.byref(n)) == B.SMOL_ERR_INVALID_ARG
    call = lambda **k: L.smol_generate(  # noqa: E731
        ctypes.byref(cfg.c()), ctypes.byref(m), k.get("ids", FAKE), None, 4, k.get("t", 16), k.get("n", 8),
        k.get("temp", 0.0), 0, 1.0, k.get("u", None), k.get("out", FAKE), k.get("kc", FAKE), FAKE,
        k.get("cap", 64), FAKE, k.get("ws_bytes", need), None)
    assert call(ids=None) == B.SMOL_ERR_INVALID_ARG
    assert call(out=None) == B.SMOL_ERR_INVALID_ARG
    assert call(kc=None) == B.SMOL_ERR_INVALID_ARG
    assert call(n=0) == B.SMOL_ERR_INVALID_ARG
    assert call(t=60, n=6) == B.SMOL_ERR_INVALID_ARG and "cache_cap" in B.smol_last_error()  # 60 + 6 - 1 > 64
    assert call(temp=0.7) == B.SMOL_ERR_INVALID_ARG and "uniforms" in B.smol_last_error()
    assert call(ws_bytes=need - 256) == B.SMOL_ERR_WORKSPACE
    assert call(kc=FAKE + 4) == B.SMOL_ERR_INVALID_ARG and "k_cache" in B.smol_last_error()
    cfg8 = _cfg(max_pos=20)
    assert L.smol_generate(ctypes.byref(cfg8.c()), ctypes.byref(m), FAKE, None, 4, 16, 8, 0.0, 0, 1.0, None, FAKE,
                           FAKE, FAKE, 64, FAKE, need, None) == B.SMOL_ERR_INVALID_ARG
    assert "max_pos" in B.smol_last_error()


def test_prefill_ex_rejects():
    cfg = _cfg()
    m, keep = _model_struct(cfg)
    need = _ws(cfg, B.SMOL_OP_PREFILL, 2, 16)[1]
    call = lambda **k: B.lib().smol_model_prefill_ex(  # noqa: E731
        ctypes.byref(cfg.c()), ctypes.byref(m), FAKE, 2, 16, k.get("pos0", 0), k.get("mask", None), FAKE,
        k.get("kc", FAKE), k.get("vc", FAKE), k.get("cap", 64), FAKE, need, None)
    assert call(pos0=-1) == B.SMOL_ERR_INVALID_ARG
    assert call(pos0=8, kc=None, vc=None, cap=0) == B.SMOL_ERR_INVALID_ARG and "pos0" in B.smol_last_error()
    assert call(pos0=50) == B.SMOL_ERR_INVALID_ARG and "cache_cap" in B.smol_last_error()  # 50 + 16 > 64
    assert call(pos0=8190, cap=9000) == B.SMOL_ERR_INVALID_ARG and "max_pos" in B.smol_last_error()
    assert call(kc=None) == B.SMOL_ERR_INVALID_ARG  # one cache without the other


def _grads_struct(null=None):
    return B.smol_layer_grads(*[None if n == null else FAKE for n in B.LAYER_FIELDS])


def _backward(cfg, w, g=None, layer=0, x=FAKE, dy=FAKE + 4096, dx=FAKE + 8192, batch=1, seq=8, pos0=0, acc=0,
              ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        n = ctypes.c_size_t(0)
        assert B.lib().smol_block_backward_workspace_size(ctypes.byref(cfg.c()), batch if batch > 0 else 1,
                                                          seq if seq > 0 else 1, ctypes.byref(n)) == 0
        ws_bytes = n.value
    g = _grads_struct() if g is None else g
    return B.lib().smol_block_backward(ctypes.byref(cfg.c()), ctypes.byref(w), layer, x, dy, batch, seq, pos0, None,
                                       dx, ctypes.byref(g), acc, ws, ws_bytes, None)


def test_block_backward_rejects():
    f32 = _cfg(dtype="f32")
    w = _layer_struct()
    n = ctypes.c_size_t(0)
    assert B.lib().smol_block_backward_workspace_size(ctypes.byref(f32.c()), 4, 512, ctypes.byref(n)) == 0
    assert n.value > 4 * 512 * (576 * 8 + 1536 * 5) * 4
    bf = _cfg()  # a bf16 config: accepted, its weights must be 16-byte aligned
    nb, nf = ctypes.c_size_t(0), ctypes.c_size_t(0)
    B.lib().smol_block_backward_workspace_size(ctypes.byref(bf.c()), 1, 8, ctypes.byref(nb))
    B.lib().smol_block_backward_workspace_size(ctypes.byref(f32.c()), 1, 8, ctypes.byref(nf))
    assert nb.value > nf.value  # room for the widened weights
    odd = B.smol_layer_weights(*[FAKE + 8 if n == "wq" else FAKE for n in B.LAYER_FIELDS])
    assert _backward(bf, odd) == B.SMOL_ERR_INVALID_ARG and "aligned" in B.smol_last_error()
    assert _backward(f32, _layer_struct(null="wo")) == B.SMOL_ERR_INVALID_ARG and "wo" in B.smol_last_error()
    assert _backward(f32, w, g=_grads_struct(null="w_up")) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, layer=30) == B.SMOL_ERR_INVALID_ARG and "layer" in B.smol_last_error()
    assert _backward(f32, w, layer=-1) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, x=None) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, dx=FAKE) == B.SMOL_ERR_INVALID_ARG and "alias" in B.smol_last_error()
    assert _backward(f32, w, dx=FAKE + 8196) == B.SMOL_ERR_INVALID_ARG and "aligned" in B.smol_last_error()
    assert _backward(f32, w, acc=2) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, batch=0) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, pos0=8190, seq=8) == B.SMOL_ERR_INVALID_ARG and "max_pos" in B.smol_last_error()
    assert _backward(f32, w, pos0=-2) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, ws=None) == B.SMOL_ERR_INVALID_ARG
    assert _backward(f32, w, ws=FAKE + 64) == B.SMOL_ERR_INVALID_ARG and "aligned" in B.smol_last_error()
    need = ctypes.c_size_t(0)
    B.lib().smol_block_backward_workspace_size(ctypes.byref(f32.c()), 1, 8, ctypes.byref(need))
    assert _backward(f32, w, ws_bytes=need.value - 1) == B.SMOL_ERR_WORKSPACE
    assert B.lib().smol_block_backward(None, ctypes.byref(w), 0, FAKE, FAKE, 1, 8, 0, None, FAKE, None, 0, FAKE,
                                       need.value, None) == B.SMOL_ERR_INVALID_ARG


def test_trim_at_eos():
    out = np.array([[1, 2], [0, 3], [0, 0], [5, 0]])
    assert B.trim_at_eos(out, 0).shape[0] == 3      # step 2: every sequence's new token is eos
    assert B.trim_at_eos(out, 9).shape[0] == 4      # never
    assert B.trim_at_eos(out[:1], 1).shape[0] == 1  # not all rows


def test_timing_rejects():
    L = B.lib()
    assert L.smol_timing_begin(-1, 4) == B.SMOL_ERR_INVALID_ARG
    assert L.smol_timing_begin(3, 0) == B.SMOL_ERR_INVALID_ARG
    assert L.smol_timing_end(None, None) == B.SMOL_ERR_INVALID_ARG


def test_product_path_does_not_import_the_oracle():
    """The binding and the package never reach oracle/ (it is test infrastructure)."""
    pkg = os.path.join(ROOT, "llama_decoder_only_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text and "#include \"oracle" not in text, f
