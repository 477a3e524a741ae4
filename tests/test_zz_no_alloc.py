"""smol_decode_step_static, the decode step that takes no workspace and allocates
nothing (its scratch is a fixed device array inside the library), against
smol_decode_step with a workspace, through the C ABI: two calls in a row, the second
with a smaller batch and other cache lengths, each compared element by element (the
same kernels run on the same inputs, so logits and the appended k/v must be
bit-identical) and against the float64 oracle at the bf16 bar."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

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


def _case(s, md, model, batch, cap, lens, seed, tol):
    cfg = B.Config.from_shape(s)
    L, nkv, d = s.n_layers, s.n_kv_heads, s.head_dim
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    kc = torch.randn(L, batch, nkv, cap, d, generator=gen, device=DEV).to(cfg.torch_dtype)
    vc = torch.randn(kc.shape, generator=gen, device=DEV).to(cfg.torch_dtype)
    ids = torch.randint(0, s.vocab, (batch,), generator=gen, device=DEV, dtype=torch.int32)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kc2, vc2 = kc.clone(), vc.clone()
    want = torch.empty(batch, s.vocab, dtype=cfg.torch_dtype, device=DEV)
    got = torch.full_like(want, float("nan"))
    B.smol_decode_step(cfg, md, ids, cl, kc, vc, want)
    B.smol_decode_step_static(cfg, md, ids, cl, kc2, vc2, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "logits differ from the workspace call"
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc), "caches differ from the workspace call"
    # and the oracle, for two sequences
    for b in (0, batch - 1):
        P = lens[b]
        kcb = [to_np(kc[l, b:b + 1, :, :P]) for l in range(L)]
        vcb = [to_np(vc[l, b:b + 1, :, :P]) for l in range(L)]
        lo, _, _ = O.decode_step(np.array([int(ids[b])]), P, omodel(model), ocfg(s), kcb, vcb)
        r = rel(to_np(got[b:b + 1]), lo)
        say(f"batch {batch}, sequence {b} at position {P}: rel {r:.3e}")
        assert r <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_decode_equals_workspace_decode_twice(dtype):
    s = S.workload("decode_bf16", n_layers=3, norm_jitter=0.1, dtype=dtype)
    say(f"static-scratch decode, {dtype}, 3 layers: batch 64 then batch 24")
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    _case(s, md, model, 64, 700, [699 - (7 * b) % 300 for b in range(64)], 1, tol)
    _case(s, md, model, 24, 300, [1 + (37 * b) % 299 for b in range(24)], 2, tol)
