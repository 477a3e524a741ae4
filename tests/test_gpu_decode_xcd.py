"""GPU tests aimed at the one-launch bf16 decode step (every layer in one persistent
launch, the batch partitioned over the eight XCDs: sequence b runs on XCD b % 8).

* Batches that leave XCD groups empty or give them one, two or three rows, with a
  different cache length per sequence (a split of the attention per row, windows of
  keys that differ per row), against the float64 oracle's decode of each sequence.
* The bounded barrier wait: with the limit forced down from the host every
  workgroup leaves through the abort path and the step's logits are NaN; the next
  call, with the normal limit, reproduces the clean result bit for bit.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.smol as O  # noqa: E402
from llama_decoder_only_amd import binding as B  # noqa: E402
from llama_decoder_only_amd import synthetic as S  # noqa: E402
from tests.gpu_helpers import TOL_BF16, ocfg, omodel, rel, say, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _setup(batch, cap, lens, n_layers=2):
    s = S.workload("decode_bf16", n_layers=n_layers, batch=batch)
    model = S.model_weights(s, 0)
    md = B.upload_model(model)
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
    return s, model, md, ks, vs, kc, vc, ids_np, ids, cl


def _decode(s, md, ids, cl, kc, vc):
    cfg = B.Config.from_shape(s)
    logits = torch.empty(ids.shape[0], s.vocab, dtype=torch.bfloat16, device=DEV)
    B.smol_decode_step(cfg, md, ids, cl, kc, vc, logits)
    torch.cuda.synchronize()
    return logits


@pytest.mark.parametrize("batch", [1, 9, 17, 24])
def test_one_launch_decode_odd_batches(batch):
    """batch 1 leaves seven XCD groups empty; 9, 17 and 24 give the groups one to three
    rows. Cache lengths differ per sequence, across the attention's split boundaries."""
    cap = 700
    rng = np.random.default_rng(batch)
    lens = [int(x) for x in rng.integers(0, cap, size=batch)]
    lens[0] = 653  # one long row in every batch
    say(f"one-launch decode batch {batch}, lens {lens[:6]}...")
    s, model, md, ks, vs, kc, vc, ids_np, ids, cl = _setup(batch, cap, lens)
    got = to_np(_decode(s, md, ids, cl, kc, vc))
    om, oc = omodel(model), ocfg(s)
    worst = 0.0
    for b_, P in enumerate(lens):
        kb = [k.f64[b_:b_ + 1, :, :P] for k in ks]
        vb = [v.f64[b_:b_ + 1, :, :P] for v in vs]
        want, nk, nv = O.decode_step(ids_np[b_:b_ + 1], P, om, oc, kb, vb)
        worst = max(worst, rel(got[b_:b_ + 1], want))
        assert rel(to_np(kc[1, b_, :, P]), nk[1][0]) <= TOL_BF16
        assert rel(to_np(vc[0, b_, :, P]), nv[0][0]) <= TOL_BF16
    say(f"worst rel = {worst:.3e}")
    assert worst <= TOL_BF16


def test_one_launch_decode_abort_path_then_recovers(monkeypatch):
    """A barrier limit of one clock tick: every workgroup times out or sees the abort
    word at its next barrier and leaves; all logits NaN. Then the normal limit again:
    the same result as a clean step, bit for bit (an aborted step can only have written
    the same k/v a clean step writes)."""
    batch, cap = 16, 300
    lens = [250 + b for b in range(batch)]
    s, model, md, ks, vs, kc, vc, ids_np, ids, cl = _setup(batch, cap, lens)
    say("one-launch decode, clean step")
    good = _decode(s, md, ids, cl, kc, vc)
    assert torch.isfinite(good.float()).all()
    say("one-launch decode, barrier limit 1 tick")
    monkeypatch.setenv("SMOL_DECODE_DEADLINE_TICKS", "1")
    bad = _decode(s, md, ids, cl, kc, vc)
    assert torch.isnan(bad.float()).all()
    monkeypatch.delenv("SMOL_DECODE_DEADLINE_TICKS")
    say("one-launch decode, normal limit again")
    again = _decode(s, md, ids, cl, kc, vc)
    assert torch.equal(again, good)
