"""GPU parity of one-hot draft verification (q_j = point mass at x_j) with the
oracle's one-hot mode: acceptance with probability p(x), replacement from p
without x, no draft logits read (the draft pointer is NULL)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Workload("onehot", B=6, K=4, V=1024, dtype=synth.F32, target_kind=0, target_scale=2.0,
                      sigma_first=0.4, sigma_last=0.8, temperature=1.0, seed=61, draft_mode=1)


def _run(name, w, prob=None, derived=False):
    from draft_verification_amd import device as D
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature} mode={w.length_mode}",
          flush=True)
    prob = prob or synth.make_problem(w)
    assert prob.draft is None
    dp = D.from_problem(prob)
    res = D.run_once(dp)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, res, orc, dtype=w.dtype, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    assert np.isnan(res["lse_draft"]).all()          # not written in one-hot mode
    # rows streamed: target rows only
    assert (res["rows_read"] <= w.K + 1).all()
    return res, orc, rep


@pytest.mark.parametrize("V", [1, 2, 255, 257, 16384, 16385, 40000])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_vocab_sweep(V, dtype):
    _run(f"one-hot V={V} dt={dtype}", BASE.with_(V=V, dtype=dtype, B=5, K=3, seed=3000 + V + dtype))


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_temperatures_and_ragged_lengths(T):
    w = BASE.with_(B=40, K=6, V=5000, temperature=T, dtype=synth.BF16, seed=62)
    prob = synth.make_problem(w)
    prob.verify_len = np.random.default_rng(62).integers(0, 7, size=40).astype(np.int32)
    _run(f"one-hot T={T} ragged", w, prob=prob)


def test_derived_confidence_is_one():
    w = BASE.with_(B=24, K=5, V=3000, length_mode=synth.LEN_TAU, tau_choices=(0.0, 0.5, 1.0, 1.5), seed=63)
    res, orc, _ = _run("one-hot tau", w, derived=True)
    np.testing.assert_array_equal(res["verify_len_out"], orc.verify_len)
    tau = synth.make_problem(w).tau
    np.testing.assert_array_equal(res["verify_len_out"], np.where(tau <= 1.0, w.K, 0))
    assert (res["survival"] == 1.0).all()


@pytest.mark.parametrize("name", ["zipf64", "sched256"])
def test_full_size(name):
    w = synth.WORKLOADS[name].with_(draft_mode=1)
    if name == "sched256":
        w = w.with_(tau_choices=(0.0,))
    res, orc, rep = _run(f"one-hot {name}", w, derived=name == "sched256")
    assert rep.exact + rep.margin == w.B
