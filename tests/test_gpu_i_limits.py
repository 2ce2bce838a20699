"""GPU parity at the library's size limits: the largest vocabulary
(SV_MAX_VOCAB = 2^20 tokens: 64 splits, so a row's merge takes every lane of a
wavefront), the longest draft block (SV_MAX_DRAFT = 256: nine launches of the
row statistics) and the largest batch (SV_MAX_BATCH sequences).
Each case is compared with the CPU oracle (tests/parity_util.py states the
bar; the largest batch compares the decisions array-wise)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SV_MAX_VOCAB, SV_MAX_DRAFT, SV_MAX_BATCH = 1048576, 256, 1048575


def _run(name, w, *, derived=False):
    from draft_verification_amd import device as D
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature} mode={w.length_mode}",
          flush=True)
    prob = synth.make_problem(w)
    res = D.run_once(D.from_problem(prob))
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, res, orc, dtype=w.dtype, greedy=w.temperature == 0, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    return res, orc


BASE = synth.Workload("limits", B=3, K=2, V=SV_MAX_VOCAB, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                      sigma_first=0.3, sigma_last=0.6, temperature=1.0, seed=180)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_largest_vocabulary(dtype, T):
    _run(f"V=2^20 dt={dtype} T={T}", BASE.with_(dtype=dtype, temperature=T, seed=181 + dtype))


def test_largest_vocabulary_greedy_and_derived_length():
    w = synth.WORKLOADS["greedy1024"].with_(B=4, K=3, V=SV_MAX_VOCAB, seed=183)
    _run("V=2^20 greedy", w)
    w = BASE.with_(B=4, K=5, length_mode=synth.LEN_TAU, tau_choices=(0.0, 1e-7), seed=184)
    _run("V=2^20 derived tau", w, derived=True)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_longest_draft_block(dtype):
    # near-identical draft rows: most sequences walk deep into the block
    w = BASE.with_(B=3, K=SV_MAX_DRAFT, V=2048, dtype=dtype, sigma_first=0.002, sigma_last=0.002, seed=185 + dtype)
    res, _ = _run(f"K=256 dt={dtype}", w)
    assert res["accepted_len"].max() >= 64


def test_largest_batch():
    w = synth.Workload("maxbatch", B=SV_MAX_BATCH, K=1, V=8, dtype=synth.F32, target_kind=0, target_scale=2.0,
                       sigma_first=0.5, sigma_last=0.5, temperature=1.0, seed=186)
    from draft_verification_amd import device as D
    print(f"[case] largest batch B={w.B} K={w.K} V={w.V}", flush=True)
    prob = synth.make_problem(w)
    res = D.run_once(D.from_problem(prob))
    orc = O.verify_problem(prob, all_rows=True)
    ok = orc.margin == 0
    print(f"[case] largest batch: {int((~ok).sum())} margin cases", flush=True)
    np.testing.assert_array_equal(res["verify_len_out"], orc.verify_len)
    np.testing.assert_array_equal(res["accepted_len"][ok], orc.accepted_len[ok])
    np.testing.assert_array_equal(res["out_tokens"][ok], orc.out_tokens[ok])
    assert (res["device_status"] == 0).all()
