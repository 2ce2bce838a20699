"""GPU parity on seeded random workloads: 120 draws over batch size, draft
length, vocabulary (including sizes that are not a multiple of the vector
width), dtype, temperature (greedy included), row distributions, drafter,
length mode (fixed with random lengths, tau with derived or given
confidences), one-hot drafts and the packed layout.  Each case is compared
with the CPU oracle element by element (tests/parity_util.py states the bar)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 120


def _case(i):
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 10))
    K = int(rng.integers(1, 41))
    V = int(rng.choice([1, 2, 7, 8, 63, 64, 257, 1000, 1024, 3001, 4096, 16384, 16385, 20000]))
    dtype = int(rng.choice([synth.F32, synth.BF16]))
    T = float(rng.choice([0.0, 0.5, 0.7, 1.0, 1.5]))
    kind = int(rng.integers(0, 2))
    sig = float(rng.choice([0.01, 0.1, 0.5, 1.5]))
    onehot = T > 0 and rng.random() < 0.2
    mode = rng.choice(["fixed", "fixed_random", "tau_derived", "tau_given"])
    if T == 0.0 and mode == "tau_derived":
        mode = "tau_given"  # a derived confidence needs a draft distribution
    packed = (not onehot) and mode in ("fixed", "fixed_random") and rng.random() < 0.25
    w = synth.Workload(f"random{i}", B=B, K=K, V=V, dtype=dtype, target_kind=kind,
                       target_scale=float(rng.choice([1.0, 2.0, 4.0])), zipf_s=1.2, zipf_jitter=0.3,
                       sigma_first=sig, sigma_last=sig * float(rng.choice([1.0, 3.0])),
                       token_mode=(2 if onehot else int(rng.integers(0, 2))), p_match=0.9,
                       temperature=T, draft_mode=1 if onehot else 0, seed=2000 + i)
    if mode.startswith("tau"):
        w = w.with_(length_mode=synth.LEN_TAU, tau_choices=(0.0, 1e-4, 0.05, 0.5, 1.0))
    prob = synth.make_problem(w)
    if mode == "fixed_random":
        prob.verify_len = rng.integers(0, K + 1, size=B).astype(np.int32)
    if mode == "tau_given":
        prob.confidence = (rng.random((B, K)) ** 0.3).astype(np.float32)
    return w, prob, mode, packed


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_workload(i):
    from draft_verification_amd import device as D
    w, prob, mode, packed = _case(i)
    print(f"[case] random {i}: B={w.B} K={w.K} V={w.V} dt={w.dtype} T={w.temperature} mode={mode} "
          f"onehot={w.draft_mode} packed={packed}", flush=True)
    if packed:
        L = prob.verify_len if prob.verify_len is not None else np.full(w.B, w.K, np.int32)
        prob.verify_len = np.asarray(L, np.int32)
        dp = D.packed_from_problem(prob, prob.verify_len)
    else:
        dp = D.from_problem(prob)
    res = D.run_once(dp)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(f"random {i}", res, orc, dtype=w.dtype, greedy=w.temperature == 0, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
