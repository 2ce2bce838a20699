"""GPU parity of long draft blocks, where the last position group deals several
rows to each workgroup (four or more position groups: K >= 11).

Acceptance is made high (draft = target + small noise, or a greedy drafter
that matches often) so that many sequences reach the last group, and low in
other cases so that the group is sparse; B * rows is chosen not to divide
evenly among the workgroups.  Every case is compared with the CPU oracle
element by element (tests/parity_util.py states the bar).
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(name, w, *, prob=None, derived=False, packed=False):
    from draft_verification_amd import device as D
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature} mode={w.length_mode}",
          flush=True)
    prob = prob or synth.make_problem(w)
    if packed:
        dp = D.packed_from_problem(prob, prob.verify_len)
    else:
        dp = D.from_problem(prob)
    res = D.run_once(dp)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, res, orc, dtype=w.dtype, greedy=w.temperature == 0, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    return res, orc


BASE = synth.Workload("late", B=7, K=16, V=16392, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                      sigma_first=0.05, sigma_last=0.1, temperature=1.0, seed=120)


def _last_group_start(K):
    """First position of the last position group (groups of 3, 3, 4, 8, 16, 16,
    ... positions over K + 1 rows; a remainder of one joins the group before)."""
    first = [3, 3, 4, 8]
    j0, ng, start, npos = 1, 0, 1, K + 1
    while j0 <= npos:
        G = first[ng] if ng < len(first) else min(first[-1] << (ng - len(first) + 1), 16)
        if npos - (j0 + G - 1) <= 1:
            G = npos - j0 + 1
        G = min(G, 16)
        start = j0
        j0 += G
        ng += 1
    return start


@pytest.mark.parametrize("K", [12, 16, 23, 40])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_high_acceptance(K, dtype):
    w = BASE.with_(K=K, dtype=dtype, B=7, sigma_first=0.01, sigma_last=0.01, seed=121 + K + dtype)
    res, _ = _run(f"late K={K} dt={dtype}", w)
    # sequences reach the last group (its rows are streamed by the late-group kernel)
    assert (res["accepted_len"] >= _last_group_start(K) - 1).sum() >= 2


@pytest.mark.parametrize("B,V", [(1, 2048), (37, 16392), (13, 40000)])
def test_mixed_acceptance(B, V):
    # noise rising along the block: some sequences stop early, some reach the end
    w = BASE.with_(B=B, V=V, sigma_first=0.05, sigma_last=1.5, seed=130 + B)
    _run(f"late mixed B={B} V={V}", w)


def test_temperature_and_derived_length():
    w = BASE.with_(B=29, K=20, V=8000, temperature=0.7, length_mode=synth.LEN_TAU,
                   tau_choices=(0.0, 1e-6, 1e-3), sigma_first=0.05, sigma_last=0.3, seed=140)
    _run("late T=0.7 tau", w, derived=True)


@pytest.mark.parametrize("K", [16, 31])
def test_greedy(K):
    w = synth.WORKLOADS["greedy1024"].with_(B=41, K=K, V=16392, p_match=0.95, seed=150 + K)
    res, _ = _run(f"late greedy K={K}", w)
    assert (res["accepted_len"] >= 12).sum() >= 5


def test_one_hot():
    w = BASE.with_(B=19, K=18, V=12000, draft_mode=1, token_mode=2, target_kind=1, zipf_s=1.3,
                   zipf_jitter=0.3, sigma_first=0.2, sigma_last=0.2, temperature=0.7, seed=160)
    _run("late one-hot", w)


@pytest.mark.parametrize("greedy", [False, True])
def test_large_batch(greedy):
    # 4101 sequences: many workgroup columns, several open sequences sharing one
    if greedy:
        w = synth.WORKLOADS["greedy1024"].with_(B=4101, K=12, V=520, p_match=0.97, seed=175)
    else:
        w = BASE.with_(B=4101, K=12, V=520, sigma_first=0.01, sigma_last=0.01, seed=176)
    res, _ = _run(f"late B=4101 greedy={greedy}", w)
    assert (res["accepted_len"] >= _last_group_start(w.K) - 1).sum() >= 50


def test_packed_ragged_lengths():
    w = BASE.with_(B=23, K=16, V=16392, seed=170)
    prob = synth.make_problem(w)
    prob.verify_len = np.random.default_rng(170).integers(0, 17, size=w.B).astype(np.int32)
    prob.verify_len[:5] = 16
    _run("late packed", w, prob=prob, packed=True)
