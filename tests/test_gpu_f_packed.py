"""Packed ("pruned, not padded") logits: sequence b brings its first L_b + 1
target rows and L_b draft rows, stacked, with row offsets (zhichai.net article,
"Under the hood", on SGLang's variable-length verification).  The outputs must
equal the dense layout's bit for bit (diagnostics included) and the oracle's on
the same logical rows."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Workload("packed", B=40, K=6, V=5000, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                      sigma_first=0.3, sigma_last=0.9, temperature=1.0, seed=81)


def _D():
    from draft_verification_amd import device as D
    return D


def _lengths(seed, Bn, K):
    L = np.random.default_rng(seed).integers(0, K + 1, size=Bn).astype(np.int32)
    L[:3] = [0, K, 1]
    return L


def _case(name, w, L, greedy=False):
    D = _D()
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature}", flush=True)
    prob = synth.make_problem(w)
    prob.verify_len = L
    dense = D.run_once(D.from_problem(prob))
    packed = D.run_once(D.packed_from_problem(prob, L))
    assert not PU.same_outputs(packed, dense)
    two = not greedy and w.draft_mode == 0
    es = 2 if w.dtype == synth.BF16 else 4
    for res in (packed, dense):
        assert not PU.check_streamed(res, w.K, w.V, es, two_rows=two)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, packed, orc, dtype=w.dtype, greedy=greedy, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    return packed, orc


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_packed_equals_dense_and_oracle(dtype, T):
    w = BASE.with_(dtype=dtype, temperature=T, seed=82 + dtype)
    _case(f"packed dt={dtype} T={T}", w, _lengths(82, w.B, w.K))


@pytest.mark.parametrize("V", [1, 257, 16385])
def test_packed_vocab_edges(V):
    w = BASE.with_(V=V, B=9, K=3, seed=90 + V)
    _case(f"packed V={V}", w, _lengths(90 + V, w.B, w.K))


def test_packed_greedy():
    w = synth.WORKLOADS["greedy1024"].with_(B=50, K=5, V=20000, seed=83)
    _case("packed greedy", w, _lengths(83, w.B, w.K), greedy=True)


def test_packed_one_hot():
    w = BASE.with_(draft_mode=1, token_mode=2, seed=84)
    _case("packed one-hot", w, _lengths(84, w.B, w.K))


def test_packed_full_size():
    w = synth.WORKLOADS["sched256"].with_(length_mode=synth.LEN_FIXED, tau_choices=())
    _case("packed sched256", w, _lengths(85, w.B, w.K))


def test_bad_row_counts():
    """A sequence whose target row count is outside [1, K+1], or whose draft
    row count is not its target count minus 1, is marked bad (a = 0, no token,
    status bit); the others are unaffected."""
    D = _D()
    w = BASE.with_(B=8, K=4, V=3000, dtype=synth.F32, seed=86)
    prob = synth.make_problem(w)
    L = np.array([2, 4, 5, 0, 3, -1, 1, 4], np.int64)   # 5 -> K+2 target rows, -1 -> none
    dp = D.packed_from_problem(prob, L)
    # one draft offset moved back a row: sequence 6 brings one draft row too few
    # and sequence 7 one too many (both bad, so neither is read); every offset
    # stays inside the packed tensor
    doff = dp.draft_row_offsets.cpu().numpy()
    doff[7] -= 1
    assert doff[7] >= doff[6]
    dp.draft_row_offsets = torch.from_numpy(doff).to(dp.target.device)
    res = D.run_once(dp)
    bad = {2, 5, 6, 7}
    assert res["device_status"][0] == 1
    for b in range(w.B):
        if b in bad:
            assert res["accepted_len"][b] == 0 and (res["out_tokens"][b] == -1).all(), b
            assert res["rows_read"][b] == 0 and res["bytes_read"][b] == 0, b
    good = [b for b in range(w.B) if b not in bad]
    prob.verify_len = np.clip(L, 0, w.K).astype(np.int32)
    orc = O.verify_problem(prob, seqs=good, all_rows=True)
    rep = PU.compare("packed bad counts", res, orc, dtype=w.dtype, prob=prob)
    assert not rep.mismatches, rep.mismatches[:5]


def _bounded(dp, bound):
    dp.max_verify_len = int(bound)
    return dp


@pytest.mark.parametrize("layout,mode", [("dense", "probs"), ("packed", "probs"), ("dense", "greedy"),
                                         ("packed", "onehot"), ("dense", "fp32")])
def test_length_bound_changes_nothing_but_the_launch(layout, mode):
    """With max_verify_len = max L_b the step launches positions 1 .. max L_b + 1
    only; its outputs (diagnostics included) equal the unbounded call's bit for
    bit, and its stream counts stay within the needed rows and the window
    (draft probabilities, greedy and one-hot drafts, bf16 and fp32)."""
    D = _D()
    w = BASE.with_(K=8, seed=87)
    if mode == "greedy":
        w = w.with_(temperature=0.0)
    elif mode == "onehot":
        w = w.with_(draft_mode=1, token_mode=2)
    elif mode == "fp32":
        w = w.with_(dtype=synth.F32)
    L = np.random.default_rng(87).integers(0, 4, size=w.B).astype(np.int32)
    L[:2] = [0, 3]
    prob = synth.make_problem(w)
    prob.verify_len = L
    make = (lambda: D.packed_from_problem(prob, L)) if layout == "packed" else (lambda: D.from_problem(prob))
    print(f"[case] bound {layout} {mode} B={w.B} K={w.K} V={w.V} max L={L.max()}", flush=True)
    free = D.run_once(make())
    es = 4 if w.dtype == synth.F32 else 2
    for bound in (int(L.max()), int(L.max()) + 2, w.K):
        res = D.run_once(_bounded(make(), bound))
        assert not PU.same_outputs(res, free), bound
        assert not PU.check_streamed(res, w.K, w.V, es, two_rows=mode in ("probs", "fp32")), bound
    assert int(free["device_status"][0]) == 0


@pytest.mark.parametrize("layout", ["dense", "packed"])
def test_length_bound_marks_longer_sequences_bad(layout):
    """A sequence whose L_b exceeds max_verify_len is marked bad (a = 0, no
    token, status bit) and none of its rows is read; the others match the
    oracle."""
    D = _D()
    w = BASE.with_(B=12, K=5, V=7000, seed=88)
    L = np.array([0, 1, 2, 3, 4, 5, 2, 1, 5, 0, 3, 2], np.int32)
    bound = 2
    prob = synth.make_problem(w)
    prob.verify_len = L
    dp = D.packed_from_problem(prob, L) if layout == "packed" else D.from_problem(prob)
    print(f"[case] bound {bound} marks bad, {layout}", flush=True)
    res = D.run_once(_bounded(dp, bound))
    assert int(res["device_status"][0]) == 1
    bad = [b for b in range(w.B) if L[b] > bound]
    for b in bad:
        assert res["accepted_len"][b] == 0 and (res["out_tokens"][b] == -1).all(), b
        assert res["rows_read"][b] == 0 and res["bytes_read"][b] == 0, b
    good = [b for b in range(w.B) if L[b] <= bound]
    orc = O.verify_problem(prob, seqs=good, all_rows=True)
    rep = PU.compare(f"bound {layout}", res, orc, dtype=w.dtype, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]


def test_length_bound_full_size_admission_lengths():
    """The full-size shape with admission-like lengths (mostly 0 .. 4) and the
    bound at their maximum, packed: equal to the unbounded dense call."""
    D = _D()
    w = synth.WORKLOADS["sched256"].with_(length_mode=synth.LEN_FIXED, tau_choices=())
    L = np.minimum(np.random.default_rng(89).geometric(0.55, size=w.B) - 1, w.K).astype(np.int32)
    prob = synth.make_problem(w)
    prob.verify_len = L
    print(f"[case] bound full size max L={L.max()} sum L={L.sum()}", flush=True)
    dense = D.run_once(D.from_problem(prob))
    res = D.run_once(_bounded(D.packed_from_problem(prob, L), int(L.max())))
    assert not PU.same_outputs(res, dense)
    assert int(res["device_status"][0]) == 0
