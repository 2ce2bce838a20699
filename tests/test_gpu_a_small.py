"""GPU parity at small shapes: every mode, ragged V and K, edge cases.

Inputs come from the shared seeded generator (synth) and are compared with the
CPU oracle element by element (tests/parity_util.py states the bar).  Sizes
span several 16384-element splits and ragged tails while the oracle finishes
in well under a second per case.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    from draft_verification_amd import device as D
    return D


def _run_case(name, w, *, prob=None, derived=False, seqs=None, sv=None):
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature} mode={w.length_mode}",
          flush=True)
    D = _dev()
    prob = prob or synth.make_problem(w)
    dp = D.from_problem(prob)
    res = D.run_once(dp, sv)
    orc = O.verify_problem(prob, seqs=seqs, all_rows=True)
    rep = PU.compare(name, res, orc, dtype=w.dtype, greedy=w.temperature == 0, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    return res, orc, rep


BASE = synth.Workload("small", B=3, K=4, V=1024, dtype=synth.F32, target_kind=0, target_scale=2.0,
                      sigma_first=0.5, sigma_last=0.9, temperature=1.0, seed=11)

VOCABS = [1, 2, 7, 8, 255, 256, 257, 513, 1024, 16383, 16384, 16385, 40000]


@pytest.mark.parametrize("V", VOCABS)
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_vocab_sweep_fixed(V, dtype):
    w = BASE.with_(V=V, dtype=dtype, B=5, K=3, seed=1000 + V + dtype)
    _run_case(f"vocab V={V} dt={dtype}", w)


@pytest.mark.parametrize("K", [1, 2, 5, 16])
@pytest.mark.parametrize("T", [0.7, 1.0])
def test_draft_length_and_temperature(K, T):
    w = BASE.with_(K=K, B=16, V=3000, temperature=T, dtype=synth.BF16, seed=2000 + K)
    _run_case(f"K={K} T={T}", w)


def test_ragged_verify_lengths_including_zero():
    w = BASE.with_(B=40, K=6, V=5000, seed=31)
    prob = synth.make_problem(w)
    rng = np.random.default_rng(31)
    prob.verify_len = rng.integers(0, 7, size=40).astype(np.int32)
    prob.verify_len[:5] = 0
    _run_case("ragged L", w, prob=prob)


def test_all_accepted_when_draft_equals_target():
    w = BASE.with_(B=8, K=5, V=20000, dtype=synth.BF16, seed=32)
    prob = synth.make_problem(w)
    prob.draft = np.ascontiguousarray(prob.target[:, :5, :])
    res, orc, rep = _run_case("q == p", w, prob=prob)
    assert np.all(res["accepted_len"] == 5)


def test_masked_rows_and_one_hot_draft():
    w = BASE.with_(B=6, K=3, V=2049, seed=33)
    prob = synth.make_problem(w)
    rng = np.random.default_rng(33)
    t, d = prob.target, prob.draft
    for b in range(6):
        for j in range(4):
            cut = rng.integers(1, 2049)
            t[b, j, rng.permutation(2049)[:cut - 1]] = -np.inf   # keep at least one finite
    # one-hot draft rows at the drafted token for sequence 0
    for j in range(3):
        d[0, j, :] = -np.inf
        d[0, j, prob.tokens[0, j]] = 0.0
    _run_case("masked / one-hot", w, prob=prob)


def test_greedy_small():
    w = synth.WORKLOADS["greedy1024"].with_(B=33, V=40000, seed=34)
    _run_case("greedy small", w)


def test_greedy_ties_lowest_index():
    w = synth.WORKLOADS["greedy1024"].with_(B=4, K=2, V=20000, seed=35)
    prob = synth.make_problem(w)
    # plant an equal maximum at a second, later split
    for b in range(4):
        for j in range(3):
            row = synth.bf16_bits_to_f32(prob.target[b, j])
            am = int(np.argmax(row))
            prob.target[b, j, (am + 17000) % 20000] = prob.target[b, j, am]
    _run_case("greedy ties", w, prob=prob)


def test_tau_given_confidence():
    w = BASE.with_(B=64, K=8, V=3000, length_mode=synth.LEN_TAU, tau_choices=(0.0, 0.2, 0.5, 1.0, 1.5), seed=36)
    prob = synth.make_problem(w)
    rng = np.random.default_rng(36)
    c = (rng.random((64, 8)) ** 0.2).astype(np.float32)
    c[:8] = 1.0
    prob.confidence = c
    res, orc, rep = _run_case("tau with given c", w, prob=prob)
    np.testing.assert_array_equal(res["verify_len_out"], orc.verify_len)


@pytest.mark.parametrize("taus", [(0.3,), (0.0,), (1.5,), (1e-3, 1e-2, 0.05)])
def test_tau_derived_confidence(taus):
    # peaked rows so that max q is large enough for tau in (0, 1) to matter
    w = synth.WORKLOADS["peaked512"].with_(B=24, K=8, V=20000, tau_choices=taus, seed=37)
    _run_case(f"tau derived {taus}", w, derived=True)


@pytest.mark.parametrize("given", [False, True])
def test_tau_special_values(given):
    # tau NaN, +inf, 1.0 (above every survival below 1) verify nothing; -inf
    # and -0.0 verify every position (reading R8)
    w = synth.WORKLOADS["peaked512"].with_(B=10, K=6, V=3000, tau_choices=(0.3,), seed=92)
    prob = synth.make_problem(w)
    prob.tau = np.array([np.nan, np.inf, -np.inf, -0.0, 1.0, 0.0, np.nan, 2.0, -1.0, 1e-30], np.float32)
    if given:
        prob.confidence = np.full((w.B, w.K), 0.9, np.float32)
    res, orc, _ = _run_case(f"tau special given={given}", w, prob=prob, derived=not given)
    L = res["verify_len_out"]
    assert L[0] == 0 and L[1] == 0 and L[4] == 0 and L[6] == 0 and L[7] == 0
    assert L[2] == w.K and L[3] == w.K and L[5] == w.K and L[8] == w.K


def test_tau_derived_greedy_rejected():
    D = _dev()
    from draft_verification_amd import binding as B
    w = synth.WORKLOADS["greedy1024"].with_(B=2, K=2, V=100, length_mode=synth.LEN_TAU, tau_choices=(0.5,))
    prob = synth.make_problem(w)
    dp = D.from_problem(prob)
    sv = D.handle_for(dp)
    with pytest.raises(B.SpecVerifyError) as ei:
        sv.run(dp.args())
    assert ei.value.status == B.SV_EINVAL
    sv.close()


def test_bad_tokens_and_lengths_set_status():
    w = BASE.with_(B=6, K=3, V=500, seed=38)
    prob = synth.make_problem(w)
    prob.draft = np.ascontiguousarray(prob.target[:, :3, :])    # everything verified is accepted
    prob.tokens[1, 0] = 500
    prob.tokens[2, 2] = -3
    prob.tokens[3, 2] = 10 ** 6                                  # past L: never read
    prob.verify_len = np.array([3, 3, 3, 2, 4, -1], np.int32)    # 4 and -1 are out of range
    res, orc, rep = _run_case("bad input", w, prob=prob)
    assert res["device_status"][0] & 1
    for b in (1, 2, 4, 5):
        assert res["accepted_len"][b] == 0 and np.all(res["out_tokens"][b] == -1)
    for b in (4, 5):    # marked bad before any row: none is read
        assert res["rows_read"][b] == 0 and res["bytes_read"][b] == 0, b
    assert res["accepted_len"][3] == 2


def test_clean_status_is_zero():
    res, _, _ = _run_case("clean", BASE)
    assert res["device_status"][0] == 0


def test_empty_batch_is_a_no_op():
    D = _dev()
    prob = synth.make_problem(BASE)
    dp = D.from_problem(prob)
    sv = D.handle_for(dp)
    a = dp.args()
    a.B = 0
    sv.run(a)
    torch.cuda.synchronize()
    assert np.all(dp.accepted_len.cpu().numpy() == -7)
    sv.close()


def test_handle_reuse_with_smaller_batch():
    # one handle sized for the larger call serves a smaller one afterwards
    D = _dev()
    from draft_verification_amd import binding as B
    big = BASE.with_(B=20, K=6, V=3000, seed=40)
    small = BASE.with_(B=3, K=2, V=3000, seed=41)
    sv = B.SpecVerify(20, 6, 3000, synth.F32, 0)
    _run_case("reuse big", big, sv=sv)
    _run_case("reuse small", small, sv=sv)
    sv.close()


def _to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_offset_logits(dtype):
    """Rows shifted far from zero: large split maxima (the exponent's constant
    term m*c is then rounded far from exact), maxima beyond 2^20 / c (the
    exact-difference path), and 1e30 (every finite logit equal in fp32, so p
    and q are uniform)."""
    w = BASE.with_(B=8, K=4, V=20000, dtype=synth.F32, seed=37)
    prob = synth.make_problem(w)
    offs = [3000.0, -3000.0, 250.0, -1.0e5, 1.0e30, -1.0e30, 3.0e6, 7.5]
    for b, o in enumerate(offs):
        prob.target[b] += np.float32(o)
        prob.draft[b] += np.float32(o)
    if dtype == synth.BF16:
        prob.target = _to_bf16_bits(prob.target)
        prob.draft = _to_bf16_bits(prob.draft)
        prob.w = w.with_(dtype=synth.BF16)
    _run_case(f"offset logits dt={dtype}", prob.w, prob=prob)
