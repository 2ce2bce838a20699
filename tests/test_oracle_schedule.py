"""Pins of the oracle's load-aware admission (umans.ai blog, section
"2. Verify smarter": rank every drafted token by survival, admit while expected
accepted tokens x step rate at that batch size rises).

Expected values come from closed forms of particular speed curves, from
Python's own sort and exact summation (math.fsum), and from invariances; none
is taken from the oracle or the GPU path.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _conf(rng, B, K, lo=0.2):
    return rng.uniform(lo, 1.0, size=(B, K)).astype(np.float32)


def _survivals(c):
    """S_bj = prod_{i<=j} c_bi, left to right in fp64."""
    B, K = c.shape
    S = np.empty((B, K), np.float64)
    for b in range(B):
        acc = 1.0
        for j in range(K):
            acc *= float(c[b, j])
            S[b, j] = acc
    return S


def _ranked(S):
    B, K = S.shape
    return sorted(((S[b, j], b, j) for b in range(B) for j in range(K)), key=lambda t: (-t[0], t[1], t[2]))


def test_constant_speed_admits_every_positive_survival():
    # speed constant: T(m+1) - T(m) = S_(m) * speed, so admission continues
    # exactly while the next survival is positive
    rng = _rng(1)
    B, K = 12, 5
    c = _conf(rng, B, K)
    c[3, 2] = 0.0          # survivals of sequence 3 from position 3 on are 0
    c[7, 0] = 0.0          # sequence 7 admits nothing
    r = O.schedule(c, np.full(B * (K + 1) + 1, 3.5))
    S = _survivals(c)
    np.testing.assert_array_equal(r.verify_len, (S > 0).sum(axis=1))
    assert r.admitted == int((S > 0).sum())
    assert r.verify_len[7] == 0 and r.verify_len[3] == 2


@pytest.mark.parametrize("n0_extra", [0, 1, 7, 30])
def test_speed_cliff_caps_the_batch(n0_extra):
    # speed 1 up to a batch of n0 tokens and 0 beyond: T drops to 0 past n0,
    # so exactly min(N, n0 - B) candidates are admitted (all survivals > 0)
    rng = _rng(2)
    B, K = 9, 4
    c = _conf(rng, B, K)
    n0 = B + n0_extra
    speed = np.where(np.arange(B * (K + 1) + 1) <= n0, 1.0, 0.0)
    r = O.schedule(c, speed)
    assert r.admitted == min(B * K, n0 - B)
    ranked = _ranked(_survivals(c))
    want = np.zeros(B, np.int32)
    for _, b, _j in ranked[:r.admitted]:
        want[b] += 1
    np.testing.assert_array_equal(r.verify_len, want)


@pytest.mark.parametrize("a,bcost", [(20.0, 0.05), (5.0, 0.5), (300.0, 0.2)])
def test_latency_model_threshold(a, bcost):
    # step time a + bcost * n, speed = 1 / (a + bcost n).  Then
    # T(m+1) > T(m)  <=>  S_(m) (a + bcost (B + m)) > bcost (B + P(m)),
    # checked with Python's sort and exact sums on the oracle's answer.
    rng = _rng(3)
    B, K = 40, 8
    c = _conf(rng, B, K, lo=0.5)
    n = np.arange(B * (K + 1) + 1, dtype=np.float64)
    r = O.schedule(c, 1.0 / (a + bcost * n))
    ranked = _ranked(_survivals(c))
    m = r.admitted
    for i in range(m):
        P = math.fsum(t[0] for t in ranked[:i])
        assert ranked[i][0] * (a + bcost * (B + i)) > bcost * (B + P) * (1 + 1e-12)
    if m < B * K:
        P = math.fsum(t[0] for t in ranked[:m])
        assert ranked[m][0] * (a + bcost * (B + m)) <= bcost * (B + P) * (1 + 1e-12)
    assert 0 < m < B * K  # the curve makes the example non-trivial


def test_expected_throughput_and_tau():
    rng = _rng(4)
    B, K = 25, 6
    c = _conf(rng, B, K)
    n = np.arange(B * (K + 1) + 1, dtype=np.float64)
    speed = 1.0 / (10.0 + 0.2 * n)
    r = O.schedule(c, speed)
    S = _survivals(c)
    admitted_sum = math.fsum(S[b, j] for b in range(B) for j in range(r.verify_len[b]))
    m = int(r.verify_len.sum())
    assert m == r.admitted
    np.testing.assert_allclose(r.expected, (B + admitted_sum) * speed[B + m], rtol=1e-13)
    ranked = _ranked(S)
    assert r.tau == ranked[m - 1][0]
    np.testing.assert_array_equal(r.survival, S)


def test_admitted_sets_are_prefixes_and_dominate():
    # with c in [0,1] every sequence's admitted positions are 1..L_b, and no
    # admitted survival is below a rejected one
    rng = _rng(5)
    B, K = 30, 10
    c = _conf(rng, B, K, lo=0.0)
    n = np.arange(B * (K + 1) + 1, dtype=np.float64)
    r = O.schedule(c, 1.0 / (3.0 + 0.1 * n))
    S = _survivals(c)
    adm = [S[b, :r.verify_len[b]] for b in range(B)]
    rej = [S[b, r.verify_len[b]:] for b in range(B)]
    lo_adm = min((x.min() for x in adm if x.size), default=np.inf)
    hi_rej = max((x.max() for x in rej if x.size), default=-np.inf)
    assert lo_adm >= hi_rej


def test_equal_survivals_admit_in_sequence_then_position_order():
    # c = 1 everywhere: every survival is 1 and the ranking falls back to
    # (b, j); a cliff after r candidates fills whole sequences first
    B, K, r_adm = 6, 4, 10
    c = np.ones((B, K), np.float32)
    speed = np.where(np.arange(B * (K + 1) + 1) <= B + r_adm, 1.0, 0.0)
    r = O.schedule(c, speed)
    np.testing.assert_array_equal(r.verify_len, [4, 4, 2, 0, 0, 0])


def test_speed_scale_does_not_change_the_decision():
    rng = _rng(6)
    B, K = 16, 8
    c = _conf(rng, B, K)
    n = np.arange(B * (K + 1) + 1, dtype=np.float64)
    s1 = 1.0 / (8.0 + 0.3 * n)
    r1 = O.schedule(c, s1)
    r2 = O.schedule(c, 1024.0 * s1)  # a power of two keeps every product exact
    np.testing.assert_array_equal(r1.verify_len, r2.verify_len)
    assert r1.admitted == r2.admitted


def test_out_of_range_confidences_are_clamped_and_flagged():
    c = np.array([[0.5, 1.5, 0.5], [np.nan, 0.9, 0.9], [-0.1, 1.0, 1.0]], np.float32)
    r = O.schedule(c, np.full(3 * 4 + 1, 1.0))
    assert r.bad
    np.testing.assert_array_equal(r.survival, [[0.5, 0.5, 0.25], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    np.testing.assert_array_equal(r.verify_len, [3, 0, 0])


def test_empty_batch():
    r = O.schedule(np.zeros((0, 4), np.float32), np.ones(1))
    assert r.admitted == 0 and r.verify_len.size == 0 and math.isnan(r.tau)
