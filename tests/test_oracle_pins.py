"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a library routine
(scipy / numpy), an invariant of the construction, or brute force.  None of the
expected values are taken from the oracle or from the GPU path.
"""
import itertools

import numpy as np
import pytest
from scipy import special

from oracle import oracle as O

F32, BF16 = O.F32, O.BF16


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16(x):
    """float -> bf16 bits, round to nearest even (test-local conversion)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _problem(rng, B, K, V, scale=2.0, noise=0.5, dtype=F32):
    t = (scale * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d = (t[:, :K, :] + noise * rng.standard_normal((B, K, V))).astype(np.float32)
    if dtype == BF16:
        t, d = _bf16(t), _bf16(d)
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    u = np.clip(u, 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    return t, d, tok, u


def _vals(a, dtype):
    return (_widen(a) if dtype == BF16 else a).astype(np.float64)


# ---------------------------------------------------------------- lse ----

def test_lse_constant_rows_closed_form():
    # a row of V equal logits c has lse(c/T) = c/T + ln V
    B, K, V = 3, 2, 1000
    for T in (1.0, 0.5, 2.0):
        t = np.zeros((B, K + 1, V), np.float32)
        d = np.zeros((B, K, V), np.float32)
        for b in range(B):
            t[b] = 0.75 * (b + 1)
            d[b] = -1.5 * (b + 1)
        tok = np.zeros((B, K), np.int32)
        u = np.full((B, K + 1), 0.5, np.float32)
        r = O.verify(t, d, tok, u, T, dtype=F32, all_rows=True)
        for b in range(B):
            np.testing.assert_allclose(r.lse_target[b], 0.75 * (b + 1) / T + np.log(V), rtol=0, atol=1e-12)
            np.testing.assert_allclose(r.lse_draft[b], -1.5 * (b + 1) / T + np.log(V), rtol=0, atol=1e-12)


def test_lse_masked_rows_closed_form():
    # k entries at 0 and V-k at -inf: lse = ln k
    V, K = 64, 1
    for k in (1, 2, 7, 64):
        t = np.full((1, K + 1, V), -np.inf, np.float32)
        d = np.full((1, K, V), -np.inf, np.float32)
        t[0, :, :k] = 0.0
        d[0, :, V - k:] = 0.0
        r = O.verify(t, d, np.zeros((1, K), np.int32), np.full((1, K + 1), 0.5, np.float32), 1.0,
                     dtype=F32, all_rows=True)
        np.testing.assert_allclose(r.lse_target[0], np.log(k), atol=1e-14)
        np.testing.assert_allclose(r.lse_draft[0], np.log(k), atol=1e-14)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_lse_matches_scipy_logsumexp(dtype, T):
    rng = _rng(1)
    t, d, tok, u = _problem(rng, 5, 3, 777, dtype=dtype)
    r = O.verify(t, d, tok, u, T, dtype=dtype, all_rows=True)
    want_t = special.logsumexp(_vals(t, dtype) / np.float64(np.float32(T)), axis=2)
    want_d = special.logsumexp(_vals(d, dtype) / np.float64(np.float32(T)), axis=2)
    np.testing.assert_allclose(r.lse_target, want_t, rtol=1e-13)
    np.testing.assert_allclose(r.lse_draft, want_d, rtol=1e-13)


# ------------------------------------------------------- acceptance -----

def test_q_equal_p_accepts_every_verified_position():
    # ratio == 1 for every token, so every u in (0,1) accepts: a = L
    rng = _rng(2)
    B, K, V = 50, 6, 300
    t, d, tok, u = _problem(rng, B, K, V)
    d = t[:, :K, :].copy()
    for L in (0, 3, 6):
        vl = np.full(B, L, np.int32)
        r = O.verify(t, d, tok, u, 1.0, dtype=F32, verify_len=vl)
        assert np.all(r.accepted_len == L)
        assert np.all(r.final_kind == O.FINAL_BONUS)
        assert np.all(r.out_tokens[:, :L] == tok[:, :L])


def test_tiny_uniform_accepts_and_large_ratio_gap_rejects():
    # u = 2^-24 accepts whenever p(x)/q(x) > 2^-24; a token with p(x) << q(x)
    # and u near 1 is rejected at position 1
    V, K = 16, 2
    t = np.zeros((1, K + 1, V), np.float32)
    d = np.zeros((1, K, V), np.float32)
    tok = np.array([[3, 5]], np.int32)
    r = O.verify(t, d, tok, np.full((1, K + 1), 2 ** -24, np.float32), 1.0, dtype=F32)
    assert r.accepted_len[0] == 2
    d2 = d.copy()
    d2[0, 0, 3] = 10.0            # q(3) >> p(3) at position 1
    r = O.verify(t, d2, tok, np.full((1, K + 1), 0.999, np.float32), 1.0, dtype=F32)
    assert r.accepted_len[0] == 0 and r.final_kind[0] == O.FINAL_RESIDUAL


def _shared_rows(rng, K, V, scale=1.5, noise=0.8):
    t = (scale * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + noise * rng.standard_normal((K, V))).astype(np.float32)
    return t, d


def _draw_from(rng, probs, n):
    c = np.cumsum(probs)
    c[-1] = 1.0
    return np.searchsorted(c, rng.random(n), side="right").astype(np.int32)


def test_expected_acceptance_is_sum_of_min_p_q():
    # E[accept at position 1] = sum_v min(p_v, q_v) for x ~ q (Monte Carlo, 6 sigma)
    rng = _rng(3)
    K, V, N = 1, 12, 200000
    t, d = _shared_rows(rng, K, V)
    p = special.softmax(t.astype(np.float64), axis=1)
    q = special.softmax(d.astype(np.float64), axis=1)
    alpha = np.minimum(p[0], q[0]).sum()
    tok = _draw_from(rng, q[0], N)[:, None]
    u = rng.random((N, K + 1)).astype(np.float32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32)
    rate = (r.accepted_len >= 1).mean()
    assert abs(rate - alpha) < 6 * np.sqrt(alpha * (1 - alpha) / N)


def test_expected_accepted_length_closed_form():
    # position-wise independent rows: E[a] = sum_{j<=L} prod_{i<=j} alpha_i
    rng = _rng(4)
    K, V, N = 4, 10, 200000
    t, d = _shared_rows(rng, K, V)
    p = special.softmax(t.astype(np.float64), axis=1)
    q = special.softmax(d.astype(np.float64), axis=1)
    alpha = np.minimum(p[:K], q).sum(axis=1)
    tok = np.stack([_draw_from(rng, q[j], N) for j in range(K)], axis=1)
    u = rng.random((N, K + 1)).astype(np.float32)
    for L in (2, 4):
        r = O.verify(t, d, tok, u, 1.0, dtype=F32, verify_len=np.full(N, L, np.int32))
        want = sum(np.prod(alpha[:j]) for j in range(1, L + 1))
        sd = r.accepted_len.std() / np.sqrt(N)
        assert abs(r.accepted_len.mean() - want) < 6 * sd


# ---------------------------------------------------------- residual ----

def test_residual_mass_identity_and_searchsorted_draw():
    # Z = sum max(0, p - q) = 1 - sum min(p, q); y = searchsorted(cumsum(r), u Z, 'right')
    rng = _rng(5)
    B, K, V = 400, 3, 257
    t, d, _, u = _problem(rng, B, K, V, noise=1.0)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        q = special.softmax(d[b].astype(np.float64), axis=1)
        for j in range(K):
            tok[b, j] = _draw_from(rng, q[j], 1)[0]
    r = O.verify(t, d, tok, u, 1.0, dtype=F32)
    n_checked = 0
    for i in range(B):
        if r.final_kind[i] != O.FINAL_RESIDUAL:
            continue
        js = r.accepted_len[i]            # 0-based row of the replacement draw
        p = special.softmax(t[i, js].astype(np.float64))
        q = special.softmax(d[i, js].astype(np.float64))
        Z = 1.0 - np.minimum(p, q).sum()
        np.testing.assert_allclose(r.residual_mass[i], Z, rtol=1e-12, atol=1e-15)
        res = np.maximum(p - q, 0.0)
        if r.margin[i] & O.MARGIN_CDF:
            continue
        y = int(np.searchsorted(np.cumsum(res), np.float64(u[i, K]) * res.sum(), side="right"))
        assert r.out_tokens[i, js] == y
        np.testing.assert_allclose(r.sampled_prob[i], res[y] / res.sum(), rtol=1e-10)
        n_checked += 1
    assert n_checked > 100


def test_one_hot_draft_residual_is_p_without_x():
    # q one-hot at x: accept iff u < p(x); the replacement is p with x removed, renormalised
    rng = _rng(6)
    V, K, B = 50, 1, 300
    t = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d = np.full((B, K, V), -np.inf, np.float32)
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    for b in range(B):
        d[b, 0, tok[b, 0]] = 0.0
    u = rng.random((B, K + 1)).astype(np.float32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32)
    for b in range(B):
        p = special.softmax(t[b, 0].astype(np.float64))
        x = tok[b, 0]
        accept = u[b, 0] < p[x]
        assert r.accepted_len[b] == int(accept)
        if not accept and not (r.margin[b] & O.MARGIN_CDF):
            res = p.copy()
            res[x] = 0.0
            y = int(np.searchsorted(np.cumsum(res) / res.sum(), np.float64(u[b, K]), side="right"))
            assert r.out_tokens[b, 0] == y


def test_bonus_draw_is_searchsorted_of_p():
    rng = _rng(7)
    B, K, V = 300, 2, 1000
    t, d, tok, u = _problem(rng, B, K, V)
    d = t[:, :K].copy()                  # q == p: everything verified is accepted
    for L in (0, 1, 2):
        r = O.verify(t, d, tok, u, 1.0, dtype=F32, verify_len=np.full(B, L, np.int32))
        for b in range(B):
            if r.margin[b] & O.MARGIN_CDF:
                continue
            p = special.softmax(t[b, L].astype(np.float64))
            y = int(np.searchsorted(np.cumsum(p), np.float64(u[b, K]), side="right"))
            assert r.out_tokens[b, L] == y
            np.testing.assert_allclose(r.sampled_prob[b], p[y], rtol=1e-12)
            assert r.residual_mass[b] == 1.0


def test_bonus_on_bf16_rows_at_temperature():
    rng = _rng(8)
    B, K, V, T = 200, 1, 513, 0.7
    t, d, tok, u = _problem(rng, B, K, V, dtype=BF16)
    r = O.verify(t, d, tok, u, T, dtype=BF16, verify_len=np.zeros(B, np.int32))
    tv = _vals(t, BF16) / np.float64(np.float32(T))
    for b in range(B):
        if r.margin[b] & O.MARGIN_CDF:
            continue
        p = special.softmax(tv[b, 0])
        assert r.out_tokens[b, 0] == int(np.searchsorted(np.cumsum(p), np.float64(u[b, K]), side="right"))


@pytest.mark.parametrize("offset", [1.0e30, -1.0e30, 3.0e38])
def test_huge_equal_logits_give_the_uniform_distribution(offset):
    # every logit equal (the noise is below one ulp of the offset): p = q = 1/V,
    # so every verified position is accepted (ratio 1), the bonus token is the
    # inverse CDF of the uniform distribution, floor(u * V), with probability 1/V,
    # and lse = offset / T + ln V
    rng = _rng(21)
    B, K, V = 16, 3, 1000
    t = (np.float32(offset) + rng.standard_normal((B, K + 1, V)).astype(np.float32)).astype(np.float32)
    d = (np.float32(offset) + rng.standard_normal((B, K, V)).astype(np.float32)).astype(np.float32)
    assert np.all(t == np.float32(offset)) and np.all(d == np.float32(offset))
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32, all_rows=True)
    assert np.all(r.accepted_len == K)
    for b in range(B):
        if r.margin[b] & O.MARGIN_CDF:
            continue
        assert r.out_tokens[b, K] == int(np.floor(np.float64(u[b, K]) * V))
        np.testing.assert_allclose(r.sampled_prob[b], 1.0 / V, rtol=1e-12)
    np.testing.assert_allclose(r.lse_target, np.float64(np.float32(offset)) + np.log(V), rtol=1e-15)


def test_bonus_draw_is_shift_invariant_at_large_offsets():
    # softmax does not change when a constant is added to the row; with an
    # offset of 2^20 and logits on a 2^-3 grid every value stays exact in fp32,
    # so the draw and its probability equal scipy's softmax of the unshifted row
    rng = _rng(22)
    B, K, V = 200, 1, 700
    base = (np.round(8 * 2.0 * rng.standard_normal((B, K + 1, V))) / 8).astype(np.float32)
    t = (base + np.float32(2 ** 20)).astype(np.float32)
    assert np.array_equal(t.astype(np.float64) - 2 ** 20, base.astype(np.float64))
    d = t[:, :K].copy()
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32, verify_len=np.zeros(B, np.int32))
    for b in range(B):
        if r.margin[b] & O.MARGIN_CDF:
            continue
        p = special.softmax(base[b, 0].astype(np.float64))
        y = int(np.searchsorted(np.cumsum(p), np.float64(u[b, K]), side="right"))
        assert r.out_tokens[b, 0] == y
        np.testing.assert_allclose(r.sampled_prob[b], p[y], rtol=1e-12)


# ------------------------------------------------------------ greedy ----

def test_greedy_prefix_and_argmax():
    rng = _rng(9)
    B, K, V = 500, 5, 300
    t, _, _, _ = _problem(rng, B, K, V, dtype=BF16)
    tv = _vals(t, BF16)
    g = np.argmax(tv, axis=2)            # numpy: first occurrence of the max
    tok = np.where(rng.random((B, K)) < 0.7, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    r = O.verify(t, None, tok, None, 0.0, dtype=BF16)
    for b in range(B):
        a = 0
        while a < K and tok[b, a] == g[b, a]:
            a += 1
        assert r.accepted_len[b] == a
        assert list(r.out_tokens[b, :a]) == list(tok[b, :a])
        assert r.out_tokens[b, a] == g[b, a]
        assert np.all(r.out_tokens[b, a + 1:] == -1)


def test_greedy_ties_take_lowest_index():
    V, K = 32, 1
    t = np.zeros((1, K + 1, V), np.float32)
    t[0, :, [5, 9, 30]] = 3.0
    r = O.verify(t, None, np.array([[5]], np.int32), None, 0.0, dtype=F32)
    assert r.accepted_len[0] == 1 and r.out_tokens[0, 1] == 5
    r = O.verify(t, None, np.array([[9]], np.int32), None, 0.0, dtype=F32)
    assert r.accepted_len[0] == 0 and r.out_tokens[0, 0] == 5


# ------------------------------------------------- survival and length --

def _brute_L(c, tau):
    S, L, out = 1.0, 0, []
    for j, cj in enumerate(c, 1):
        S *= float(cj)
        out.append(S)
        if S >= tau:
            L = j
    return L, out


def test_verify_length_brute_force_with_given_confidence():
    rng = _rng(10)
    B, K, V = 200, 6, 20
    t, d, tok, u = _problem(rng, B, K, V)
    c = rng.random((B, K)).astype(np.float32) ** 0.3
    c[:20] = 1.0
    tau = rng.choice(np.array([0.0, 1e-3, 0.1, 0.3, 0.5, 0.9, 1.0, 1.5], np.float32), B)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32, length_mode=O.LEN_TAU, confidence=c, tau=tau)
    for b in range(B):
        L, S = _brute_L(c[b].astype(np.float64), float(tau[b]))
        assert r.verify_len[b] == L
        np.testing.assert_allclose(r.survival[b], S, rtol=1e-15)
        if tau[b] <= 0:
            assert L == K
        if np.all(c[b] == 1.0) and tau[b] <= 1.0:
            assert L == K
        if tau[b] > 1.0:
            assert L == 0
        assert r.accepted_len[b] <= L


def test_derived_confidence_is_max_draft_probability():
    rng = _rng(11)
    B, K, V = 60, 5, 40
    t, d, tok, u = _problem(rng, B, K, V, scale=3.0)
    T = 0.8
    tau = np.full(B, 0.01, np.float32)
    r = O.verify(t, d, tok, u, T, dtype=F32, length_mode=O.LEN_TAU, tau=tau)
    q = special.softmax(d.astype(np.float64) / np.float64(np.float32(T)), axis=2)
    cmax = q.max(axis=2)
    for b in range(B):
        L, S = _brute_L(cmax[b], 0.01)
        assert r.verify_len[b] == L
        np.testing.assert_allclose(r.survival[b], S, rtol=1e-12)
        assert np.all(np.diff(r.survival[b]) <= 0)


# --------------------------------------------------------- bad input ----

def test_out_of_range_token_marks_sequence_bad():
    rng = _rng(12)
    B, K, V = 4, 3, 30
    t, d, tok, u = _problem(rng, B, K, V)
    d = t[:, :K].copy()                  # everything verified is accepted
    tok[1, 0] = V                        # tested at position 1
    tok[2, 2] = -1                       # tested at position 3
    tok[3, 2] = V + 5                    # not tested: L = 2
    vl = np.array([3, 3, 3, 2], np.int32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32, verify_len=vl)
    assert r.final_kind[0] == O.FINAL_BONUS and r.accepted_len[0] == 3
    for b in (1, 2):
        assert r.final_kind[b] == O.FINAL_BAD_INPUT and r.accepted_len[b] == 0
        assert np.all(r.out_tokens[b] == -1)
    assert r.final_kind[3] == O.FINAL_BONUS and r.accepted_len[3] == 2
    r = O.verify(t[:1], d[:1], tok[:1], u[:1], 1.0, dtype=F32, verify_len=np.array([K + 1], np.int32))
    assert r.final_kind[0] == O.FINAL_BAD_INPUT


def test_accept_margin_is_flagged():
    # place u within 1e-7 of the ratio p(x)/q(x) computed by scipy
    V, K = 8, 1
    rng = _rng(13)
    t = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    d = rng.standard_normal((1, K, V)).astype(np.float32)
    p = special.softmax(t[0, 0].astype(np.float64))
    q = special.softmax(d[0, 0].astype(np.float64))
    x = int(np.argmin(p / q))
    ratio = p[x] / q[x]
    u = np.array([[np.float32(ratio), 0.5]], np.float32)
    assert abs(float(u[0, 0]) - ratio) < 1e-6
    r = O.verify(t, d, np.array([[x]], np.int32), u, 1.0, dtype=F32)
    assert r.margin[0] & O.MARGIN_ACCEPT


@pytest.mark.parametrize("noise", [0.002, 0.01, 1.0])
def test_cdf_gap_is_relative_to_residual_mass(noise):
    # The final draw's CDF gap (distance of w = u Z to the nearest step of
    # cumsum(max(0, p - q))) is reported relative to Z itself; nearly equal
    # rows (noise 0.002, 0.01) give Z far below 1, unequal rows (noise 1) not.
    rng = _rng(17)
    B, K, V = 60, 1, 300
    t, d, _, u = _problem(rng, B, K, V, noise=noise)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        p = special.softmax(t[b, 0].astype(np.float64))
        q = special.softmax(d[b, 0].astype(np.float64))
        tok[b, 0] = int(np.argmin(p / q))    # p(x) < q(x): ratio below 1
    u[:, 0] = 1 - 2 ** -24                  # so the position is rejected
    r = O.verify(t, d, tok, u, 1.0, dtype=F32)
    zs = []
    for b in range(B):
        assert r.final_kind[b] == O.FINAL_RESIDUAL
        p = special.softmax(t[b, 0].astype(np.float64))
        q = special.softmax(d[b, 0].astype(np.float64))
        res = np.maximum(p - q, 0.0)
        C = np.cumsum(res)
        Z = C[-1]
        w = np.float64(u[b, K]) * Z
        y = int(np.searchsorted(C, w, side="right"))
        gap = min(abs(w - (C[y - 1] if y > 0 else 0.0)), abs(C[y] - w))
        np.testing.assert_allclose(r.residual_mass[b], Z, rtol=1e-10)
        np.testing.assert_allclose(r.cdf_gap[b], gap / Z, rtol=1e-6, atol=1e-15)
        assert bool(r.margin[b] & O.MARGIN_CDF) == (gap / Z < 1e-6)
        zs.append(Z)
    zs = np.array(zs)
    assert (zs < 0.05).all() if noise < 0.1 else (zs > 0.1).all()
