"""Pins of the oracle's margin outputs: the flags and the alternative token that
let the GPU comparison treat a near-tie as either outcome.

Each relaxes what the parity tests compare, so a mistake in one would hide a
GPU mismatch instead of raising one.  The expected values come from numpy's
searchsorted on a cumulative sum computed here in fp64 (scipy's softmax for
the probabilities), from cumulative products computed here, and from speed
curves built to tie exactly; none is taken from the oracle or the GPU path.
"""
import numpy as np
import pytest
from scipy import special

from oracle import oracle as O

F32 = O.F32


def _rng(seed):
    return np.random.default_rng(seed)


def _f32_near(x, side):
    """The fp32 value nearest to x strictly below (side < 0) or above (side > 0)."""
    f = np.float32(x)
    if side < 0:
        while np.float64(f) >= x:
            f = np.nextafter(f, np.float32(-np.inf))
    else:
        while np.float64(f) <= x:
            f = np.nextafter(f, np.float32(np.inf))
    return f


# ------------------------------------------------------- bonus-draw alt token

@pytest.mark.parametrize("side", [-1, 1])
def test_bonus_alt_token_is_the_token_across_the_nearest_step(side):
    # Bonus draw (w = u, Z = 1): u is placed one fp32 step below or above the
    # CDF step C_k; the drawn token is searchsorted(C, u, 'right') and the
    # token across the step is what the draw gives on the other side of C_k.
    rng = _rng(31)
    V, K = 40, 1
    t = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()                                   # q = p: position 1 accepted
    p = special.softmax(t[0, 1].astype(np.float64))       # the bonus row
    C = np.cumsum(p)
    for k in (3, 17, 30):
        uf = _f32_near(C[k], side)
        u = np.array([[0.5, uf]], np.float32)
        r = O.verify(t, d, np.zeros((1, K), np.int32), u, 1.0, dtype=F32)
        assert r.final_kind[0] == O.FINAL_BONUS and r.accepted_len[0] == 1
        w = np.float64(uf)
        y = int(np.searchsorted(C, w, side="right"))
        gap = abs(w - C[k])
        other = int(np.searchsorted(C, w - 2 * side * gap, side="right"))
        assert int(r.out_tokens[0, 1]) == y == (k + 1 if side > 0 else k)
        assert int(r.alt_token[0]) == other == (k if side > 0 else k + 1)
        np.testing.assert_allclose(r.cdf_gap[0], gap, rtol=1e-9, atol=1e-18)
        assert r.margin[0] & O.MARGIN_CDF                # an fp32 step is far below 1e-6


def test_bonus_draw_away_from_a_step_is_not_a_margin():
    rng = _rng(32)
    V, K = 40, 1
    t = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()
    p = special.softmax(t[0, 1].astype(np.float64))
    C = np.cumsum(p)
    k = 12
    mid = 0.5 * (C[k] + C[k + 1])
    u = np.array([[0.5, np.float32(mid)]], np.float32)
    r = O.verify(t, d, np.zeros((1, K), np.int32), u, 1.0, dtype=F32)
    assert int(r.out_tokens[0, 1]) == k + 1
    assert not (r.margin[0] & O.MARGIN_CDF)
    w = np.float64(u[0, 1])
    np.testing.assert_allclose(r.cdf_gap[0], min(w - C[k], C[k + 1] - w), rtol=1e-9)


# ------------------------------------------------- replacement-draw alt token

def _rejected_residual(seed, V, zero_every=0):
    """One sequence, K = 1, rejected at position 1, with target and draft rows
    such that max(0, p - q) has zero-mass tokens (every `zero_every`-th token
    gets q > p).  Returns (t, d, tok, residual masses r in fp64)."""
    rng = _rng(seed)
    K = 1
    t = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + 0.3 * rng.standard_normal((1, K, V))).astype(np.float32)
    if zero_every:
        d[0, 0, ::zero_every] = t[0, 0, ::zero_every] + 2.0   # q > p there: no residual mass
    p = special.softmax(t[0, 0].astype(np.float64))
    q = special.softmax(d[0, 0].astype(np.float64))
    x = int(np.argmin(p / q))                                 # ratio < 1
    return t, d, np.array([[x]], np.int32), np.maximum(p - q, 0.0)


@pytest.mark.parametrize("zero_every", [0, 3])
@pytest.mark.parametrize("side", [-1, 1])
def test_replacement_alt_token_skips_zero_mass_tokens(zero_every, side):
    # w = u Z with u one fp32 step away from C_k / Z: the drawn token and the
    # token across the nearest step both come from searchsorted on the fp64
    # cumulative residual, which steps over tokens of zero mass.
    V = 60
    t, d, tok, res = _rejected_residual(41 + zero_every, V, zero_every)
    C = np.cumsum(res)
    Z = C[-1]
    pos = np.nonzero(res > 0)[0]
    for k in pos[[2, len(pos) // 2, -3]]:
        uf = _f32_near(C[k] / Z, side)
        u = np.array([[1 - 2 ** -24, uf]], np.float32)          # position 1 rejected
        r = O.verify(t, d, tok, u, 1.0, dtype=F32)
        assert r.final_kind[0] == O.FINAL_RESIDUAL and r.accepted_len[0] == 0
        w = np.float64(uf) * Z
        y = int(np.searchsorted(C, w, side="right"))
        gap = abs(w - C[k])
        other = int(np.searchsorted(C, w - 2 * side * gap, side="right"))
        assert int(r.out_tokens[0, 0]) == y
        assert int(r.alt_token[0]) == other
        assert res[y] > 0 and res[other] > 0
        np.testing.assert_allclose(r.residual_mass[0], Z, rtol=1e-12)
        np.testing.assert_allclose(r.cdf_gap[0], gap / Z, rtol=1e-6, atol=1e-18)
        assert r.margin[0] & O.MARGIN_CDF


def test_replacement_last_token_margin_has_no_alt_above():
    # w one fp32 step below the last CDF step: the nearest step is the top of
    # the last positive token; nothing lies across it, so alt is -1
    V = 50
    t, d, tok, res = _rejected_residual(47, V)
    C = np.cumsum(res)
    Z = C[-1]
    last = int(np.nonzero(res > 0)[0][-1])
    uf = _f32_near(1.0, -1)
    u = np.array([[1 - 2 ** -24, uf]], np.float32)
    r = O.verify(t, d, tok, u, 1.0, dtype=F32)
    w = np.float64(uf) * Z
    if abs(C[last] - w) < abs(w - C[last - 1]):
        assert int(r.out_tokens[0, 0]) == last
        assert int(r.alt_token[0]) == -1


# ---------------------------------------------------------- survival margin

@pytest.mark.parametrize("rel,flag", [(5e-7, True), (-5e-7, True), (5e-6, False), (-5e-6, False)])
def test_survival_margin_flag(rel, flag):
    # given confidences: S_j = prod c (fp64 here); tau = S_j (1 + rel) for a j
    # the length walk looks at flags the sequence iff |rel| < 1e-6
    rng = _rng(51)
    B, K, V = 3, 6, 16
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()
    c = rng.uniform(0.6, 0.95, size=(B, K)).astype(np.float32)
    S = np.cumprod(c.astype(np.float64), axis=1)
    jsel = [1, 3, 5]                                     # 0-based positions of the near-tie
    tau = np.array([np.float32(S[b, jsel[b]] * (1 + rel)) for b in range(B)], np.float32)
    u = np.full((B, K + 1), 0.5, np.float32)
    r = O.verify(t, d, np.zeros((B, K), np.int32), u, 1.0, dtype=F32, length_mode=O.LEN_TAU,
                 confidence=c, tau=tau)
    for b in range(B):
        Lref = int((S[b] >= np.float64(tau[b])).sum())
        assert int(r.verify_len[b]) == Lref
        near = abs(S[b, jsel[b]] - np.float64(tau[b])) < 1e-6 * np.float64(tau[b])
        assert near == flag
        assert bool(r.margin[b] & O.MARGIN_SURVIVAL) == flag
        np.testing.assert_allclose(r.survival[b], S[b], rtol=1e-15)


def test_survival_margin_at_the_first_position():
    # clear margins everywhere: no flag; tau within 1e-7 of S_1: flagged
    B, K, V = 1, 6, 16
    rng = _rng(52)
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()
    c = np.array([[0.9, 0.2, 1.0, 1.0, 1.0, 1.0]], np.float32)
    S = np.cumprod(c.astype(np.float64), axis=1)
    tau = np.array([np.float32(0.5)], np.float32)        # L = 1; S_2 = 0.18 decides
    r = O.verify(t, d, np.zeros((B, K), np.int32), np.full((B, K + 1), 0.5, np.float32), 1.0, dtype=F32,
                 length_mode=O.LEN_TAU, confidence=c, tau=tau)
    assert int(r.verify_len[0]) == 1
    assert not (r.margin[0] & O.MARGIN_SURVIVAL)
    # the same tau at S_1 (1 + 1e-7): flagged
    tau2 = np.array([np.float32(S[0, 0] * (1 + 1e-7))], np.float32)
    r2 = O.verify(t, d, np.zeros((B, K), np.int32), np.full((B, K + 1), 0.5, np.float32), 1.0, dtype=F32,
                  length_mode=O.LEN_TAU, confidence=c, tau=tau2)
    assert r2.margin[0] & O.MARGIN_SURVIVAL


# ------------------------------------------------------- admission near tie

def test_admission_exact_tie_is_flagged():
    # speed chosen so that T(m*+1) == T(m*) up to rounding at m*, and T falls
    # steeply after: the oracle stops at m* or m*+1 and flags the near tie
    rng = _rng(61)
    B, K = 6, 4
    c = rng.uniform(0.3, 1.0, size=(B, K)).astype(np.float32)
    S = np.cumprod(c.astype(np.float64), axis=1)
    ranked = sorted(((S[b, j], b, j) for b in range(B) for j in range(K)), key=lambda x: (-x[0], x[1], x[2]))
    n = B * (K + 1) + 1
    mstar = 9
    speed = np.empty(n, np.float64)
    # T(m) = (B + P_m) speed[B + m]: rising until m*, equal at m* + 1, then falling
    P_m = np.concatenate([[0.0], np.cumsum([x[0] for x in ranked])])
    T = np.array([1.0 + 0.01 * m for m in range(mstar + 1)] + [1.0 + 0.01 * mstar] +
                 [0.5] * (B * K - mstar - 1))
    speed[:] = 1.0
    for m in range(B * K + 1):
        speed[B + m] = T[m] / (B + P_m[m])
    r = O.schedule(c, speed)
    assert r.margin
    assert r.admitted in (mstar, mstar + 1)
    # survivals and lengths follow the ranking for whichever stop was taken
    L = np.zeros(B, np.int32)
    for i in range(r.admitted):
        L[ranked[i][1]] += 1
    np.testing.assert_array_equal(r.verify_len, L)


def test_admission_clear_stop_is_not_flagged():
    rng = _rng(62)
    B, K = 6, 4
    c = rng.uniform(0.3, 1.0, size=(B, K)).astype(np.float32)
    S = np.cumprod(c.astype(np.float64), axis=1)
    ranked = sorted(((S[b, j], b, j) for b in range(B) for j in range(K)), key=lambda x: (-x[0], x[1], x[2]))
    P_m = np.concatenate([[0.0], np.cumsum([x[0] for x in ranked])])
    mstar = 9
    T = np.array([1.0 + 0.01 * m for m in range(mstar + 1)] + [0.9] * (B * K - mstar))
    speed = np.ones(B * (K + 1) + 1, np.float64)
    for m in range(B * K + 1):
        speed[B + m] = T[m] / (B + P_m[m])
    r = O.schedule(c, speed)
    assert not r.margin
    assert r.admitted == mstar
