"""End-to-end pins of the oracle: emitted tokens follow the target distribution.

The pages state that the acceptance rule is built so that accepted tokens follow
the target model's distribution exactly (umans.ai blog, "Speculative decoding,
briefly"; zhichai.net, "Why LLMs speak so slowly"), and that even the
load-dependent truncation keeps this property when the length decision does not
look at the sampled tokens (umans.ai blog, "2. Verify smarter").

With synthetic rows that do not depend on the prefix, the target "model" emits
t_j ~ p_j independently, so for every position j and every prefix w:
    P(t_j = v | at least j tokens emitted, t_<j = w) = p_j(v).

Exact check (V <= 4, K <= 3): the oracle's output is piecewise constant in the
uniforms.  The cells are delimited by the acceptance ratios (for u_1..u_K) and
by the steps of the final draw's CDF (for u_{K+1}); the test computes those cell
edges itself (scipy softmax, fp64), evaluates the oracle once at the midpoint
of every cell and weights the result by the cell's volume times the draft
probability of x.  A wrong sign, a dropped term or a wrong row in the oracle
moves some midpoint output and breaks the identity.
"""
import itertools
from collections import defaultdict

import numpy as np
import pytest
from scipy import special, stats

from oracle import oracle as O


def _rows(seed, K, V, scale=1.2, noise=0.9):
    rng = np.random.default_rng(seed)
    t = (scale * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + noise * rng.standard_normal((K, V))).astype(np.float32)
    return t, d


def _cells(masses):
    """(midpoint of the CDF cell, mass share) for every token with mass > 0."""
    Z = masses.sum()
    C = np.concatenate([[0.0], np.cumsum(masses)]) / Z
    return [((C[v] + C[v + 1]) / 2, masses[v] / Z, v) for v in range(len(masses)) if masses[v] > 0]


def _enumerate(t, d, L, T):
    """All (x, u) cell representatives and their probabilities, for verify length L."""
    K, V = d.shape
    p = special.softmax(t.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    q = special.softmax(d.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    toks, us, ws = [], [], []
    for x in itertools.product(range(V), repeat=K):
        wx = np.prod([q[j, x[j]] for j in range(K)])
        acc = [min(1.0, p[j, x[j]] / q[j, x[j]]) for j in range(K)]
        for a in range(L + 1):
            u = np.full(K + 1, 0.5)
            w = wx
            for j in range(a):
                u[j] = acc[j] / 2
                w *= acc[j]
            if a < L:
                rej = 1.0 - acc[a]
                if rej <= 0:
                    continue
                u[a] = (acc[a] + 1.0) / 2
                w *= rej
                final = np.maximum(p[a] - q[a], 0.0)
            else:
                final = p[L]
            for mid, share, _ in _cells(final):
                uu = u.copy()
                uu[K] = mid
                toks.append(x)
                us.append(uu)
                ws.append(w * share)
    return (np.array(toks, np.int32), np.array(us, np.float32), np.array(ws), p, q)


def _check_lossless(out_tokens, accepted, weights, p, L):
    total = weights.sum()
    assert abs(total - 1.0) < 1e-12
    K1, V = p.shape
    # joint law of emitted sequences
    joint = defaultdict(float)
    for toks, a, w in zip(out_tokens, accepted, weights):
        joint[tuple(int(v) for v in toks[:a + 1])] += w
    for j in range(L + 1):
        cond = defaultdict(lambda: np.zeros(V))
        for seq, w in joint.items():
            if len(seq) > j:
                cond[seq[:j]][seq[j]] += w
        assert cond, "no sequence emits position %d" % j
        for prefix, m in cond.items():
            np.testing.assert_allclose(m / m.sum(), p[j], rtol=0, atol=1e-12)
    return joint


def _expected_emitted(p, q, L):
    alpha = np.minimum(p[:len(q)], q).sum(axis=1)
    return 1.0 + sum(np.prod(alpha[:j]) for j in range(1, L + 1))


@pytest.mark.parametrize("V,K", [(2, 1), (3, 2), (4, 2), (3, 3)])
@pytest.mark.parametrize("L_choice", ["full", "short", "zero"])
def test_exact_losslessness_fixed_length(V, K, L_choice):
    t, d = _rows(100 + 10 * V + K, K, V)
    L = {"full": K, "short": max(K - 1, 0), "zero": 0}[L_choice]
    T = 1.0 if V != 3 else 0.8
    toks, us, ws, p, q = _enumerate(t, d, L, T)
    B = len(ws)
    r = O.verify(t, d, toks, us, T, dtype=O.F32, verify_len=np.full(B, L, np.int32))
    assert np.all(r.margin == 0)
    _check_lossless(r.out_tokens, r.accepted_len, ws, p, L)
    mean_emitted = float(np.dot(ws, r.accepted_len + 1))
    assert abs(mean_emitted - _expected_emitted(p, q, L)) < 1e-12


@pytest.mark.parametrize("mode", ["given_c", "max_q"])
def test_exact_losslessness_confidence_scheduled(mode):
    V, K, T = 3, 3, 1.0
    t, d = _rows(7, K, V, scale=2.0, noise=0.4)
    q = special.softmax(d.astype(np.float64), axis=1)
    if mode == "given_c":
        c = np.array([0.9, 0.7, 0.5], np.float32)
        tau = 0.5
        S = np.cumprod(c.astype(np.float64))
    else:
        c = None
        S = np.cumprod(q.max(axis=1))
        tau = float(np.float32((S[0] + S[1]) / 2))   # between S_1 and S_2 -> L = 1
    L = int(max([0] + [j + 1 for j in range(K) if S[j] >= tau]))
    toks, us, ws, p, q = _enumerate(t, d, L, T)
    B = len(ws)
    conf = None if c is None else np.tile(c, (B, 1))
    r = O.verify(t, d, toks, us, T, dtype=O.F32, length_mode=O.LEN_TAU, confidence=conf,
                 tau=np.full(B, tau, np.float32))
    assert np.all(r.verify_len == L)
    _check_lossless(r.out_tokens, r.accepted_len, ws, p, L)


# ------------------------------------------------------------- chi-square --

def _sample_problem(seed, K, V, N, T=1.0):
    t, d = _rows(seed, K, V, scale=1.0, noise=0.7)
    rng = np.random.default_rng(seed + 1)
    q = special.softmax(d.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    toks = np.empty((N, K), np.int32)
    for j in range(K):
        c = np.cumsum(q[j])
        c[-1] = 1.0
        toks[:, j] = np.searchsorted(c, rng.random(N), side="right")
    u = np.clip(rng.random((N, K + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    p = special.softmax(t.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    return t, d, toks, u, p, q


def _chi2_pvalues(out_tokens, accepted, p, L):
    pv = []
    for j in range(L + 1):
        sel = accepted >= j
        counts = np.bincount(out_tokens[sel, j], minlength=p.shape[1])
        pv.append(stats.chisquare(counts, p[j] * sel.sum()).pvalue)
    return pv


def test_chi_square_fixed_length():
    K, V, N = 4, 8, 300000
    t, d, toks, u, p, q = _sample_problem(21, K, V, N)
    r = O.verify(t, d, toks, u, 1.0, dtype=O.F32)
    pv = _chi2_pvalues(r.out_tokens, r.accepted_len, p, K)
    assert min(pv) > 1e-4, pv


def test_chi_square_tau_mode_max_q():
    K, V, N, T = 4, 8, 300000, 0.9
    t, d, toks, u, p, q = _sample_problem(22, K, V, N, T)
    S = np.cumprod(q.max(axis=1))
    tau = float(S[2]) * 0.999                      # L = 3
    r = O.verify(t, d, toks, u, T, dtype=O.F32, length_mode=O.LEN_TAU, tau=np.full(N, tau, np.float32))
    assert np.all(r.verify_len == 3)
    pv = _chi2_pvalues(r.out_tokens, r.accepted_len, p, 3)
    assert min(pv) > 1e-4, pv


def test_leaky_length_rule_is_detected():
    # Negative control: a confidence that looks at the sampled token
    # (c_j = q_j(x_j)) lets the length decision depend on the draft sample,
    # which the pages warn breaks losslessness ("2. Verify smarter").  The same
    # chi-square test must reject it.
    K, V, N = 2, 8, 300000
    t, d, toks, u, p, q = _sample_problem(23, K, V, N)
    leak = np.stack([q[j, toks[:, j]] for j in range(K)], axis=1).astype(np.float32)
    tau = float(np.median(leak[:, 0]))
    r = O.verify(t, d, toks, u, 1.0, dtype=O.F32, length_mode=O.LEN_TAU, confidence=leak,
                 tau=np.full(N, tau, np.float32))
    sel = np.ones(N, bool)
    counts = np.bincount(r.out_tokens[sel, 0], minlength=V)
    assert stats.chisquare(counts, p[0] * N).pvalue < 1e-8
