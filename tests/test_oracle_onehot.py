"""Pins of the oracle's one-hot draft mode: the drafter chose its tokens
greedily, so the draft distribution at position j is the point mass at x_j (the
`draft_sample_method: greedy` option of vLLM's DSpark support, techvisionai
blog, Chapter 7).  Acceptance then has probability p_j(x_j) and the replacement
is p_j with x_j removed and renormalised.

Expected values come from scipy's softmax, numpy's searchsorted, exact
enumeration of the uniforms' cells, and equality with the probability mode fed
one-hot draft logits (itself pinned elsewhere).
"""
import itertools
from collections import defaultdict

import numpy as np
import pytest
from scipy import special

from oracle import oracle as O


def _p(t, T):
    return special.softmax(t.astype(np.float64) / np.float64(np.float32(T)), axis=-1)


def _rows(seed, B, K, V, scale=1.5):
    rng = np.random.default_rng(seed)
    t = (scale * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    # drafted tokens: likely ones (the top few of each target row), as a good drafter's
    x = np.argsort(-t[:, :K, :], axis=2)[:, :, :3]
    pick = rng.integers(0, 3, size=(B, K))
    tok = np.take_along_axis(x, pick[..., None], axis=2)[..., 0].astype(np.int32)
    u = np.clip(rng.random((B, K + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    return t, tok, u


def test_acceptance_probability_is_p_of_x():
    B, K, V, T = 400, 1, 50, 0.9
    t, tok, u = _rows(1, B, K, V)
    r = O.verify(t, None, tok, u, T, dtype=O.F32, draft_mode=O.DRAFT_ONEHOT)
    p = _p(t, T)
    for b in range(B):
        if r.margin[b] & O.MARGIN_ACCEPT:
            continue
        assert r.accepted_len[b] == int(u[b, 0] < p[b, 0, tok[b, 0]])


def test_replacement_is_p_without_x():
    B, K, V, T = 300, 1, 64, 1.0
    t, tok, u = _rows(2, B, K, V)
    u[:, 0] = 1 - 2 ** -24  # reject at position 1 unless p(x) = 1
    r = O.verify(t, None, tok, u, T, dtype=O.F32, draft_mode=O.DRAFT_ONEHOT)
    p = _p(t, T)
    for b in range(B):
        assert r.accepted_len[b] == 0 and r.final_kind[b] == O.FINAL_RESIDUAL
        res = p[b, 0].copy()
        res[tok[b, 0]] = 0.0
        Z = res.sum()
        np.testing.assert_allclose(r.residual_mass[b], 1.0 - p[b, 0, tok[b, 0]], rtol=1e-12)
        if r.margin[b] & O.MARGIN_CDF:
            continue
        y = int(np.searchsorted(np.cumsum(res), np.float64(u[b, K]) * Z, side="right"))
        assert r.out_tokens[b, 0] == y and y != tok[b, 0]
        np.testing.assert_allclose(r.sampled_prob[b], p[b, 0, y] / Z, rtol=1e-10)


def test_derived_confidence_is_one():
    B, K, V = 20, 4, 30
    t, tok, u = _rows(3, B, K, V)
    tau = np.where(np.arange(B) % 2 == 0, 0.7, 1.5).astype(np.float32)
    r = O.verify(t, None, tok, u, 1.0, dtype=O.F32, length_mode=O.LEN_TAU, tau=tau, draft_mode=O.DRAFT_ONEHOT)
    np.testing.assert_array_equal(r.survival, np.ones((B, K)))
    np.testing.assert_array_equal(r.verify_len, np.where(tau <= 1.0, K, 0))
    assert np.isnan(r.lse_draft).all()


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_equals_probability_mode_with_one_hot_draft_logits(T):
    B, K, V = 120, 3, 200
    t, tok, u = _rows(4, B, K, V)
    d = np.full((B, K, V), -np.inf, np.float32)
    for b in range(B):
        for j in range(K):
            d[b, j, tok[b, j]] = 0.0
    r1 = O.verify(t, None, tok, u, T, dtype=O.F32, draft_mode=O.DRAFT_ONEHOT)
    r2 = O.verify(t, d, tok, u, T, dtype=O.F32)
    np.testing.assert_array_equal(r1.accepted_len, r2.accepted_len)
    np.testing.assert_array_equal(r1.out_tokens, r2.out_tokens)
    np.testing.assert_array_equal(r1.final_kind, r2.final_kind)
    np.testing.assert_allclose(r1.residual_mass, r2.residual_mass, rtol=1e-13)
    np.testing.assert_allclose(r1.sampled_prob, r2.sampled_prob, rtol=1e-12)


def _cells(masses):
    Z = masses.sum()
    C = np.concatenate([[0.0], np.cumsum(masses)]) / Z
    return [((C[v] + C[v + 1]) / 2, masses[v] / Z) for v in range(len(masses)) if masses[v] > 0]


@pytest.mark.parametrize("V,K", [(2, 1), (3, 2), (4, 3)])
def test_exact_losslessness(V, K):
    # For every fixed drafted block x and every prefix of it, the emitted token
    # at position j follows p_j exactly.  The output is piecewise constant in the
    # uniforms; each cell is evaluated once at its midpoint.
    rng = np.random.default_rng(50 + V)
    t = (1.3 * rng.standard_normal((K + 1, V))).astype(np.float32)
    p = _p(t, 1.0)
    for x in itertools.product(range(V), repeat=K):
        acc = [p[j, x[j]] for j in range(K)]
        toks, us, ws = [], [], []
        for a in range(K + 1):
            u = np.full(K + 1, 0.5)
            w = 1.0
            for j in range(a):
                u[j] = acc[j] / 2
                w *= acc[j]
            if a < K:
                u[a] = (acc[a] + 1.0) / 2
                w *= 1.0 - acc[a]
                final = p[a].copy()
                final[x[a]] = 0.0
            else:
                final = p[K]
            for mid, share in _cells(final):
                uu = u.copy()
                uu[K] = mid
                toks.append(x)
                us.append(uu)
                ws.append(w * share)
        toks = np.array(toks, np.int32)
        r = O.verify(np.broadcast_to(t, (len(ws), K + 1, V)).copy(), None, toks, np.array(us, np.float32), 1.0,
                     dtype=O.F32, draft_mode=O.DRAFT_ONEHOT)
        ws = np.array(ws)
        assert abs(ws.sum() - 1.0) < 1e-12
        joint = defaultdict(float)
        for o, a, w in zip(r.out_tokens, r.accepted_len, ws):
            joint[tuple(int(v) for v in o[:a + 1])] += w
        for j in range(K + 1):
            cond = defaultdict(lambda: np.zeros(V))
            for seq, w in joint.items():
                if len(seq) > j:
                    cond[seq[:j]][seq[j]] += w
            for prefix, m in cond.items():
                np.testing.assert_allclose(m / m.sum(), p[j], rtol=0, atol=1e-12)
