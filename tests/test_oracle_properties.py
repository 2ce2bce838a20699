"""Structural properties of the oracle's outputs on random small problems
(hypothesis, derandomized).  They follow from the construction itself, not
from the oracle:

- the emitted block is the accepted prefix of the drafted tokens, one final
  token and -1 padding; 0 <= a <= L <= K;
- greedy: the final token is the argmax of target row a+1 (lowest id on ties)
  and every accepted token equals the argmax of its row;
- sampling: the final token has positive mass under its draw: max(0, p - q) for
  a replacement, p for a bonus.  The reported residual mass is in [0, 1] and
  the reported probability is in (0, 1];
- a q that equals p accepts every verified position (the ratio is 1 and u < 1).
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import oracle as O

F32 = O.F32


def _softmax(z):
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


problems = st.fixed_dictionaries({
    "B": st.integers(1, 5),
    "K": st.integers(1, 5),
    "V": st.integers(1, 40),
    "T": st.sampled_from([0.0, 0.5, 1.0, 2.0]),
    "scale": st.sampled_from([0.0, 0.5, 2.0, 6.0]),
    "noise": st.sampled_from([0.0, 0.1, 1.0, 3.0]),
    "fixed": st.booleans(),
    "seed": st.integers(0, 2 ** 31 - 1),
})


def _make(pr):
    rng = np.random.default_rng(pr["seed"])
    B, K, V = pr["B"], pr["K"], pr["V"]
    t = (pr["scale"] * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d = (t[:, :K, :] + pr["noise"] * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    u = np.clip(rng.random((B, K + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    vl = rng.integers(0, K + 1, size=B).astype(np.int32) if pr["fixed"] else None
    return t, d, tok, u, vl


@settings(max_examples=300, deadline=None, derandomize=True)
@given(problems)
def test_emitted_block_structure(pr):
    t, d, tok, u, vl = _make(pr)
    T = pr["T"]
    r = O.verify(t, d, tok, u if T > 0 else None, T, dtype=F32, verify_len=vl)
    B, K, V = pr["B"], pr["K"], pr["V"]
    for b in range(B):
        a, L = int(r.accepted_len[b]), int(r.verify_len[b])
        assert 0 <= a <= L <= K
        if vl is not None:
            assert L == int(vl[b])
        out = r.out_tokens[b]
        assert np.array_equal(out[:a], tok[b, :a])
        assert 0 <= int(out[a]) < V
        assert np.all(out[a + 1:] == -1)
        y, j = int(out[a]), a  # the final token is drawn from row a+1 (0-based row a)
        if T == 0.0:
            row = t[b, j].astype(np.float64)
            assert y == int(np.argmax(row))
            for i in range(a):
                assert int(tok[b, i]) == int(np.argmax(t[b, i].astype(np.float64)))
            continue
        p = _softmax(t[b, j].astype(np.float64) / T)
        z = float(r.residual_mass[b])
        py = float(r.sampled_prob[b])
        assert 0.0 < py <= 1.0 + 1e-12
        if a < L:  # replacement after a rejection at position a+1
            q = _softmax(d[b, j].astype(np.float64) / T)
            assert 0.0 <= z <= 1.0 + 1e-12
            if z > 0.0:
                assert p[y] - q[y] > -1e-12, (p[y], q[y])
        else:  # bonus
            assert z == 1.0
            assert p[y] > 0.0


@settings(max_examples=100, deadline=None, derandomize=True)
@given(problems)
def test_draft_equal_to_target_accepts_every_verified_position(pr):
    t, _, tok, u, vl = _make(pr)
    K = pr["K"]
    if pr["T"] == 0.0:
        return
    r = O.verify(t, t[:, :K, :].copy(), tok, u, pr["T"], dtype=F32, verify_len=vl)
    np.testing.assert_array_equal(r.accepted_len, r.verify_len)
