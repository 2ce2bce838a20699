"""The seeded input generator: Philox pinned to its published known answers,
C and Python transcriptions agree, uniforms have the stated exact form, and
drafted tokens follow softmax(draft / T)."""
import os

import numpy as np
import pytest
from scipy import special, stats

from synth import philox_ref, synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w = [int(x, 16) for x in line.split()]
        yield w[0:4], w[4:6], w[6:10]


@pytest.mark.parametrize("ctr,key,want", list(_kat_rows()))
def test_philox_known_answers(ctr, key, want):
    assert synth.philox4x32_10(ctr, key) == want
    assert philox_ref.philox4x32_10(ctr, key) == want


def test_c_and_python_twins_agree():
    for seed, row, stream in [(1, 0, 1), (7, 123, 5), (2**31 + 5, 99999, 3)]:
        words = synth.philox_words(seed, row, stream, 64)
        for c in range(64):
            ref = philox_ref.philox4x32_10((c, row, stream, 0), (seed, 0))
            assert list(words[4 * c:4 * c + 4]) == ref


def test_uniform_exact_form_and_twin():
    u = synth.uniforms(3, 4099)
    k = (u.astype(np.float64) * 2 ** 24 - 1) / 2
    assert np.all(k == np.round(k)) and np.all(u > 0) and np.all(u < 1)
    for i in (0, 1, 2, 3, 4, 1000, 4098):
        assert float(u[i]) == philox_ref.uniform_u24(3, i)


def test_uniforms_are_uniform():
    u = synth.uniforms(11, 200000).astype(np.float64)
    counts = np.histogram(u, bins=50, range=(0, 1))[0]
    assert stats.chisquare(counts).pvalue > 1e-4


def test_problem_is_deterministic_and_shaped():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.make_problem(w), synth.make_problem(w)
    assert a.target.shape == (4, 5, 1024) and a.draft.shape == (4, 4, 1024)
    assert np.array_equal(a.target, b.target) and np.array_equal(a.draft, b.draft)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.uniforms, b.uniforms)
    c = synth.make_problem(w.with_(seed=9))
    assert not np.array_equal(a.uniforms, c.uniforms)


def test_planted_maximum_is_the_argmax():
    w = synth.WORKLOADS["greedy1024"].with_(B=8, V=4096)
    p = synth.make_problem(w)
    t = synth.bf16_bits_to_f32(p.target)
    am = t.argmax(axis=2)
    assert np.all(t.max(axis=2) == 8.0)
    # a matched draft token equals the planted argmax; the mismatch rate is about 0.2
    match = (p.tokens == am[:, :-1]).mean()
    assert 0.6 < match < 0.95


def test_zipf_rows_are_permuted_ranks():
    w = synth.WORKLOADS["zipf64"].with_(B=2, K=2, V=4096, zipf_jitter=0.0)
    p = synth.make_problem(w)
    t = synth.bf16_bits_to_f32(p.target).astype(np.float64)
    # without jitter the sorted row is -s ln(1..V) rounded to bf16
    want = np.sort(-1.1 * np.log(np.arange(1, 4097)))
    got = np.sort(t[0, 0])
    assert np.max(np.abs(got - want)) < 0.02 * np.max(np.abs(want)) + 1e-6


def test_draft_tokens_follow_softmax_of_draft():
    # many rows, small vocabulary: sampled-token counts against summed probabilities
    w = synth.WORKLOADS["tiny"].with_(B=20000, K=1, V=6, temperature=0.8, sigma_first=0.5, sigma_last=0.5)
    p = synth.make_problem(w)
    d = p.draft[:, 0, :].astype(np.float64)
    q = special.softmax(d / 0.8, axis=1)
    expected = q.sum(axis=0)
    counts = np.bincount(p.tokens[:, 0], minlength=6)
    assert stats.chisquare(counts, expected).pvalue > 1e-4


def test_admission_inputs_are_seeded_and_in_range():
    c1, s1 = synth.admission_inputs(3, 8, 5)
    c2, s2 = synth.admission_inputs(3, 8, 5)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    assert c1.shape == (8, 5) and c1.dtype == np.float32
    assert (c1 >= 0.3).all() and (c1 < 1.0).all()
    assert s1.size == 8 * 6 + 1 and (np.diff(s1) < 0).all()


def test_greedy_drafter_tokens_are_the_draft_rows_first_maximum():
    w = synth.WORKLOADS["tiny"].with_(B=6, K=3, V=700, dtype=synth.BF16, token_mode=2, seed=71)
    prob = synth.make_problem(w)
    d = synth.bf16_bits_to_f32(prob.draft)
    np.testing.assert_array_equal(prob.tokens, np.argmax(d, axis=2))
