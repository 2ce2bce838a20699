"""The parity helper must turn every kind of bad device output into a
mismatch: a NaN residual mass or drawn-token probability, a missing log-sum-exp
or survival of a row the step evaluates, and diagnostics written where the
step has none.  Device outputs here are made from the oracle's own outputs
(rounded to fp32, as the device reports them) with one fault planted at a time.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests import parity_util as PU


def _problem(seed, B=6, K=5, V=64, noise=0.5):
    rng = np.random.default_rng(seed)
    t = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d = (t[:, :K] + noise * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K), dtype=np.int32)
    u = np.clip(rng.random((B, K + 1)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    return t, d, tok, u


def _as_device(orc, B, K, survival=True):
    f = lambda a: np.asarray(a, np.float64).astype(np.float32)
    return {
        "accepted_len": orc.accepted_len.copy(), "out_tokens": orc.out_tokens.copy(),
        "verify_len_out": orc.verify_len.copy(), "lse_target": f(orc.lse_target), "lse_draft": f(orc.lse_draft),
        "survival": f(orc.survival) if survival else np.full((B, K), np.nan, np.float32),
        "residual_mass": f(orc.residual_mass), "sampled_prob": f(orc.sampled_prob),
    }


def _fixed():
    t, d, tok, u = _problem(1)
    orc = O.verify(t, d, tok, u, 1.0, dtype=O.F32)
    return orc, _as_device(orc, *tok.shape)


def _derived():
    t, d, tok, u = _problem(2, noise=0.05)
    B, K = tok.shape
    tau = np.full(B, 0.0, np.float32)
    orc = O.verify(t, d, tok, u, 1.0, dtype=O.F32, length_mode=O.LEN_TAU, tau=tau)
    return orc, _as_device(orc, B, K), tau


def test_clean_copy_passes():
    orc, g = _fixed()
    rep = PU.compare("clean", g, orc, dtype=O.F32)
    assert not rep.mismatches and rep.exact == len(orc.seq)


@pytest.mark.parametrize("field", ["residual_mass", "sampled_prob"])
def test_nan_probability_is_a_mismatch(field):
    orc, g = _fixed()
    b = int(np.nonzero(orc.final_kind != O.FINAL_BAD_INPUT)[0][0])
    g[field][b] = np.nan
    rep = PU.compare("nan", g, orc, dtype=O.F32)
    assert any(m[0] == b for m in rep.mismatches), rep.mismatches
    assert rep.max_rel_prob != rep.max_rel_prob   # the report shows the NaN


def test_inf_probability_is_a_mismatch():
    orc, g = _fixed()
    g["residual_mass"][0] = np.inf
    rep = PU.compare("inf", g, orc, dtype=O.F32)
    assert any(m[0] == 0 for m in rep.mismatches)


def test_missing_lse_target_row_is_a_mismatch():
    orc, g = _fixed()
    b = 0
    g["lse_target"][b, int(orc.accepted_len[b])] = np.nan       # the final draw's row
    rep = PU.compare("lse_t", g, orc, dtype=O.F32)
    assert any(m[1].get("kind") == "lse_target missing" for m in rep.mismatches)


def test_missing_lse_draft_row_is_a_mismatch():
    orc, g = _fixed()
    b = int(np.nonzero(orc.verify_len > 0)[0][0])
    g["lse_draft"][b, 0] = np.nan                                 # position 1 is always tested when L > 0
    rep = PU.compare("lse_d", g, orc, dtype=O.F32)
    assert any(m[1].get("kind") == "lse_draft missing" for m in rep.mismatches)


def test_missing_survival_is_a_mismatch():
    orc, g, tau = _derived()
    b = 0
    g["survival"][b, 0] = np.nan
    rep = PU.compare("surv", g, orc, dtype=O.F32, derived=True, tau=tau)
    assert any(m[1].get("kind") == "survival missing" for m in rep.mismatches)


def test_no_survival_at_all_is_a_mismatch_in_derived_mode():
    t, d, tok, u = _problem(3)
    B, K = tok.shape
    tau = np.full(B, 0.0, np.float32)
    orc = O.verify(t, d, tok, u, 1.0, dtype=O.F32, length_mode=O.LEN_TAU, tau=tau)
    g = _as_device(orc, B, K, survival=False)
    rep = PU.compare("no surv", g, orc, dtype=O.F32, derived=True, tau=tau)
    assert sum(m[1].get("kind") == "survival missing" for m in rep.mismatches) == B


def test_survival_written_in_fixed_mode_is_a_mismatch():
    orc, g = _fixed()
    g["survival"][:] = 0.5
    rep = PU.compare("fixed surv", g, orc, dtype=O.F32)
    assert any(m[1].get("kind") == "survival written in fixed-length mode" for m in rep.mismatches)


def test_wrong_survival_value_is_a_mismatch():
    orc, g, tau = _derived()
    g["survival"][1, 0] *= 1.001
    rep = PU.compare("surv value", g, orc, dtype=O.F32, derived=True, tau=tau)
    assert any(m[1].get("kind") == "survival" for m in rep.mismatches)


def test_derived_without_thresholds_is_refused():
    orc, g, _ = _derived()
    with pytest.raises(ValueError):
        PU.compare("no tau", g, orc, dtype=O.F32, derived=True)
