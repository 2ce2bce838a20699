"""GPU parity for bf16 rows whose pairs of elements are far apart.

bf16 logits arrive as 32-bit words holding two elements each (the even index
in the low half, the odd index in the high half).  These rows put the largest
logits in one half of every pair, move every logit far below or above zero, or
fill one half of every pair with -inf, at temperatures where m c is large; the
outputs must match the oracle, which sees the elements one at a time.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Workload("reference", B=6, K=4, V=40000, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                      sigma_first=0.4, sigma_last=0.9, temperature=1.0, seed=71)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _shift_odd(a: np.ndarray, shift: float) -> np.ndarray:
    """bf16 rows with every odd-index logit moved by `shift` (-inf: set to -inf)."""
    f = synth.bf16_bits_to_f32(a).copy()
    if np.isinf(shift):
        f[..., 1::2] = -np.inf
    else:
        f[..., 1::2] += np.float32(shift)
    return _bf16_bits(f)


def _check(name, prob, T=1.0):
    from draft_verification_amd import device as D
    w = prob.w
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} T={T}", flush=True)
    res = D.run_once(D.from_problem(prob))
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, res, orc, dtype=w.dtype, greedy=False, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    assert int(res["device_status"][0]) == 0


@pytest.mark.parametrize("n,shift", enumerate([-2.0, -20.0, -50.0, -np.inf]))
def test_high_halves_below_the_low_halves(n, shift):
    prob = synth.make_problem(BASE.with_(seed=71 + n))
    prob.target = _shift_odd(prob.target, shift)
    prob.draft = _shift_odd(prob.draft, shift)
    _check(f"odd logits {shift:+}", prob)


def test_low_halves_minus_infinity():
    # the even-index elements are -inf: every word reads as its high element
    # with all-ones noise bits below it
    prob = synth.make_problem(BASE.with_(seed=77))
    for name in ("target", "draft"):
        f = synth.bf16_bits_to_f32(getattr(prob, name)).copy()
        f[..., 0::2] = -np.inf
        setattr(prob, name, _bf16_bits(f))
    _check("even logits -inf", prob)


@pytest.mark.parametrize("offset", [-40.0, 40.0])
def test_rows_of_one_sign(offset):
    # every logit negative (the smallest bits are the maximum) or positive
    prob = synth.make_problem(BASE.with_(seed=79 + int(offset > 0)))
    for name in ("target", "draft"):
        f = synth.bf16_bits_to_f32(getattr(prob, name)) + np.float32(offset)
        setattr(prob, name, _bf16_bits(f))
    _check(f"logits {offset:+}", prob)


def test_large_logits_at_low_temperature():
    # logits near 50 at T = 0.25: m c is large and the terms span the whole
    # fp32 range below the maximum
    prob = synth.make_problem(BASE.with_(seed=78, temperature=0.25))
    for name in ("target", "draft"):
        f = synth.bf16_bits_to_f32(getattr(prob, name)) * np.float32(3.0) + np.float32(50.0)
        setattr(prob, name, _bf16_bits(f))
    _check("large logits T=0.25", prob, T=0.25)
