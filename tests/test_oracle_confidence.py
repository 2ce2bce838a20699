"""Pins of the oracle's calibrated, causally delayed confidences (umans.ai
blog, "2. Verify smarter": per-position temperatures, confidence from two steps
earlier; zhichai.net, "Under the hood": Sequential Temperature Scaling).

Expected values come from scipy's expit and from the definition of a delay
line (the value handed over at step t is the one measured at step t - delay);
none comes from the oracle or the GPU path."""
import numpy as np
import pytest
from scipy import special

from oracle import oracle as O


def _steps(seed, n, B, K, scale=3.0):
    rng = np.random.default_rng(seed)
    return [(scale * rng.standard_normal((B, K))).astype(np.float32) for _ in range(n)]


def test_calibration_is_expit_of_scaled_logits():
    z = _steps(1, 1, 40, 7)
    T = np.array([0.5, 0.8, 1.0, 1.3, 2.0, 3.5, 10.0])
    now, out, bad = O.calibrated_confidence_steps(z, T, delay=0, c_default=0.0)
    want = special.expit(z[0].astype(np.float64) / T).astype(np.float32)
    np.testing.assert_array_equal(now[0], want)
    np.testing.assert_array_equal(out[0], want)      # delay 0 hands over the current value
    assert not bad[0]


@pytest.mark.parametrize("delay", [1, 2, 3])
def test_delay_line(delay):
    z = _steps(2, 7, 12, 5)
    T = np.linspace(0.7, 1.9, 5)
    now, out, _ = O.calibrated_confidence_steps(z, T, delay=delay, c_default=0.25)
    for t in range(7):
        want = now[t - delay] if t >= delay else np.full((12, 5), 0.25, np.float32)
        np.testing.assert_array_equal(out[t], want)


def test_reset_starts_a_slot_over():
    z = _steps(3, 6, 4, 3)
    T = np.ones(3)
    resets = [None, None, None, np.array([0, 1, 0, 0], bool), None, np.array([0, 0, 1, 0], bool)]
    now, out, _ = O.calibrated_confidence_steps(z, T, delay=2, c_default=0.0, resets=resets)
    # slot 1 reset at step 3: default at steps 3 and 4, then the value of step 3
    np.testing.assert_array_equal(out[3][1], 0.0)
    np.testing.assert_array_equal(out[4][1], 0.0)
    np.testing.assert_array_equal(out[5][1], now[3][1])
    # slot 2 reset at step 5: default again although it had history
    np.testing.assert_array_equal(out[5][2], 0.0)
    # untouched slot 0 is a plain delay line
    np.testing.assert_array_equal(out[5][0], now[3][0])


def test_decision_is_causal():
    # what is handed over at step t does not depend on logits of steps after t - delay
    z = _steps(4, 6, 8, 4)
    T = np.full(4, 1.2)
    _, out1, _ = O.calibrated_confidence_steps(z, T, delay=2, c_default=0.1)
    z2 = [x.copy() for x in z]
    z2[4] += 5.0
    z2[5] -= 5.0
    _, out2, _ = O.calibrated_confidence_steps(z2, T, delay=2, c_default=0.1)
    for t in range(6):
        np.testing.assert_array_equal(out1[t], out2[t])


def test_temperature_ordering_and_limits():
    # a larger temperature pulls every confidence towards 1/2; z = 0 gives 1/2 exactly
    z = [np.array([[-4.0, -1.0, 0.0, 1.0, 4.0]], np.float32)]
    lo, _, _ = O.calibrated_confidence_steps(z, np.full(5, 0.5), delay=0, c_default=0.0)
    hi, _, _ = O.calibrated_confidence_steps(z, np.full(5, 4.0), delay=0, c_default=0.0)
    assert lo[0][0, 2] == 0.5 and hi[0][0, 2] == 0.5
    assert np.all(np.abs(hi[0] - 0.5) <= np.abs(lo[0] - 0.5))
    big = [np.array([[-1e4, 1e4]], np.float32)]
    n, _, _ = O.calibrated_confidence_steps(big, np.ones(2), delay=0, c_default=0.0)
    np.testing.assert_array_equal(n[0], [[0.0, 1.0]])


def test_invalid_temperature_gives_zero_and_flags():
    z = _steps(5, 1, 3, 3)
    now, _, bad = O.calibrated_confidence_steps(z, np.array([1.0, 0.0, np.nan]), delay=0, c_default=0.0)
    assert bad[0]
    np.testing.assert_array_equal(now[0][:, 1:], 0.0)
