"""GPU parity of the load-aware admission (spec_verify_schedule) with the oracle.

Outside the oracle's margin cases (a stop decision within 1e-9 relative) the
admitted count, every L_b, the smallest admitted survival and the survivals
themselves match bit for bit; the expected rate within 1e-12 relative (the
prefix sums are added in a different fixed order).
"""
import math

import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _B():
    from draft_verification_amd import binding
    return binding


def _latency_speed(n_max, a, b):
    n = np.arange(n_max + 1, dtype=np.float64)
    return 1.0 / (a + b * n)


def _run_sched(sv, conf, speed):
    B = _B()
    Bn, K = conf.shape
    dev = torch.device("cuda")
    c_d = torch.from_numpy(np.ascontiguousarray(conf, np.float32)).to(dev)
    s_d = torch.from_numpy(np.ascontiguousarray(speed, np.float64)).to(dev)
    vl = torch.full((max(Bn, 1),), -7, dtype=torch.int32, device=dev)
    surv = torch.full((max(Bn * K, 1),), -1.0, dtype=torch.float32, device=dev)
    adm = torch.full((1,), -1, dtype=torch.int32, device=dev)
    tau = torch.zeros(1, dtype=torch.float32, device=dev)
    exp_ = torch.zeros(1, dtype=torch.float64, device=dev)
    st = torch.full((1,), -1, dtype=torch.int32, device=dev)
    args = B.make_sched_args(Bn, K, confidence=c_d, speed=s_d, n_speed=speed.size, verify_len_out=vl, survival=surv,
                             admitted=adm, tau=tau, expected_rate=exp_, device_status=st)
    sv.schedule(args)
    torch.cuda.synchronize()
    return dict(verify_len=vl.cpu().numpy()[:Bn], survival=surv.cpu().numpy()[:Bn * K].reshape(Bn, K),
                admitted=int(adm.item()), tau=float(tau.item()), expected=float(exp_.item()), status=int(st.item()))


def _compare(name, g, o):
    print(f"[sched] {name}: admitted gpu {g['admitted']} oracle {o.admitted} margin {o.margin}", flush=True)
    np.testing.assert_array_equal(g["survival"], o.survival.astype(np.float32))
    assert g["status"] == (_B().SV_STATUS_BAD_INPUT if o.bad else 0)
    if o.margin:
        assert g["verify_len"].sum() == g["admitted"]
        return
    assert g["admitted"] == o.admitted
    np.testing.assert_array_equal(g["verify_len"], o.verify_len)
    if o.admitted:
        assert g["tau"] == np.float32(o.tau)
    else:
        assert math.isnan(g["tau"])
    np.testing.assert_allclose(g["expected"], o.expected, rtol=1e-12)


@pytest.fixture(scope="module")
def sv():
    B = _B()
    h = B.SpecVerify(4096, 256, 1024, B.SV_BF16, 0)
    yield h
    h.close()


@pytest.mark.parametrize("a,b", [(20.0, 0.05), (5.0, 0.5), (300.0, 0.2), (1.0, 1e-4)])
def test_random_confidences(sv, a, b):
    rng = np.random.default_rng(int(a * 10 + b * 1000))
    Bn, K = 256, 16
    conf = rng.uniform(0.3, 1.0, size=(Bn, K)).astype(np.float32)
    speed = _latency_speed(Bn * (K + 1), a, b)
    _compare(f"latency a={a} b={b}", _run_sched(sv, conf, speed), O.schedule(conf, speed))


def test_ties_zeros_and_certain_positions(sv):
    rng = np.random.default_rng(7)
    Bn, K = 300, 12
    conf = rng.choice(np.array([0.5, 0.75, 1.0], np.float32), size=(Bn, K))
    conf[5:40, 3] = 0.0
    conf[50:60] = 1.0
    for n0_extra in (0, 17, 900, 3600):
        speed = np.where(np.arange(Bn * (K + 1) + 1) <= Bn + n0_extra, 2.0, 0.0)
        _compare(f"cliff +{n0_extra}", _run_sched(sv, conf, speed), O.schedule(conf, speed))
    speed = _latency_speed(Bn * (K + 1), 4.0, 0.03)
    _compare("ties latency", _run_sched(sv, conf, speed), O.schedule(conf, speed))
    speed = np.full(Bn * (K + 1) + 1, 1.25)
    _compare("ties constant", _run_sched(sv, conf, speed), O.schedule(conf, speed))


@pytest.mark.parametrize("Bn,K", [(1, 1), (1, 16), (3, 5), (1000, 7), (4096, 16), (7, 32), (100, 33), (40, 256)])
def test_shapes(sv, Bn, K):
    rng = np.random.default_rng(Bn * 31 + K)
    conf = rng.uniform(0.0, 1.0, size=(Bn, K)).astype(np.float32) ** 0.3
    speed = _latency_speed(Bn * (K + 1) + 5, 50.0, 0.02)
    _compare(f"B={Bn} K={K}", _run_sched(sv, conf, speed), O.schedule(conf, speed))


def test_bad_confidences_then_clean_call(sv):
    conf = np.array([[0.5, 1.5, 0.5], [np.nan, 0.9, 0.9], [-0.1, 1.0, 1.0], [0.9, 0.9, 0.9]], np.float32)
    speed = np.full(4 * 4 + 1, 1.0)
    _compare("bad", _run_sched(sv, conf, speed), O.schedule(conf, speed))
    good = np.clip(np.nan_to_num(conf, nan=0.0), 0, 1).astype(np.float32)
    g = _run_sched(sv, good, speed)
    assert g["status"] == 0
    _compare("clean after bad", g, O.schedule(good, speed))


def test_deterministic(sv):
    rng = np.random.default_rng(11)
    conf = rng.uniform(0.2, 1.0, size=(512, 16)).astype(np.float32)
    speed = _latency_speed(512 * 17, 10.0, 0.05)
    g1, g2 = _run_sched(sv, conf, speed), _run_sched(sv, conf, speed)
    for k in g1:
        np.testing.assert_array_equal(np.asarray(g1[k]), np.asarray(g2[k]))


def test_schedule_feeds_a_verify_step():
    """Admission decides L_b on the device; the verify step consumes it in fixed
    mode, and the whole is compared with the oracle's admission followed by the
    oracle's verification."""
    from draft_verification_amd import device as D
    B = _B()
    w = synth.WORKLOADS["tiny"].with_(B=64, K=8, V=3000, seed=41)
    prob = synth.make_problem(w)
    rng = np.random.default_rng(41)
    conf = rng.uniform(0.4, 1.0, size=(w.B, w.K)).astype(np.float32)
    speed = _latency_speed(w.B * (w.K + 1), 2.0, 0.05)
    o_s = O.schedule(conf, speed)
    assert not o_s.margin and 0 < o_s.admitted < w.B * w.K
    dp = D.from_problem(prob)
    sv = B.SpecVerify(w.B, w.K, w.V, w.dtype, 0)
    dev = torch.device("cuda")
    c_d = torch.from_numpy(conf).to(dev)
    s_d = torch.from_numpy(speed).to(dev)
    vl = torch.empty(w.B, dtype=torch.int32, device=dev)
    sv.schedule(B.make_sched_args(w.B, w.K, confidence=c_d, speed=s_d, n_speed=speed.size, verify_len_out=vl))
    a = dp.args()
    a.length_mode = B.SV_LEN_FIXED
    a.verify_len_in = int(vl.data_ptr())
    sv.run(a)
    torch.cuda.synchronize()
    res = dp.fetch()
    sv.close()
    np.testing.assert_array_equal(vl.cpu().numpy(), o_s.verify_len)
    prob.verify_len = o_s.verify_len.astype(np.int32)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare("schedule -> verify", res, orc, dtype=w.dtype, greedy=False, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
