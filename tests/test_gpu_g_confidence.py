"""GPU parity of calibrated, causally delayed confidences (spec_verify_confidence)
with the oracle over several consecutive calls: the calibrated values within one
fp32 ulp (the device takes e^x in fp64 through its own exp2, the oracle through
libm), the hand-over from `delay` calls earlier and the slot resets exactly."""
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


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _steps(seed, n, Bn, K):
    rng = np.random.default_rng(seed)
    z = [(3.0 * rng.standard_normal((Bn, K))).astype(np.float32) for _ in range(n)]
    resets = [None] + [rng.random(Bn) < 0.15 for _ in range(n - 1)]
    return z, resets


def _run_steps(sv, z, T, resets, delay, c_default):
    B = _B()
    dev = torch.device("cuda")
    Bn, K = z[0].shape
    T_d = torch.from_numpy(np.asarray(T, np.float32)).to(dev)
    nows, outs, stats = [], [], []
    for t, zt in enumerate(z):
        z_d = torch.from_numpy(zt).to(dev)
        r_d = None if resets[t] is None else torch.from_numpy(resets[t].astype(np.int32)).to(dev)
        now = torch.full((Bn, K), -1.0, dtype=torch.float32, device=dev)
        out = torch.full((Bn, K), -1.0, dtype=torch.float32, device=dev)
        st = torch.full((1,), -1, dtype=torch.int32, device=dev)
        sv.confidence(B.make_conf_args(Bn, K, conf_logits=z_d, temperature=T_d, conf_out=out, delay=delay,
                                       c_default=c_default, reset=r_d, conf_now=now, device_status=st))
        torch.cuda.synchronize()
        nows.append(now.cpu().numpy())
        outs.append(out.cpu().numpy())
        stats.append(int(st.item()))
    return nows, outs, stats


@pytest.mark.parametrize("delay", [0, 1, 2, 4])
def test_steps_match_the_oracle(delay):
    B = _B()
    Bn, K = 300, 16
    sv = B.SpecVerify(Bn, K, 1024, B.SV_BF16, 0)
    z, resets = _steps(100 + delay, 7, Bn, K)
    T = np.linspace(0.6, 2.5, K).astype(np.float32)
    g_now, g_out, g_st = _run_steps(sv, z, T, resets, delay, 0.125)
    sv.close()
    o_now, o_out, o_bad = O.calibrated_confidence_steps(z, T, delay, 0.125, resets)
    for t in range(len(z)):
        assert _ulps(g_now[t], o_now[t]).max() <= 1, t
        # the hand-over picks the same step (or the default) for every slot
        d = _ulps(g_out[t], o_out[t])
        assert d.max() <= 1, t
        assert g_st[t] == 0 and not o_bad[t]
    print(f"[conf] delay {delay}: exact {np.mean([np.mean(_ulps(a, b) == 0) for a, b in zip(g_now, o_now)]):.6f}",
          flush=True)


def test_invalid_temperature_and_status_clears():
    B = _B()
    sv = B.SpecVerify(8, 4, 1024, B.SV_BF16, 0)
    z, _ = _steps(7, 2, 8, 4)
    T = np.array([1.0, 0.0, -2.0, np.nan], np.float32)
    g_now, _, g_st = _run_steps(sv, z[:1], T, [None], 0, 0.0)
    assert g_st[0] == B.SV_STATUS_BAD_INPUT
    assert (g_now[0][:, 1:] == 0.0).all()
    g_now, _, g_st = _run_steps(sv, z[1:], np.ones(4, np.float32), [None], 0, 0.0)
    assert g_st[0] == 0
    sv.close()


def test_confidence_schedule_verify_chain():
    """Three calls as an engine would make them at one step: delayed calibrated
    confidences -> admission -> verification, against the oracle's three
    definitions chained on the host."""
    from draft_verification_amd import device as D
    B = _B()
    w = synth.WORKLOADS["tiny"].with_(B=48, K=6, V=4000, seed=91)
    prob = synth.make_problem(w)
    sv = B.SpecVerify(w.B, w.K, w.V, w.dtype, 0)
    dev = torch.device("cuda")
    rng = np.random.default_rng(91)
    z = [(1.5 + rng.standard_normal((w.B, w.K))).astype(np.float32) for _ in range(3)]
    T = np.linspace(0.8, 1.6, w.K).astype(np.float32)
    T_d = torch.from_numpy(T).to(dev)
    conf = torch.empty((w.B, w.K), dtype=torch.float32, device=dev)
    for zt in z:   # two steps of history, then the step that is verified
        sv.confidence(B.make_conf_args(w.B, w.K, conf_logits=torch.from_numpy(zt).to(dev), temperature=T_d,
                                       conf_out=conf, delay=2, c_default=0.0))
    n = np.arange(w.B * (w.K + 1) + 1, dtype=np.float64)
    speed = 1.0 / (2.0 + 0.04 * n)
    vl = torch.empty(w.B, dtype=torch.int32, device=dev)
    sv.schedule(B.make_sched_args(w.B, w.K, confidence=conf, speed=torch.from_numpy(speed).to(dev),
                                  n_speed=speed.size, verify_len_out=vl))
    dp = D.from_problem(prob)
    a = dp.args()
    a.verify_len_in = int(vl.data_ptr())
    sv.run(a)
    res = dp.fetch()
    sv.close()
    _, o_out, _ = O.calibrated_confidence_steps(z, T, 2, 0.0)
    g_conf = conf.cpu().numpy()
    assert _ulps(g_conf, o_out[-1]).max() <= 1
    # the oracle's own chain: its calibrated, delayed confidences feed its
    # admission rule, whose lengths feed its verification; nothing is taken
    # from the device.  The device's confidences may differ by one fp32 ulp,
    # which can only change the admission where two ranked survivals at the
    # stop are that close: then the admitted count must still agree.
    o_conf = np.asarray(o_out[-1], np.float32)
    o_s = O.schedule(o_conf, speed)
    assert not o_s.margin and o_s.admitted > 0
    g_L = vl.cpu().numpy()
    S = np.sort(o_s.survival.reshape(-1))[::-1]
    m = o_s.admitted
    boundary_tie = 0 < m < S.size and abs(S[m - 1] - S[m]) <= 4 * np.spacing(np.float32(S[m - 1]))
    if boundary_tie:
        assert int(g_L.sum()) == m
    else:
        np.testing.assert_array_equal(g_L, o_s.verify_len)
    prob.verify_len = o_s.verify_len.astype(np.int32)
    same = np.nonzero(g_L == o_s.verify_len)[0]    # every sequence unless the stop is a near tie
    orc = O.verify_problem(prob, seqs=same, all_rows=True)
    rep = PU.compare("confidence -> schedule -> verify", res, orc, dtype=w.dtype, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
