"""GPU properties: bitwise determinism, batch invariance, and the emitted
distribution (chi-square) on many sequences sharing one set of rows."""
import numpy as np
import pytest
from scipy import special, stats

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _D():
    from draft_verification_amd import device as D
    return D


def test_bitwise_determinism():
    D = _D()
    w = synth.WORKLOADS["zipf64"].with_(B=32)
    prob = synth.make_problem(w)
    print("[case] determinism zipf B32", flush=True)
    dp = D.from_problem(prob)
    sv = D.handle_for(dp)
    outs = []
    for _ in range(5):
        sv.run(dp.args())
        outs.append(dp.fetch())
    sv.close()
    for o in outs[1:]:
        assert not PU.same_outputs(o, outs[0])
    for o in outs:
        assert not PU.check_streamed(o, w.K, w.V, 2, two_rows=True)


@pytest.mark.parametrize("name,derived", [("zipf64", False), ("greedy1024", False), ("sched256", True)])
def test_timed_runs_match_untimed_runs(name, derived):
    # per-kernel timing launches every kernel with events attached to the
    # dispatch; the outputs must not change, and every kernel of the step must
    # report a positive time (the residual pass only where it runs)
    D = _D()
    w = synth.WORKLOADS[name].with_(B=24)
    if derived:
        w = w.with_(tau_choices=(0.0,))
    prob = synth.make_problem(w)
    print(f"[case] timed runs {name} B24", flush=True)
    dp = D.from_problem(prob)
    sv = D.handle_for(dp)
    sv.run(dp.args())
    ref = dp.fetch()
    sv.timing_begin(3)
    for _ in range(3):
        sv.run(dp.args())
    timed = dp.fetch()
    ms, runs = sv.timing_end()
    sv.close()
    assert runs == 3
    assert not PU.same_outputs(ref, timed)
    greedy = w.temperature == 0
    for k in ("sv_plan", "sv_stream", "sv_draw"):
        assert ms[k] > 0.0, (k, ms)
    assert (ms["sv_resid"] > 0.0) == (not greedy), ms
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(f"timed {name}", timed, orc, dtype=w.dtype, greedy=greedy, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]


def test_two_handles_on_two_streams():
    # separate handles are independent: two steps enqueued on two streams at
    # once give the same outputs as each run alone on the default stream
    D = _D()
    probs = [synth.make_problem(synth.WORKLOADS["zipf64"].with_(B=48, seed=71)),
             synth.make_problem(synth.WORKLOADS["peaked512"].with_(B=40, K=12, V=30000, seed=72))]
    print("[case] two handles on two streams", flush=True)
    dps = [D.from_problem(p) for p in probs]
    hs = [D.handle_for(dp) for dp in dps]
    alone = []
    for h, dp in zip(hs, dps):
        h.run(dp.args())
        alone.append(dp.fetch())
        dp.alloc_outputs(True, "cuda:0")  # fresh output buffers (sentinels) for the concurrent runs
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ev = torch.cuda.Event()
    ev.record()
    for st in streams:
        st.wait_event(ev)
    for rep in range(3):
        for h, dp, st in zip(hs, dps, streams):
            h.run(dp.args(), st.cuda_stream)
    torch.cuda.synchronize()
    for dp, ref in zip(dps, alone):
        got = dp.fetch()
        assert not PU.same_outputs(ref, got)
    for h in hs:
        h.close()


@pytest.mark.parametrize("name", ["zipf64", "greedy1024"])
def test_graph_capture_replays(name):
    # a step is only kernel launches on the caller's stream, so it can be
    # captured in a HIP graph; every replay, with eager work and
    # synchronisations between replays, must give the eager outputs
    D = _D()
    prob = synth.make_problem(synth.WORKLOADS[name].with_(B=32, seed=73))
    print(f"[case] graph capture {name}", flush=True)
    dp = D.from_problem(prob)
    sv = D.handle_for(dp)
    sv.run(dp.args())
    ref = dp.fetch()
    dp.alloc_outputs(True, "cuda:0")
    args = dp.args()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sv.run(args)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.run(args)
    for rep in range(4):
        for t in (dp.accepted_len, dp.out_tokens, dp.verify_len_out):
            t.fill_(-9)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dp.fetch()
        assert not PU.same_outputs(ref, got), rep
    del g
    sv.close()


@pytest.mark.parametrize("name", ["zipf64", "peaked512"])
def test_batch_invariance(name):
    D = _D()
    w = synth.WORKLOADS[name].with_(B=48, V=40000)
    prob = synth.make_problem(w)
    print(f"[case] batch invariance {name}", flush=True)
    full = D.run_once(D.from_problem(prob))
    sel = np.array([47, 3, 3, 20, 0, 11, 29], np.int64)
    sub = synth.Problem(w.with_(B=len(sel)), np.ascontiguousarray(prob.target[sel]),
                        np.ascontiguousarray(prob.draft[sel]), np.ascontiguousarray(prob.tokens[sel]),
                        np.ascontiguousarray(prob.uniforms[sel]), None,
                        None if prob.tau is None else np.ascontiguousarray(prob.tau[sel]))
    part = D.run_once(D.from_problem(sub))
    part.pop("device_status")
    assert not PU.same_outputs(part, full, sel)


def _shared_rows(seed, K, V, T):
    rng = np.random.default_rng(seed)
    t = (1.0 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + 0.7 * rng.standard_normal((K, V))).astype(np.float32)
    q = special.softmax(d.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    p = special.softmax(t.astype(np.float64) / np.float64(np.float32(T)), axis=1)
    return t, d, p, q


@pytest.mark.parametrize("mode", ["fixed", "tau"])
def test_chi_square_shared_rows(mode):
    # 2e5 sequences verify the same rows (batch stride 0) with fresh draft samples
    # and uniforms: the emitted token at each position follows p_j, and every
    # sequence matches the oracle exactly outside the margin.
    D = _D()
    K, V, N, T = 4, 8, 200000, 0.9
    t, d, p, q = _shared_rows(50, K, V, T)
    toks = np.stack([synth.uniforms(600 + j, N) for j in range(K)], axis=1)
    for j in range(K):
        c = np.cumsum(q[j]); c[-1] = 1.0
        toks[:, j] = np.searchsorted(c, toks[:, j], side="right")
    toks = toks.astype(np.int32)
    u = synth.uniforms(700, N * (K + 1)).reshape(N, K + 1)
    if mode == "tau":
        S = np.cumprod(q.max(axis=1))
        tau = np.full(N, np.float32(S[2] * 0.999), np.float32)
        L = 3
        dp = D.DeviceProblem.upload(t, d, toks, u, T, D.F32, length_mode=1, tau=tau)
    else:
        tau, L = None, K
        dp = D.DeviceProblem.upload(t, d, toks, u, T, D.F32)
    print(f"[case] chi-square {mode} N={N}", flush=True)
    res = D.run_once(dp)
    orc = O.verify(t, d, toks, u, T, dtype=O.F32, length_mode=1 if tau is not None else 0, tau=tau)
    rep = PU.compare(f"chi2 {mode}", res, orc, dtype=O.F32, derived=tau is not None, tau=tau)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    for j in range(L + 1):
        sel = res["accepted_len"] >= j
        counts = np.bincount(res["out_tokens"][sel, j], minlength=V)
        pv = stats.chisquare(counts, p[j] * sel.sum()).pvalue
        assert pv > 1e-4, (j, pv)


def test_one_handle_across_call_kinds():
    """A handle's step state (control words, counters, stream marks) is zero
    between steps: calls of every kind and shape in a row on one handle give
    the outputs of the same calls on fresh handles, bit for bit (stream counts
    within their bounds)."""
    D = _D()
    from draft_verification_amd import binding as B
    V, Bmax, Kmax = 20000, 24, 8
    peaked = synth.WORKLOADS["peaked512"].with_(B=Bmax, K=Kmax, V=V, dtype=synth.BF16, seed=301)
    cases = []
    # fixed lengths, counted
    p0 = synth.make_problem(synth.WORKLOADS["zipf64"].with_(B=Bmax, K=Kmax, V=V, seed=302))
    cases.append(("fixed counted", lambda: D.from_problem(p0), True))
    # open length walks (derived confidences), not counted
    p1 = synth.make_problem(peaked.with_(tau_choices=(0.05, 0.3, 0.6)))
    cases.append(("open walks", lambda: D.from_problem(p1), False))
    # given confidences, a smaller batch and block
    p2 = synth.make_problem(peaked.with_(B=9, K=5, length_mode=synth.LEN_TAU, tau_choices=(0.0, 0.3, 0.7)))
    p2.confidence = (np.random.default_rng(303).random((9, 5)) ** 0.3).astype(np.float32)
    cases.append(("given confidences", lambda: D.from_problem(p2), True))
    # greedy
    p3 = synth.make_problem(synth.WORKLOADS["greedy1024"].with_(B=Bmax, K=Kmax, V=V, seed=304))
    cases.append(("greedy", lambda: D.from_problem(p3), True))
    # packed rows with bad counts and a length bound
    p4 = synth.make_problem(synth.WORKLOADS["zipf64"].with_(B=12, K=Kmax, V=V, seed=305))
    L4 = np.array([0, 3, 9, 2, 1, -1, 4, 4, 2, 0, 6, 3], np.int64)

    def packed():
        dp = D.packed_from_problem(p4, L4)
        dp.max_verify_len = 5
        return dp
    cases.append(("packed, bad counts", packed, True))
    # bad lengths in the dense layout, then the first call again
    p5 = synth.make_problem(synth.WORKLOADS["zipf64"].with_(B=Bmax, K=Kmax, V=V, seed=306))
    p5.verify_len = np.array([8, -2, 3, 9, 0] + [5] * (Bmax - 5), np.int32)
    cases.append(("bad lengths", lambda: D.from_problem(p5), True))
    cases.append(("fixed counted again", lambda: D.from_problem(p0), True))

    sv = B.SpecVerify(Bmax, Kmax, V, synth.BF16, 0)
    for name, make, counts in cases:
        print(f"[case] one handle: {name}", flush=True)
        dp = make()
        sv.run(dp.args(counts=counts))
        got = dp.fetch()
        ref = D.run_once(make())
        assert not PU.same_outputs(got, ref), name
        np.testing.assert_array_equal(got["device_status"], ref["device_status"])
        if counts:
            assert not PU.check_streamed(got, dp.K, V, 2, two_rows=name != "greedy"), name
            for b in np.flatnonzero(got["out_tokens"][:, 0] < 0):  # marked bad: no row read
                assert got["rows_read"][b] == 0, (name, b)
    sv.close()
