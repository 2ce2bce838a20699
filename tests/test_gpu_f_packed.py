"""Packed ("pruned, not padded") logits: sequence b brings its first L_b + 1
target rows and L_b draft rows, stacked, with row offsets (zhichai.net article,
"Under the hood", on SGLang's variable-length verification).  The outputs must
equal the dense layout's bit for bit (diagnostics included) and the oracle's on
the same logical rows."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Workload("packed", B=40, K=6, V=5000, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                      sigma_first=0.3, sigma_last=0.9, temperature=1.0, seed=81)


def _D():
    from draft_verification_amd import device as D
    return D


def _lengths(seed, Bn, K):
    L = np.random.default_rng(seed).integers(0, K + 1, size=Bn).astype(np.int32)
    L[:3] = [0, K, 1]
    return L


def _case(name, w, L, greedy=False):
    D = _D()
    print(f"[case] {name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} T={w.temperature}", flush=True)
    prob = synth.make_problem(w)
    prob.verify_len = L
    dense = D.run_once(D.from_problem(prob))
    packed = D.run_once(D.packed_from_problem(prob, L))
    assert not PU.same_outputs(packed, dense)
    two = not greedy and w.draft_mode == 0
    es = 2 if w.dtype == synth.BF16 else 4
    for res in (packed, dense):
        assert not PU.check_streamed(res, w.K, w.V, es, two_rows=two)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(name, packed, orc, dtype=w.dtype, greedy=greedy, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    return packed, orc


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_packed_equals_dense_and_oracle(dtype, T):
    w = BASE.with_(dtype=dtype, temperature=T, seed=82 + dtype)
    _case(f"packed dt={dtype} T={T}", w, _lengths(82, w.B, w.K))


@pytest.mark.parametrize("V", [1, 257, 16385])
def test_packed_vocab_edges(V):
    w = BASE.with_(V=V, B=9, K=3, seed=90 + V)
    _case(f"packed V={V}", w, _lengths(90 + V, w.B, w.K))


def test_packed_greedy():
    w = synth.WORKLOADS["greedy1024"].with_(B=50, K=5, V=20000, seed=83)
    _case("packed greedy", w, _lengths(83, w.B, w.K), greedy=True)


def test_packed_one_hot():
    w = BASE.with_(draft_mode=1, token_mode=2, seed=84)
    _case("packed one-hot", w, _lengths(84, w.B, w.K))


def test_packed_full_size():
    w = synth.WORKLOADS["sched256"].with_(length_mode=synth.LEN_FIXED, tau_choices=())
    _case("packed sched256", w, _lengths(85, w.B, w.K))


def test_bad_row_counts():
    """A sequence whose target row count is outside [1, K+1], or whose draft
    row count is not its target count minus 1, is marked bad (a = 0, no token,
    status bit); the others are unaffected."""
    D = _D()
    w = BASE.with_(B=8, K=4, V=3000, dtype=synth.F32, seed=86)
    prob = synth.make_problem(w)
    L = np.array([2, 4, 5, 0, 3, -1, 1, 4], np.int64)   # 5 -> K+2 target rows, -1 -> none
    dp = D.packed_from_problem(prob, L)
    # one draft offset moved back a row: sequence 6 brings one draft row too few
    # and sequence 7 one too many (both bad, so neither is read); every offset
    # stays inside the packed tensor
    doff = dp.draft_row_offsets.cpu().numpy()
    doff[7] -= 1
    assert doff[7] >= doff[6]
    dp.draft_row_offsets = torch.from_numpy(doff).to(dp.target.device)
    res = D.run_once(dp)
    bad = {2, 5, 6, 7}
    assert res["device_status"][0] == 1
    for b in range(w.B):
        if b in bad:
            assert res["accepted_len"][b] == 0 and (res["out_tokens"][b] == -1).all(), b
    good = [b for b in range(w.B) if b not in bad]
    prob.verify_len = np.clip(L, 0, w.K).astype(np.int32)
    orc = O.verify_problem(prob, seqs=good, all_rows=True)
    rep = PU.compare("packed bad counts", res, orc, dtype=w.dtype, prob=prob)
    assert not rep.mismatches, rep.mismatches[:5]
