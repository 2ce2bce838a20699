"""spec_verify_run_noalloc against spec_verify_run through the C ABI.

Two no-allocation calls in a row share the library's static workspace, the
second on a smaller batch, block and vocabulary than the first, so it starts
from the first call's leftovers.  Each call's outputs must equal, bit for bit,
those of spec_verify_run on a handle of its own for the same inputs (the
stream counts depend on timing and are bounded instead).  A warm call must not
change the device's free memory.
"""
import numpy as np
import pytest

from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# an open confidence walk over a ragged vocabulary of 5 splits, then a fixed
# verify length over 2 splits: different kernels variants, B, K and V
LARGE = synth.Workload("noalloc-large", B=24, K=12, V=70001, dtype=synth.BF16, target_kind=0, target_scale=2.0,
                       sigma_first=0.3, sigma_last=1.2, temperature=1.0, length_mode=synth.LEN_TAU,
                       tau_choices=(0.0, 0.2, 0.5, 2.0), seed=4101)
SMALL = synth.Workload("noalloc-small", B=5, K=3, V=20000, dtype=synth.F32, target_kind=0, target_scale=2.0,
                       sigma_first=0.02, sigma_last=0.6, temperature=0.8, seed=4102)


def _handle_result(prob):
    from draft_verification_amd import device as D
    dp = D.from_problem(prob)
    return D.run_once(dp)


def _noalloc_result(prob, *, check_memory):
    from draft_verification_amd import binding as B
    from draft_verification_amd import device as D
    w = prob.w
    dp = D.from_problem(prob)
    cfg = B.Config(w.B, w.K, w.V, w.dtype, 0)
    args = dp.args()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(0)[0] if check_memory else None
    B.run_noalloc(cfg, args)
    res = dp.fetch()
    if check_memory:
        assert torch.cuda.mem_get_info(0)[0] == free0
    return res


def _check(name, res_ref, res, prob):
    w = prob.w
    print(f"[noalloc] {name} B={w.B} K={w.K} V={w.V}", flush=True)
    assert int(res["device_status"][0]) == 0
    diff = PU.same_outputs(res_ref, res)
    assert not diff, f"{name}: outputs differ from spec_verify_run: {diff}"
    # a derived-confidence walk with 0 < tau <= 1 stays open until the device closes it
    open_walk = None
    if w.length_mode == synth.LEN_TAU and prob.confidence is None:
        open_walk = (prob.tau > 0) & (prob.tau <= 1)
    bad = PU.check_streamed(res, w.K, w.V, 2 if w.dtype == synth.BF16 else 4, two_rows=True, open_walk=open_walk)
    assert not bad, bad[:5]


def test_two_calls_in_a_row_match_the_handle_path():
    big, small = synth.make_problem(LARGE), synth.make_problem(SMALL)
    ref_big, ref_small = _handle_result(big), _handle_result(small)
    res_big = _noalloc_result(big, check_memory=False)
    _check("first call", ref_big, res_big, big)
    res_small = _noalloc_result(small, check_memory=True)
    _check("second call, smaller", ref_small, res_small, small)
    # the tested positions differ in kind between the calls: rejections and
    # bonus draws both occur
    assert (ref_big["accepted_len"] < ref_big["verify_len_out"]).any()
    assert (ref_big["accepted_len"] == ref_big["verify_len_out"]).any()


def test_oversized_call_is_rejected_before_device_work():
    from draft_verification_amd import binding as B
    # 2048 sequences of 16 positions over 129280 tokens need about 30 MB
    cfg = B.Config(2048, 16, 129280, B.SV_BF16, 0)
    fake = 1 << 40
    a = B.make_args(2048, 16, target=fake, draft=fake, tokens=fake, uniforms=fake, temperature=1.0,
                    target_strides=(17 * 129280, 129280), draft_strides=(16 * 129280, 129280),
                    accepted_len=fake, out_tokens=fake, verify_len_out=fake)
    with pytest.raises(B.SpecVerifyError) as e:
        B.run_noalloc(cfg, a)
    assert e.value.status == B.SV_EUNSUPPORTED
