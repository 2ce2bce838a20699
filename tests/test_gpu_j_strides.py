"""GPU parity with strided logits: rows padded in memory (row stride > V),
gaps between sequences (batch stride > rows x row stride), and a base pointer
off the 16-byte alignment.  Aligned padding keeps the 16-byte vector loads;
odd padding or an odd base takes the per-element path.  The oracle reads the
same logical rows (tests/parity_util.py states the bar)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _strided(host, rows, V, pad, gap, shift, dtype):
    """Device copy of host [B][rows][V] with row stride V + pad, batch stride
    rows (V + pad) + gap and `shift` leading elements; returns (view at the
    first logical element, batch stride, row stride)."""
    B = host.shape[0]
    rs = V + pad
    bs = rows * rs + gap
    tdt = torch.int16 if dtype == synth.BF16 else torch.float32
    flat = torch.full((shift + B * bs,), 0, dtype=tdt, device="cuda")
    src = torch.from_numpy(host.view(np.int16) if dtype == synth.BF16 else host).to("cuda")
    for b in range(B):
        blk = flat[shift + b * bs: shift + b * bs + rows * rs].view(rows, rs)
        blk[:, :V].copy_(src[b])
    return flat[shift:], bs, rs


CASES = [
    # dtype, pad, gap, shift, temperature
    (synth.BF16, 8, 0, 0, 1.0),     # aligned padding: vector path with strides
    (synth.BF16, 8, 40, 8, 0.7),    # aligned padding, sequence gaps, aligned shift
    (synth.BF16, 3, 5, 0, 1.0),     # odd padding: per-element path
    (synth.BF16, 0, 0, 1, 1.0),     # contiguous rows, base off alignment
    (synth.F32, 4, 12, 4, 1.0),     # fp32 aligned
    (synth.F32, 1, 0, 0, 0.7),      # fp32 odd padding
    (synth.BF16, 8, 16, 0, 0.0),    # greedy (target rows only)
]


@pytest.mark.parametrize("dtype,pad,gap,shift,T", CASES)
def test_strided_logits(dtype, pad, gap, shift, T):
    from draft_verification_amd import device as D
    if T == 0.0:
        w = synth.WORKLOADS["greedy1024"].with_(B=9, K=5, V=20000, dtype=dtype, seed=190 + pad)
    else:
        w = synth.Workload("strides", B=9, K=5, V=20000, dtype=dtype, target_kind=0, target_scale=2.0,
                           sigma_first=0.3, sigma_last=0.6, temperature=T, seed=190 + pad + gap)
    print(f"[case] strides dt={dtype} pad={pad} gap={gap} shift={shift} T={T}", flush=True)
    prob = synth.make_problem(w)
    dp = D.from_problem(prob)
    t, tbs, trs = _strided(prob.target, w.K + 1, w.V, pad, gap, shift, dtype)
    dp.target, dp.target_strides = t, (tbs, trs)
    if prob.draft is not None and T > 0:
        d, dbs, drs = _strided(prob.draft, w.K, w.V, pad, gap, shift, dtype)
        dp.draft, dp.draft_strides = d, (dbs, drs)
    res = D.run_once(dp)
    orc = O.verify_problem(prob, all_rows=True)
    rep = PU.compare(f"strides {dtype} {pad} {gap} {shift} {T}", res, orc, dtype=dtype, greedy=T == 0.0, prob=prob)
    print(rep.line(), flush=True)
    assert not rep.mismatches, rep.mismatches[:5]
    assert res["device_status"][0] == 0
