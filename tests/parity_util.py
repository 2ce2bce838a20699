"""Element-by-element comparison of the HIP path with the CPU oracle.

The bar:
  * verify lengths, accepted lengths and emitted tokens are bit-exact, except
    for sequences the oracle flags as margin cases (|u - p/q| < 1e-6 at a tested
    position, a normalised CDF gap < 1e-6 at the final draw, or a survival within
    1e-6 (relative) of tau); those are counted and reported.  For a CDF-only
    margin the emitted prefix must still match and the final token must be one
    of the two tokens on either side of the nearest CDF step.
  * log-sum-exp values and the residual mass / drawn-token probability agree to
    1e-5 relative for fp32 inputs and 2e-3 for bf16 inputs (the stated bar), and
    also to TIGHT_RTOL, the bound the arithmetic gives (row sums carry ~1e-8
    relative error, outputs are rounded once to fp32).  An lse error d scales
    every probability of the row by e^d, so for lse the error is measured
    relative to max(|lse|, 1): plain relative error is ill-conditioned near 0.
    The drawn-token probability max(0, p - q)/Z suffers cancellation when
    p ~ q (the row-sum error is amplified by p/(p - q)), so it is held to the
    stated bar only.  The residual mass Z = sum max(0, p - q) is a difference of
    two unit masses whose error the fp32 token masses bound in absolute terms
    (~1e-8): for a replacement draw, Z's and r_y / Z's errors are measured
    relative to max(Z, Z_FLOOR), as the oracle measures its CDF-gap margin.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import oracle as O

TIGHT_RTOL = 2e-6
Z_FLOOR = 0.1  # the oracle's SVO_Z_FLOOR


def stated_rtol(dtype):
    return 1e-5 if dtype == O.F32 else 2e-3


@dataclass
class Report:
    name: str
    n: int = 0
    exact: int = 0
    margin: int = 0
    margin_disagree: int = 0
    mismatches: list = field(default_factory=list)
    max_rel_lse: float = 0.0
    max_rel_prob: float = 0.0

    def line(self):
        return (f"[parity] {self.name}: sequences={self.n} exact={self.exact} margin={self.margin} "
                f"(gpu differs inside margin: {self.margin_disagree}) mismatches={len(self.mismatches)} "
                f"max_rel_lse={self.max_rel_lse:.2e} max_rel_prob={self.max_rel_prob:.2e}")


def _rel(got, want, floor=1e-300):
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    return np.abs(got - want) / np.maximum(np.abs(want), floor)


def compare(name, gpu: dict, orc: O.OracleResult, *, dtype, greedy=False, derived=False) -> Report:
    rep = Report(name)
    K1 = gpu["out_tokens"].shape[1]
    K = K1 - 1
    tol = stated_rtol(dtype)
    for i, b in enumerate(orc.seq):
        rep.n += 1
        m = int(orc.margin[i])
        g_a, o_a = int(gpu["accepted_len"][b]), int(orc.accepted_len[i])
        g_L, o_L = int(gpu["verify_len_out"][b]), int(orc.verify_len[i])
        g_tok, o_tok = gpu["out_tokens"][b], orc.out_tokens[i]
        same = g_a == o_a and g_L == o_L and np.array_equal(g_tok, o_tok)
        if m == 0:
            if same:
                rep.exact += 1
            else:
                rep.mismatches.append((int(b), dict(gpu_a=g_a, ora_a=o_a, gpu_L=g_L, ora_L=o_L,
                                                    gpu_tok=g_tok.tolist(), ora_tok=o_tok.tolist())))
                continue
        else:
            rep.margin += 1
            if not same:
                rep.margin_disagree += 1
            if m == O.MARGIN_CDF:
                ok = (g_a == o_a and g_L == o_L and np.array_equal(g_tok[:o_a], o_tok[:o_a])
                      and int(g_tok[o_a]) in (int(o_tok[o_a]), int(orc.alt_token[i]))
                      and np.all(g_tok[o_a + 1:] == -1))
                if not ok:
                    rep.mismatches.append((int(b), dict(kind="cdf-margin", gpu_tok=g_tok.tolist(),
                                                        ora_tok=o_tok.tolist(), alt=int(orc.alt_token[i]))))
                continue
            if not same:
                continue
        if greedy or orc.final_kind[i] == O.FINAL_BAD_INPUT:
            continue
        # diagnostics, where the GPU wrote them (NaN = untouched)
        lt = gpu["lse_target"][b] if gpu.get("lse_target") is not None else None
        if lt is not None:
            # rows 1..a+1 must be present
            need = np.arange(o_a + 1)
            if np.any(np.isnan(lt[need])):
                rep.mismatches.append((int(b), dict(kind="lse_target missing", rows=need.tolist())))
            wrote = ~np.isnan(lt)
            r = _rel(lt[wrote], orc.lse_target[i][wrote], 1.0)
            if r.size:
                rep.max_rel_lse = max(rep.max_rel_lse, float(r.max()))
                if r.max() > min(tol, TIGHT_RTOL):
                    rep.mismatches.append((int(b), dict(kind="lse_target", rel=float(r.max()))))
        ld = gpu["lse_draft"][b] if gpu.get("lse_draft") is not None else None
        if ld is not None:
            wrote = ~np.isnan(ld)
            r = _rel(ld[wrote], orc.lse_draft[i][wrote], 1.0)
            if r.size:
                rep.max_rel_lse = max(rep.max_rel_lse, float(r.max()))
                if r.max() > min(tol, TIGHT_RTOL):
                    rep.mismatches.append((int(b), dict(kind="lse_draft", rel=float(r.max()))))
        sv = gpu["survival"][b] if gpu.get("survival") is not None else None
        if sv is not None and (derived or not np.all(np.isnan(sv))):
            wrote = ~np.isnan(sv)
            r = _rel(sv[wrote], orc.survival[i][wrote])
            if r.size and r.max() > TIGHT_RTOL:
                rep.mismatches.append((int(b), dict(kind="survival", rel=float(r.max()))))
        if gpu.get("residual_mass") is not None:
            z, pz = float(gpu["residual_mass"][b]), float(gpu["sampled_prob"][b])
            # Z and r_y / Z carry Z's error, which arithmetic on the token masses
            # bounds in absolute terms: it is measured relative to max(Z, Z_FLOOR)
            zo = float(orc.residual_mass[i])
            scale = zo / max(zo, Z_FLOOR) if orc.final_kind[i] == O.FINAL_RESIDUAL and zo > 0 else 1.0
            for got, want in ((z, orc.residual_mass[i]), (pz, orc.sampled_prob[i])):
                r = float(_rel(got, want)) * scale
                rep.max_rel_prob = max(rep.max_rel_prob, r)
                if r > tol:
                    rep.mismatches.append((int(b), dict(kind="residual prob", got=got, want=float(want), rel=r)))
    return rep
