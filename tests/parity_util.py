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
    The residual mass Z and the drawn token's probability r_y / Z are held to
    the stated bar relative to their own values at every Z (the library forms
    each token's residual from the exact logit difference, so it keeps its
    relative accuracy as p and q approach each other).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import oracle as O

TIGHT_RTOL = 2e-6


# Outputs that count what the step streamed: rows of positions dispatched
# before an earlier rejection was known are read or not depending on timing, so
# these vary from run to run (within the bounds check_streamed tests).
STREAM_COUNTS = ("rows_read", "bytes_read")


def same_outputs(a: dict, b: dict, sel=None):
    """Names of the outputs (other than the stream counts) that differ bitwise
    between two fetched results (``sel``: batch rows of ``b`` to compare)."""
    bad = []
    for k, v in a.items():
        if v is None or k in STREAM_COUNTS or b.get(k) is None:
            continue
        w = b[k] if sel is None else b[k][sel]
        if not np.array_equal(np.asarray(v).view(np.uint8), np.asarray(w).view(np.uint8)):
            bad.append(k)
    return bad


def check_streamed(res: dict, K: int, V: int, elem_bytes: int, *, two_rows: bool, open_walk=None):
    """The stream counts lie between the rows the outputs depend on (target
    rows 1..a+1 and the tested draft rows) and the verify window (every row up
    to L + 1; with an open length walk every draft row); bytes lie between the
    needed rows and the rows touched.  Returns a list of violations."""
    out = []
    if res.get("rows_read") is None:
        return out
    a = res["accepted_len"].astype(np.int64)
    L = res["verify_len_out"].astype(np.int64)
    rows = res["rows_read"].astype(np.int64)
    byt = res["bytes_read"].astype(np.int64) if res.get("bytes_read") is not None else None
    for b in range(len(a)):
        if res["out_tokens"][b][min(int(a[b]), K)] < 0:
            continue  # a sequence marked bad
        ob = bool(open_walk[b]) if open_walk is not None else False
        lo = (a[b] + 1) + (min(a[b] + 1, L[b]) if two_rows else 0)
        hi = ((K + 1) if ob else (L[b] + 1)) + ((K if ob else L[b]) if two_rows else 0)
        if not (lo <= rows[b] <= hi):
            out.append((b, "rows", int(rows[b]), int(lo), int(hi)))
        if byt is not None and not (lo * V * elem_bytes <= byt[b] <= rows[b] * V * elem_bytes):
            out.append((b, "bytes", int(byt[b]), int(lo * V * elem_bytes), int(rows[b] * V * elem_bytes)))
    return out


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


def _walk_draft_rows(a, L, K, *, derived, tau_b, onehot):
    """Draft rows (1-based, as a boolean mask over 1..K) whose statistics the
    step's walk evaluates: the tested positions 1..min(a+1, L), and with a
    derived confidence while the verify-length walk is open (0 < tau <= 1)
    every position up to min(L+1, K)."""
    need = np.zeros(K, bool)
    if onehot:
        return need
    need[:min(a + 1, L)] = True
    if derived and tau_b is not None and 0.0 < tau_b <= 1.0:
        need[:min(L + 1, K)] = True
    return need


def _survival_rows(a, L, K, *, derived, conf_given, tau_b, onehot):
    """Positions whose survival S_j the step reports: every position with a
    given confidence (or a one-hot draft, c = 1), else with a derived
    confidence the positions whose draft row the walk evaluates."""
    if conf_given or (derived and onehot):
        return np.ones(K, bool)
    if derived:
        return _walk_draft_rows(a, L, K, derived=True, tau_b=tau_b, onehot=False)
    return np.zeros(K, bool)


def _track(cur, value):
    """Running maximum for the report that keeps a NaN visible."""
    value = float(value)
    if cur != cur or value != value:
        return float("nan")
    return max(cur, value)


def _bad(r, tol):
    """A relative error fails unless it is a number within tol (NaN fails)."""
    return not (r <= tol)


def compare(name, gpu: dict, orc: O.OracleResult, *, dtype, greedy=False, derived=False, tau=None,
            conf_given=False, onehot=False, prob=None) -> Report:
    """``derived``: tau mode with c = max draft probability (then ``tau``, the
    per-sequence thresholds, says where the verify-length walk was open);
    ``conf_given``: tau mode with given confidences; ``onehot``: one-hot
    drafts.  ``prob`` (a generator problem) sets all four from its inputs.
    Diagnostics the step must report (lse of the rows it evaluates,
    survivals) are required, not only compared where present."""
    if prob is not None:
        tau_mode = prob.w.length_mode == O.LEN_TAU
        derived = tau_mode and prob.confidence is None
        conf_given = tau_mode and prob.confidence is not None
        tau = prob.tau if tau_mode else None
        onehot = getattr(prob.w, "draft_mode", O.DRAFT_PROBS) == O.DRAFT_ONEHOT
    rep = Report(name)
    K1 = gpu["out_tokens"].shape[1]
    K = K1 - 1
    tol = stated_rtol(dtype)
    if derived and tau is None and not onehot:
        raise ValueError("compare: a derived confidence needs the thresholds to know the walk")
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
        tau_b = None if tau is None else float(np.asarray(tau).reshape(-1)[b])
        # diagnostics: rows the step evaluates must be present; every value
        # present is compared with the oracle's (NaN = not written)
        lt = gpu["lse_target"][b] if gpu.get("lse_target") is not None else None
        if lt is not None:
            need = np.arange(o_a + 1)
            if np.any(np.isnan(lt[need])):
                rep.mismatches.append((int(b), dict(kind="lse_target missing", rows=need.tolist())))
            wrote = ~np.isnan(lt)
            r = _rel(lt[wrote], orc.lse_target[i][wrote], 1.0)
            if r.size:
                rep.max_rel_lse = _track(rep.max_rel_lse, r.max())
                if _bad(r.max(), min(tol, TIGHT_RTOL)):
                    rep.mismatches.append((int(b), dict(kind="lse_target", rel=float(r.max()))))
        ld = gpu["lse_draft"][b] if gpu.get("lse_draft") is not None else None
        if ld is not None:
            need = _walk_draft_rows(o_a, o_L, K, derived=derived, tau_b=tau_b, onehot=onehot)
            if np.any(np.isnan(ld[need])):
                rep.mismatches.append((int(b), dict(kind="lse_draft missing", rows=np.nonzero(need)[0].tolist())))
            if onehot and not np.all(np.isnan(ld)):
                rep.mismatches.append((int(b), dict(kind="lse_draft written for one-hot drafts")))
            wrote = ~np.isnan(ld)
            r = _rel(ld[wrote], orc.lse_draft[i][wrote], 1.0)
            if r.size:
                rep.max_rel_lse = _track(rep.max_rel_lse, r.max())
                if _bad(r.max(), min(tol, TIGHT_RTOL)):
                    rep.mismatches.append((int(b), dict(kind="lse_draft", rel=float(r.max()))))
        sv = gpu["survival"][b] if gpu.get("survival") is not None else None
        if sv is not None:
            need = _survival_rows(o_a, o_L, K, derived=derived, conf_given=conf_given, tau_b=tau_b, onehot=onehot)
            if np.any(np.isnan(sv[need])):
                rep.mismatches.append((int(b), dict(kind="survival missing", rows=np.nonzero(need)[0].tolist())))
            if not (derived or conf_given) and not np.all(np.isnan(sv)):
                rep.mismatches.append((int(b), dict(kind="survival written in fixed-length mode")))
            wrote = ~np.isnan(sv)
            r = _rel(sv[wrote], orc.survival[i][wrote])
            if r.size and _bad(r.max(), TIGHT_RTOL):
                rep.mismatches.append((int(b), dict(kind="survival", rel=float(r.max()))))
        if gpu.get("residual_mass") is not None:
            z, pz = float(gpu["residual_mass"][b]), float(gpu["sampled_prob"][b])
            for what, got, want in (("residual mass", z, orc.residual_mass[i]), ("sampled prob", pz, orc.sampled_prob[i])):
                r = float(_rel(got, want))
                rep.max_rel_prob = _track(rep.max_rel_prob, r)
                if _bad(r, tol):
                    rep.mismatches.append((int(b), dict(kind=what, got=got, want=float(want), rel=r)))
    return rep
