"""CPU oracle for batched draft verification -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path never does.

Thin ctypes wrapper around ``sv_oracle.c`` (plain fp64 C, one sequence at a
time).  Every function there cites the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "libsv_oracle.so")

F32, BF16 = 0, 1
LEN_FIXED, LEN_TAU = 0, 1
FINAL_RESIDUAL, FINAL_BONUS, FINAL_GREEDY, FINAL_BAD_INPUT = 0, 1, 2, 3
MARGIN_ACCEPT, MARGIN_CDF, MARGIN_SURVIVAL = 1, 2, 4
DRAFT_PROBS, DRAFT_ONEHOT = 0, 1
MARGIN = 1e-6


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP over sequences)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("target", ctypes.c_void_p), ("target_batch_stride", ctypes.c_int64), ("target_row_stride", ctypes.c_int64),
        ("draft", ctypes.c_void_p), ("draft_batch_stride", ctypes.c_int64), ("draft_row_stride", ctypes.c_int64),
        ("tokens", ctypes.c_void_p), ("uniforms", ctypes.c_void_p), ("temperature", ctypes.c_float),
        ("length_mode", ctypes.c_int32), ("verify_len_in", ctypes.c_void_p), ("confidence", ctypes.c_void_p),
        ("tau", ctypes.c_void_p), ("seq_index", ctypes.c_void_p), ("n_seq", ctypes.c_int32),
        ("all_rows", ctypes.c_int32), ("n_threads", ctypes.c_int32), ("draft_mode", ctypes.c_int32),
    ]


class _Result(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "accepted_len", "out_tokens", "verify_len", "lse_target", "lse_draft", "survival",
        "residual_mass", "sampled_prob", "final_kind", "margin", "accept_gap", "cdf_gap", "alt_token")]


class _SchedProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("confidence", ctypes.c_void_p),
                ("speed", ctypes.c_void_p), ("n_speed", ctypes.c_int32)]


class _SchedResult(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "verify_len", "survival", "admitted", "tau", "expected", "margin", "bad")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.svo_verify.restype = ctypes.c_int
        L.svo_verify.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Result)]
        L.svo_max_threads.restype = ctypes.c_int
        L.svo_max_threads.argtypes = []
        L.svo_schedule.restype = ctypes.c_int
        L.svo_schedule.argtypes = [ctypes.POINTER(_SchedProblem), ctypes.POINTER(_SchedResult)]
        _lib = L
    return _lib


@dataclass
class OracleResult:
    seq: np.ndarray            # which sequences (batch indices) these rows describe
    accepted_len: np.ndarray
    out_tokens: np.ndarray
    verify_len: np.ndarray
    lse_target: np.ndarray
    lse_draft: np.ndarray
    survival: np.ndarray
    residual_mass: np.ndarray
    sampled_prob: np.ndarray
    final_kind: np.ndarray
    margin: np.ndarray
    accept_gap: np.ndarray
    cdf_gap: np.ndarray
    alt_token: np.ndarray


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def verify(target: np.ndarray, draft: Optional[np.ndarray], tokens: np.ndarray, uniforms: Optional[np.ndarray],
           temperature: float, *, dtype: int, length_mode: int = LEN_FIXED,
           verify_len: Optional[np.ndarray] = None, confidence: Optional[np.ndarray] = None,
           tau: Optional[np.ndarray] = None, seqs: Optional[Sequence[int]] = None,
           all_rows: bool = False, threads: int = 0, V: Optional[int] = None,
           draft_mode: int = DRAFT_PROBS) -> OracleResult:
    """Run the fp64 definition on host arrays.

    ``target`` is [B][K+1][V] (float32, or uint16 bf16 bits when dtype == BF16),
    or [K+1][V] to share one set of rows across all B sequences (B is then taken
    from ``tokens``).  ``draft`` likewise [B][K][V] or [K][V].  With
    ``draft_mode == DRAFT_ONEHOT`` the draft distribution is the point mass at
    each drafted token and ``draft`` is not read (may be None).
    """
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, K = tokens.shape
    want = np.float32 if dtype == F32 else np.uint16
    target = np.ascontiguousarray(target, dtype=want)
    if target.ndim == 2:
        t_bs = 0
        Vv = target.shape[1]
        assert target.shape[0] == K + 1
    else:
        assert target.shape[:2] == (B, K + 1)
        Vv = target.shape[2]
        t_bs = (K + 1) * Vv
    if draft is not None:
        draft = np.ascontiguousarray(draft, dtype=want)
        d_bs = 0 if draft.ndim == 2 else K * Vv
        assert draft.shape[-1] == Vv
    else:
        d_bs = 0
    if uniforms is not None:
        uniforms = np.ascontiguousarray(uniforms, dtype=np.float32)
        assert uniforms.shape == (B, K + 1)
    vl = None if verify_len is None else np.ascontiguousarray(verify_len, dtype=np.int32)
    cf = None if confidence is None else np.ascontiguousarray(confidence, dtype=np.float32)
    ta = None if tau is None else np.ascontiguousarray(tau, dtype=np.float32)
    if seqs is None:
        sidx = np.arange(B, dtype=np.int32)
    else:
        sidx = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
    n = len(sidx)
    P = _Problem(B, K, Vv, dtype, _ptr(target), t_bs, Vv, _ptr(draft), d_bs, Vv, _ptr(tokens), _ptr(uniforms),
                 float(temperature), length_mode, _ptr(vl), _ptr(cf), _ptr(ta), _ptr(sidx), n,
                 int(all_rows), int(threads), int(draft_mode))
    out = OracleResult(
        seq=sidx,
        accepted_len=np.empty(n, np.int32), out_tokens=np.empty((n, K + 1), np.int32),
        verify_len=np.empty(n, np.int32), lse_target=np.empty((n, K + 1), np.float64),
        lse_draft=np.empty((n, K), np.float64), survival=np.empty((n, K), np.float64),
        residual_mass=np.empty(n, np.float64), sampled_prob=np.empty(n, np.float64),
        final_kind=np.empty(n, np.int32), margin=np.empty(n, np.int32),
        accept_gap=np.empty(n, np.float64), cdf_gap=np.empty(n, np.float64), alt_token=np.empty(n, np.int32))
    R = _Result(*[_ptr(getattr(out, f)) for f in (
        "accepted_len", "out_tokens", "verify_len", "lse_target", "lse_draft", "survival",
        "residual_mass", "sampled_prob", "final_kind", "margin", "accept_gap", "cdf_gap", "alt_token")])
    rc = lib().svo_verify(ctypes.byref(P), ctypes.byref(R))
    if rc != 0:
        raise ValueError("oracle: arguments outside the definition")
    return out


def verify_problem(prob, seqs=None, all_rows=False, threads=0) -> OracleResult:
    """Run the oracle on a ``synth.Problem``."""
    w = prob.w
    return verify(prob.target, prob.draft, prob.tokens, prob.uniforms if w.temperature > 0 else prob.uniforms,
                  w.temperature, dtype=w.dtype, length_mode=w.length_mode, verify_len=prob.verify_len,
                  confidence=prob.confidence, tau=prob.tau, seqs=seqs, all_rows=all_rows, threads=threads,
                  draft_mode=getattr(w, "draft_mode", DRAFT_PROBS))


def max_threads() -> int:
    return int(lib().svo_max_threads())


@dataclass
class ScheduleResult:
    verify_len: np.ndarray   # [B] int32
    survival: np.ndarray     # [B][K] float64
    admitted: int            # m
    tau: float               # smallest admitted survival (NaN if none)
    expected: float          # T(m) = (B + sum of admitted survivals) * speed[B + m]
    margin: bool             # a stop decision at or before m was a near tie
    bad: bool                # a confidence was outside [0, 1]


def schedule(confidence: np.ndarray, speed: np.ndarray) -> ScheduleResult:
    """Load-aware admission (sv_oracle.c ``svo_schedule``): rank every drafted
    position by survival and admit while expected tokens x step rate rises.

    confidence: [B][K] float32; speed: steps per second at a batch of n tokens,
    n = 0 .. B (K + 1) at least."""
    c = np.ascontiguousarray(confidence, dtype=np.float32)
    B, K = c.shape
    sp = np.ascontiguousarray(speed, dtype=np.float64)
    vl = np.zeros(B, np.int32)
    surv = np.zeros((B, K), np.float64)
    adm = np.zeros(1, np.int32)
    tau = np.zeros(1, np.float64)
    exp_ = np.zeros(1, np.float64)
    mar = np.zeros(1, np.int32)
    bad = np.zeros(1, np.int32)
    prob = _SchedProblem(B, K, c.ctypes.data, sp.ctypes.data, sp.size)
    res = _SchedResult(vl.ctypes.data, surv.ctypes.data, adm.ctypes.data, tau.ctypes.data, exp_.ctypes.data,
                       mar.ctypes.data, bad.ctypes.data)
    rc = lib().svo_schedule(ctypes.byref(prob), ctypes.byref(res))
    if rc != 0:
        raise ValueError(f"svo_schedule failed ({rc})")
    return ScheduleResult(vl, surv, int(adm[0]), float(tau[0]), float(exp_[0]), bool(mar[0]), bool(bad[0]))


def calibrated_confidence_steps(logits_steps, temperature, delay: int, c_default: float, resets=None):
    """Calibrated, causally delayed confidences over a sequence of steps.

    umans.ai blog, section "2. Verify smarter": raw confidence gets a
    per-position temperature fitted on held-out data, and the production
    version sizes the truncation from confidence measured two steps earlier (a
    causal barrier between the decision and the tokens); zhichai.net article,
    section "Under the hood": Sequential Temperature Scaling.

    Reading where the pages leave it open: at each step the calibrated
    confidence of position j is sigmoid(z_j / T_j), in fp64, rounded to fp32
    (a temperature that is not finite and positive gives 0 and flags bad
    input); the value handed to the length decision is the calibrated value
    of the same slot and position from ``delay`` steps earlier, or
    ``c_default`` while the slot has fewer than ``delay`` earlier steps since
    its last reset (a new sequence in the slot); delay 0 hands over the
    current value.

    logits_steps: list of [B][K] arrays (one per step, in order);
    temperature: [K]; resets: list of [B] bool arrays (or None).
    Returns (now, out, bad): lists of [B][K] float32 arrays and of bools."""
    T = np.asarray(temperature, dtype=np.float64)
    Bn, K = np.asarray(logits_steps[0]).shape
    history = [[] for _ in range(Bn)]          # calibrated rows of each slot since its reset
    nows, outs, bads = [], [], []
    for t, z in enumerate(logits_steps):
        z = np.asarray(z, dtype=np.float32).astype(np.float64)
        now = np.empty((Bn, K), np.float32)
        bad = False
        for b in range(Bn):
            for j in range(K):
                if not (np.isfinite(T[j]) and T[j] > 0.0):
                    bad = True
                    now[b, j] = 0.0
                else:
                    with np.errstate(over="ignore"):  # exp(+large) = inf gives 0 exactly
                        now[b, j] = np.float32(1.0 / (1.0 + np.exp(-z[b, j] / T[j])))
        out = np.empty((Bn, K), np.float32)
        for b in range(Bn):
            if resets is not None and resets[t] is not None and resets[t][b]:
                history[b] = []
            if delay == 0:
                out[b] = now[b]
            elif len(history[b]) >= delay:
                out[b] = history[b][-delay]
            else:
                out[b] = np.float32(c_default)
            history[b].append(now[b].copy())
        nows.append(now)
        outs.append(out)
        bads.append(bad)
    return nows, outs, bads
