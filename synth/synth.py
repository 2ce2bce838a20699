"""Seeded synthetic problems for batched draft verification.

Shared by the CPU oracle tests, the GPU parity tests and the benchmark.  It
makes inputs only -- logits, drafted tokens, uniforms, thresholds -- and holds
none of the verifier's arithmetic.  The heavy lifting is in ``sv_synth.c``
(Philox4x32-10 per Salmon et al., SC'11; Box-Muller normals; Fisher-Yates rank
permutations; Gumbel-max draft tokens), built into ``libsv_synth.so``.

The five workloads follow the problem statement of the pages: a target model
verifies a block of K drafted tokens per sequence over a vocabulary of about
128K entries, with confidence-scheduled verify lengths.  Their shapes and value
distributions are listed in ``WORKLOADS``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_synth.c")
_LIB = os.path.join(_HERE, "libsv_synth.so")

F32, BF16 = 0, 1
LEN_FIXED, LEN_TAU = 0, 1


def build(force: bool = True) -> str:
    """Compile libsv_synth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Spec(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("target_kind", ctypes.c_int32), ("target_scale", ctypes.c_double),
        ("zipf_s", ctypes.c_double), ("zipf_jitter", ctypes.c_double),
        ("plant", ctypes.c_int32), ("plant_value", ctypes.c_double),
        ("make_draft", ctypes.c_int32), ("sigma_first", ctypes.c_double), ("sigma_last", ctypes.c_double),
        ("token_mode", ctypes.c_int32), ("temperature", ctypes.c_double), ("p_match", ctypes.c_double),
        ("seed_target", ctypes.c_uint32), ("seed_draft", ctypes.c_uint32),
        ("seed_tokens", ctypes.c_uint32), ("seed_aux", ctypes.c_uint32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.synth_make_problem.restype = ctypes.c_int
        L.synth_make_problem.argtypes = [ctypes.POINTER(_Spec), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_uniforms.restype = None
        L.synth_uniforms.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
        L.synth_choose_tau.restype = None
        L.synth_choose_tau.argtypes = [ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        L.synth_philox4x32_10.restype = None
        L.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_philox_words.restype = None
        L.synth_philox_words.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        _lib = L
    return _lib


@dataclass(frozen=True)
class Workload:
    """One synthetic verification workload (shapes, distributions, seeds)."""
    name: str
    B: int
    K: int
    V: int
    dtype: int                 # F32 or BF16 for both logit tensors
    target_kind: int           # 0 gaussian, 1 zipf
    target_scale: float = 1.0
    zipf_s: float = 0.0
    zipf_jitter: float = 0.0
    plant: bool = False
    plant_value: float = 8.0
    make_draft: bool = True
    sigma_first: float = 0.5
    sigma_last: float = 0.5
    token_mode: int = 0        # 0 sample from q, 1 planted argmax w.p. p_match, 2 greedy drafter
    p_match: float = 0.8
    temperature: float = 1.0   # passed to the verifier; 0 = greedy
    length_mode: int = LEN_FIXED
    fixed_len: Optional[int] = None   # None -> K
    tau_choices: tuple = ()           # LEN_TAU: per-sequence tau drawn from these
    seed: int = 1                     # uniforms use key seed; other streams 100+, 200+, ...
    draft_mode: int = 0               # 0 draft probabilities; 1 one-hot drafts (the draft logits
                                      # only serve to draw the tokens and are not handed over)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny verify: 4 sequences, 4 drafted positions, V=1024, fp32; target 2*N(0,1),
    # draft = target + N(0, 0.5); T = 1; every position verified; uniform seed 1.
    "tiny": Workload("tiny", B=4, K=4, V=1024, dtype=F32, target_kind=0, target_scale=2.0,
                     sigma_first=0.5, sigma_last=0.5, temperature=1.0, seed=1),
    # Zipf-shaped rows: logit = -1.1 ln(rank) + N(0, 0.3), rank a seeded permutation per row;
    # draft = target + N(0, 0.7); B=64, K=8, V=129280, bf16; verify length 8.
    "zipf64": Workload("zipf64", B=64, K=8, V=129280, dtype=BF16, target_kind=1, zipf_s=1.1,
                       zipf_jitter=0.3, sigma_first=0.7, sigma_last=0.7, temperature=1.0, seed=2),
    # Confidence-scheduled block: B=256, K=16, V=129280, bf16, target 2*N(0,1); draft noise
    # sigma rising linearly 0.3 -> 1.5 along the block (suffix decay); c = max draft prob;
    # tau = 0.3.
    "sched256": Workload("sched256", B=256, K=16, V=129280, dtype=BF16, target_kind=0, target_scale=2.0,
                         sigma_first=0.3, sigma_last=1.5, temperature=1.0, length_mode=LEN_TAU,
                         tau_choices=(0.3,), seed=3),
    # Greedy verify: B=1024, K=8, V=129280, bf16, N(0,1) rows with one planted maximum 8.0;
    # drafted token = that argmax w.p. 0.8 else a uniform random id; T = 0.
    "greedy1024": Workload("greedy1024", B=1024, K=8, V=129280, dtype=BF16, target_kind=0, target_scale=1.0,
                           plant=True, plant_value=8.0, make_draft=False, token_mode=1, p_match=0.8,
                           temperature=0.0, seed=4),
    # Peaked rows: -1.3 ln(rank) + N(0, 0.3), fp32, sampled at T = 0.7; draft = target + N(0, 0.2);
    # B=512, K=16; per-sequence tau in {0.2, 0.4, 0.6} chosen by seed; c = max draft prob.
    "peaked512": Workload("peaked512", B=512, K=16, V=129280, dtype=F32, target_kind=1, zipf_s=1.3,
                          zipf_jitter=0.3, sigma_first=0.2, sigma_last=0.2, temperature=0.7,
                          length_mode=LEN_TAU, tau_choices=(0.2, 0.4, 0.6), seed=5),
}


@dataclass
class Problem:
    """Host arrays for one verification call (row-major, V contiguous)."""
    w: Workload
    target: np.ndarray            # [B][K+1][V] float32, or uint16 holding bf16 bits
    draft: Optional[np.ndarray]   # [B][K][V] or None
    tokens: np.ndarray            # [B][K] int32
    uniforms: np.ndarray          # [B][K+1] float32
    verify_len: Optional[np.ndarray]  # [B] int32 (fixed mode) or None (=> K)
    tau: Optional[np.ndarray]     # [B] float32 (tau mode)
    confidence: Optional[np.ndarray] = None  # [B][K] float32 (caller-provided c) or None

    @property
    def B(self): return self.w.B

    @property
    def K(self): return self.w.K

    @property
    def V(self): return self.w.V


def uniforms(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_uniforms(np.uint32(seed), n, out.ctypes.data)
    return out


def make_problem(w: Workload) -> Problem:
    """Generate the host arrays of workload ``w`` (deterministic in its seed)."""
    B, K, V = w.B, w.K, w.V
    el = np.float32 if w.dtype == F32 else np.uint16
    target = np.empty((B, K + 1, V), dtype=el)
    draft = np.empty((B, K, V), dtype=el) if w.make_draft else None
    tokens = np.empty((B, K), dtype=np.int32)
    s = _Spec(B, K, V, w.dtype, w.target_kind, w.target_scale, w.zipf_s, w.zipf_jitter,
              int(w.plant), w.plant_value, int(w.make_draft), w.sigma_first, w.sigma_last,
              w.token_mode, w.temperature if w.temperature > 0 else 1.0, w.p_match,
              100 + w.seed, 200 + w.seed, 300 + w.seed, 400 + w.seed)
    rc = lib().synth_make_problem(ctypes.byref(s), target.ctypes.data,
                                  draft.ctypes.data if draft is not None else None, tokens.ctypes.data)
    if rc != 0:
        raise RuntimeError("planted maximum not unique; pick another seed")
    if w.draft_mode == 1:
        draft = None
    u = uniforms(w.seed, B * (K + 1)).reshape(B, K + 1)
    verify_len = None
    tau = None
    if w.length_mode == LEN_FIXED and w.fixed_len is not None:
        verify_len = np.full(B, w.fixed_len, dtype=np.int32)
    if w.length_mode == LEN_TAU:
        ch = np.asarray(w.tau_choices, dtype=np.float32)
        tau = np.empty(B, dtype=np.float32)
        lib().synth_choose_tau(np.uint32(400 + w.seed), B, ch.ctypes.data, len(ch), tau.ctypes.data)
    return Problem(w, target, draft, tokens, u, verify_len, tau)


def admission_inputs(seed: int, B: int, K: int, lo: float = 0.3, a: float = 20.0, b: float = 0.05):
    """Seeded inputs of the admission decision: per-position confidences
    uniform in [lo, 1) from the Philox uniform stream (key 500 + seed), and a
    step-rate curve of a verify batch of n tokens with step time a + b n
    (n = 0 .. B (K + 1)).  A stand-in for a confidence head and a startup
    profile of the engine."""
    u = uniforms(500 + seed, B * K).reshape(B, K).astype(np.float64)
    conf = (lo + (1.0 - lo) * u).astype(np.float32)
    n = np.arange(B * (K + 1) + 1, dtype=np.float64)
    return conf, 1.0 / (a + b * n)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one counter block via the C library (for tests)."""
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.empty(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return [int(x) for x in o]


def philox_words(seed: int, row: int, stream: int, n_blocks: int) -> np.ndarray:
    o = np.empty(4 * n_blocks, dtype=np.uint32)
    lib().synth_philox_words(np.uint32(seed), np.uint32(row), np.uint32(stream), np.uint32(n_blocks), o.ctypes.data)
    return o


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32)
