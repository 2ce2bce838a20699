"""Device plumbing around the C ABI: torch owns the buffers, the library computes.

``DeviceProblem`` uploads host arrays of one verification call to HBM and
allocates the outputs; ``launch`` enqueues one step through the binding;
``fetch`` copies the outputs back.  Nothing here computes any part of the step.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B

F32, BF16 = B.SV_F32, B.SV_BF16


def _dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device, non_blocking=False)


@dataclass
class DeviceProblem:
    B: int
    K: int
    V: int
    dtype: int
    temperature: float
    length_mode: int
    target: torch.Tensor
    draft: Optional[torch.Tensor]
    tokens: torch.Tensor
    uniforms: Optional[torch.Tensor]
    verify_len: Optional[torch.Tensor]
    confidence: Optional[torch.Tensor]
    tau: Optional[torch.Tensor]
    target_strides: tuple
    draft_strides: tuple
    # outputs
    accepted_len: torch.Tensor = None
    out_tokens: torch.Tensor = None
    verify_len_out: torch.Tensor = None
    lse_target: Optional[torch.Tensor] = None
    lse_draft: Optional[torch.Tensor] = None
    survival: Optional[torch.Tensor] = None
    residual_mass: Optional[torch.Tensor] = None
    sampled_prob: Optional[torch.Tensor] = None
    rows_read: Optional[torch.Tensor] = None
    bytes_read: Optional[torch.Tensor] = None
    device_status: Optional[torch.Tensor] = None
    draft_mode: int = B.SV_DRAFT_PROBS
    target_row_offsets: Optional[torch.Tensor] = None  # packed rows: [B+1] int64
    draft_row_offsets: Optional[torch.Tensor] = None
    max_verify_len: int = 0  # fixed lengths: the caller's bound on every L_b (0: none)

    @staticmethod
    def upload(target: np.ndarray, draft: Optional[np.ndarray], tokens: np.ndarray,
               uniforms: Optional[np.ndarray], temperature: float, dtype: int, *,
               length_mode: int = B.SV_LEN_FIXED, verify_len=None, confidence=None, tau=None,
               diagnostics: bool = True, device="cuda:0", draft_mode: int = B.SV_DRAFT_PROBS) -> "DeviceProblem":
        """Copy host arrays to the GPU.  ``target`` is [B][K+1][V] or [K+1][V]
        (shared by all sequences); bf16 is passed as uint16 bit patterns."""
        Bn, K = tokens.shape
        V = target.shape[-1]
        tstr = (0 if target.ndim == 2 else (K + 1) * V, V)
        dstr = (0, V) if draft is None else (0 if draft.ndim == 2 else K * V, V)
        if dtype == BF16:
            target = target.view(np.int16)
            draft = None if draft is None else draft.view(np.int16)
        dp = DeviceProblem(Bn, K, V, dtype, float(temperature), length_mode,
                           _dev(target, device), _dev(draft, device), _dev(tokens.astype(np.int32), device),
                           _dev(uniforms, device), _dev(verify_len, device), _dev(confidence, device),
                           _dev(tau, device), tstr, dstr)
        dp.draft_mode = int(draft_mode)
        dp.alloc_outputs(diagnostics, device)
        return dp

    def alloc_outputs(self, diagnostics: bool, device):
        Bn, K = self.B, self.K
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.accepted_len = torch.full((Bn,), -7, **i32)
        self.out_tokens = torch.full((Bn, K + 1), -7, **i32)
        self.verify_len_out = torch.full((Bn,), -7, **i32)
        self.device_status = torch.full((1,), -7, **i32)
        self.rows_read = torch.full((Bn,), -7, **i32)
        self.bytes_read = torch.full((Bn,), -7, dtype=torch.int64, device=device)
        if diagnostics:
            nan = float("nan")
            self.lse_target = torch.full((Bn, K + 1), nan, **f32)
            self.lse_draft = torch.full((Bn, K), nan, **f32)
            self.survival = torch.full((Bn, K), nan, **f32)
            self.residual_mass = torch.full((Bn,), nan, **f32)
            self.sampled_prob = torch.full((Bn,), nan, **f32)

    def args(self, counts: bool = True) -> B.Args:
        """The call's C struct; counts=False leaves out the optional stream
        counts (rows_read, bytes_read), which cost the step a little work."""
        return B.make_args(
            self.B, self.K, target=self.target, draft=self.draft, tokens=self.tokens, uniforms=self.uniforms,
            temperature=self.temperature, target_strides=self.target_strides, draft_strides=self.draft_strides,
            length_mode=self.length_mode, verify_len=self.verify_len, confidence=self.confidence, tau=self.tau,
            accepted_len=self.accepted_len, out_tokens=self.out_tokens, verify_len_out=self.verify_len_out,
            lse_target=self.lse_target, lse_draft=self.lse_draft, survival=self.survival,
            residual_mass=self.residual_mass, sampled_prob=self.sampled_prob,
            rows_read=self.rows_read if counts else None, device_status=self.device_status,
            draft_mode=self.draft_mode, target_row_offsets=self.target_row_offsets,
            draft_row_offsets=self.draft_row_offsets, bytes_read=self.bytes_read if counts else None,
            max_verify_len=self.max_verify_len)

    def fetch(self) -> dict:
        torch.cuda.synchronize()
        out = {}
        for name in ("accepted_len", "out_tokens", "verify_len_out", "device_status", "rows_read", "bytes_read",
                     "lse_target",
                     "lse_draft", "survival", "residual_mass", "sampled_prob"):
            t = getattr(self, name)
            out[name] = None if t is None else t.cpu().numpy()
        return out


def from_problem(prob, diagnostics: bool = True, device="cuda:0") -> DeviceProblem:
    """Upload a ``synth.Problem``."""
    w = prob.w
    return DeviceProblem.upload(prob.target, prob.draft, prob.tokens,
                                prob.uniforms if w.temperature > 0 else None, w.temperature, w.dtype,
                                length_mode=w.length_mode, verify_len=prob.verify_len,
                                confidence=prob.confidence, tau=prob.tau, diagnostics=diagnostics, device=device,
                                draft_mode=getattr(w, "draft_mode", B.SV_DRAFT_PROBS))


def packed_from_problem(prob, lengths: Optional[np.ndarray] = None, diagnostics: bool = True,
                        device="cuda:0") -> DeviceProblem:
    """Upload a ``synth.Problem`` in the packed ("pruned, not padded") layout:
    sequence b brings its first L_b + 1 target rows and L_b draft rows, stacked
    in sequence order, with row offsets.  ``lengths`` (default: the problem's
    fixed verify lengths, else K) gives L_b; a count outside the valid range is
    passed through as given (the library marks such a sequence bad)."""
    w = prob.w
    Bn, K = prob.tokens.shape
    if lengths is None:
        lengths = prob.verify_len if prob.verify_len is not None else np.full(Bn, K, np.int32)
    lengths = np.asarray(lengths, dtype=np.int64)
    toff = np.concatenate([[0], np.cumsum(lengths + 1)]).astype(np.int64)
    doff = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    V = prob.target.shape[-1]
    # rows a sequence declares beyond the dense tensor's K + 1 repeat its last row
    tp = np.concatenate([prob.target[b, np.minimum(np.arange(max(int(lengths[b]) + 1, 0)), K)] for b in range(Bn)]
                        + [np.zeros((0, V), prob.target.dtype)])
    dp_rows = None
    if prob.draft is not None:
        dp_rows = np.concatenate([prob.draft[b, np.minimum(np.arange(max(int(lengths[b]), 0)), K - 1)]
                                  for b in range(Bn)] + [np.zeros((0, V), prob.draft.dtype)])
    tp = np.ascontiguousarray(tp if tp.shape[0] else np.zeros((1, V), prob.target.dtype))
    if dp_rows is not None:
        dp_rows = np.ascontiguousarray(dp_rows if dp_rows.shape[0] else np.zeros((1, V), prob.draft.dtype))
    if w.dtype == BF16:
        tp = tp.view(np.int16)
        dp_rows = None if dp_rows is None else dp_rows.view(np.int16)
    d = DeviceProblem(Bn, K, V, w.dtype, float(w.temperature), B.SV_LEN_FIXED,
                      _dev(tp, device), _dev(dp_rows, device), _dev(prob.tokens.astype(np.int32), device),
                      _dev(prob.uniforms if w.temperature > 0 else None, device), None, None, None, (0, V), (0, V))
    d.draft_mode = int(getattr(w, "draft_mode", B.SV_DRAFT_PROBS))
    d.target_row_offsets = _dev(toff, device)
    d.draft_row_offsets = _dev(doff, device) if dp_rows is not None else None
    d.alloc_outputs(diagnostics, device)
    return d


def handle_for(dp: DeviceProblem, device: int = 0, max_batch: Optional[int] = None,
               max_draft: Optional[int] = None) -> B.SpecVerify:
    return B.SpecVerify(max_batch or dp.B, max_draft or dp.K, dp.V, dp.dtype, device)


def run_once(dp: DeviceProblem, sv: Optional[B.SpecVerify] = None) -> dict:
    own = sv is None
    if own:
        sv = handle_for(dp)
    sv.run(dp.args())
    res = dp.fetch()
    if own:
        sv.close()
    return res
