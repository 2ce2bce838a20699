"""Python binding of the spec_verify C ABI (ctypes; argument marshalling only).

Every step of the verification runs in the HIP kernels of libspec_verify.so.
This module only turns device tensors (torch) or raw device addresses into the
C structs declared in include/spec_verify.h.  If the library is missing it
raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspec_verify.so")

SV_OK, SV_EINVAL, SV_ENOMEM, SV_EDEVICE, SV_EUNSUPPORTED = 0, -1, -2, -3, -4
SV_F32, SV_BF16 = 0, 1
SV_LEN_FIXED, SV_LEN_TAU = 0, 1
SV_DRAFT_PROBS, SV_DRAFT_ONEHOT = 0, 1
SV_STATUS_BAD_INPUT, SV_STATUS_INCOMPLETE = 1, 2

EXPORTED = (
    "spec_verify_create", "spec_verify_check", "spec_verify_run", "spec_verify_destroy",
    "spec_verify_status_string", "spec_verify_timing_begin", "spec_verify_timing_end",
    "spec_verify_kernel_count", "spec_verify_kernel_name", "spec_verify_sched_check", "spec_verify_schedule",
    "spec_verify_conf_check", "spec_verify_confidence", "spec_verify_run_noalloc",
)
SV_MAX_CONF_DELAY = 4
SV_MAX_SCHED_BATCH, SV_MAX_SCHED_CANDIDATES = 4096, 65536
SV_NOALLOC_SCRATCH_BYTES = 16777216


class Config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_draft", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("device", ctypes.c_int32)]


class Args(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("target_batch_stride", ctypes.c_int64),
        ("target_row_stride", ctypes.c_int64),
        ("draft_logits", ctypes.c_void_p), ("draft_batch_stride", ctypes.c_int64),
        ("draft_row_stride", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p), ("uniforms", ctypes.c_void_p),
        ("temperature", ctypes.c_float), ("length_mode", ctypes.c_int32),
        ("verify_len_in", ctypes.c_void_p), ("confidence", ctypes.c_void_p), ("tau", ctypes.c_void_p),
        ("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("verify_len_out", ctypes.c_void_p),
        ("lse_target", ctypes.c_void_p), ("lse_draft", ctypes.c_void_p), ("survival", ctypes.c_void_p),
        ("residual_mass", ctypes.c_void_p), ("sampled_prob", ctypes.c_void_p), ("rows_read", ctypes.c_void_p),
        ("device_status", ctypes.c_void_p), ("draft_mode", ctypes.c_int32),
        ("target_row_offsets", ctypes.c_void_p), ("draft_row_offsets", ctypes.c_void_p),
        ("bytes_read", ctypes.c_void_p), ("max_verify_len", ctypes.c_int32),
    ]


class SchedArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("confidence", ctypes.c_void_p), ("speed", ctypes.c_void_p),
        ("n_speed", ctypes.c_int32), ("verify_len_out", ctypes.c_void_p), ("survival", ctypes.c_void_p),
        ("admitted", ctypes.c_void_p), ("tau", ctypes.c_void_p), ("expected_rate", ctypes.c_void_p),
        ("device_status", ctypes.c_void_p),
    ]


class ConfArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("conf_logits", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p), ("reset", ctypes.c_void_p), ("delay", ctypes.c_int32),
        ("c_default", ctypes.c_float), ("conf_now", ctypes.c_void_p), ("conf_out", ctypes.c_void_p),
        ("device_status", ctypes.c_void_p),
    ]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspec_verify.so (built in-tree by draft_verification_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; run draft_verification_amd.build.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.spec_verify_create.restype = ctypes.c_int
        L.spec_verify_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_void_p)]
        L.spec_verify_check.restype = ctypes.c_int
        L.spec_verify_check.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Args)]
        L.spec_verify_run.restype = ctypes.c_int
        L.spec_verify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(Args), ctypes.c_void_p]
        L.spec_verify_destroy.restype = ctypes.c_int
        L.spec_verify_destroy.argtypes = [ctypes.c_void_p]
        L.spec_verify_status_string.restype = ctypes.c_char_p
        L.spec_verify_status_string.argtypes = [ctypes.c_int]
        L.spec_verify_timing_begin.restype = ctypes.c_int
        L.spec_verify_timing_begin.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.spec_verify_timing_end.restype = ctypes.c_int
        L.spec_verify_timing_end.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]
        L.spec_verify_kernel_count.restype = ctypes.c_int32
        L.spec_verify_kernel_count.argtypes = []
        L.spec_verify_kernel_name.restype = ctypes.c_char_p
        L.spec_verify_kernel_name.argtypes = [ctypes.c_int32]
        L.spec_verify_sched_check.restype = ctypes.c_int
        L.spec_verify_sched_check.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(SchedArgs)]
        L.spec_verify_schedule.restype = ctypes.c_int
        L.spec_verify_schedule.argtypes = [ctypes.c_void_p, ctypes.POINTER(SchedArgs), ctypes.c_void_p]
        L.spec_verify_conf_check.restype = ctypes.c_int
        L.spec_verify_conf_check.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ConfArgs)]
        L.spec_verify_confidence.restype = ctypes.c_int
        L.spec_verify_confidence.argtypes = [ctypes.c_void_p, ctypes.POINTER(ConfArgs), ctypes.c_void_p]
        L.spec_verify_run_noalloc.restype = ctypes.c_int
        L.spec_verify_run_noalloc.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Args), ctypes.c_void_p]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().spec_verify_status_string(int(status)).decode()


def kernel_names() -> list:
    L = lib()
    return [L.spec_verify_kernel_name(k).decode() for k in range(L.spec_verify_kernel_count())]


def _addr(x) -> Optional[int]:
    """Device address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def make_args(B: int, K: int, *, target, draft=None, tokens, uniforms=None, temperature: float,
              target_strides: Sequence[int], draft_strides: Sequence[int] = (0, 0),
              length_mode: int = SV_LEN_FIXED, verify_len=None, confidence=None, tau=None,
              accepted_len, out_tokens, verify_len_out, lse_target=None, lse_draft=None, survival=None,
              residual_mass=None, sampled_prob=None, rows_read=None, device_status=None,
              draft_mode: int = SV_DRAFT_PROBS, target_row_offsets=None, draft_row_offsets=None,
              bytes_read=None, max_verify_len: int = 0) -> Args:
    """Fill an Args struct.  Strides are (batch, row) in elements."""
    return Args(
        B, K, _addr(target), int(target_strides[0]), int(target_strides[1]),
        _addr(draft), int(draft_strides[0]), int(draft_strides[1]),
        _addr(tokens), _addr(uniforms), float(temperature), int(length_mode),
        _addr(verify_len), _addr(confidence), _addr(tau),
        _addr(accepted_len), _addr(out_tokens), _addr(verify_len_out),
        _addr(lse_target), _addr(lse_draft), _addr(survival), _addr(residual_mass), _addr(sampled_prob),
        _addr(rows_read), _addr(device_status), int(draft_mode), _addr(target_row_offsets),
        _addr(draft_row_offsets), _addr(bytes_read), int(max_verify_len))


def check(cfg: Config, args: Args) -> int:
    """Host-only argument check (no device work)."""
    return int(lib().spec_verify_check(ctypes.byref(cfg), ctypes.byref(args)))


def make_sched_args(B: int, K: int, *, confidence, speed, n_speed: int, verify_len_out, survival=None,
                    admitted=None, tau=None, expected_rate=None, device_status=None) -> SchedArgs:
    """Fill a SchedArgs struct (device tensors or addresses)."""
    return SchedArgs(B, K, _addr(confidence), _addr(speed), int(n_speed), _addr(verify_len_out), _addr(survival),
                     _addr(admitted), _addr(tau), _addr(expected_rate), _addr(device_status))


def make_conf_args(B: int, K: int, *, conf_logits, temperature, conf_out, delay: int = 2, c_default: float = 0.0,
                   reset=None, conf_now=None, device_status=None) -> ConfArgs:
    """Fill a ConfArgs struct (device tensors or addresses)."""
    return ConfArgs(B, K, _addr(conf_logits), _addr(temperature), _addr(reset), int(delay), float(c_default),
                    _addr(conf_now), _addr(conf_out), _addr(device_status))


def conf_check(cfg: Config, args: ConfArgs) -> int:
    """Host-only check of a confidence call (no device work)."""
    return int(lib().spec_verify_conf_check(ctypes.byref(cfg), ctypes.byref(args)))


def sched_check(cfg: Config, args: SchedArgs) -> int:
    """Host-only check of an admission call (no device work)."""
    return int(lib().spec_verify_sched_check(ctypes.byref(cfg), ctypes.byref(args)))


def run_noalloc(cfg: Config, args: Args, stream: Optional[int] = None) -> None:
    """Enqueue one step without a handle: the library's static per-device
    workspace, no device allocation (see spec_verify_run_noalloc)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream(cfg.device).cuda_stream
    rc = lib().spec_verify_run_noalloc(ctypes.byref(cfg), ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_run_noalloc")


class SpecVerify:
    """Owns one spec_verify handle (and its device workspace)."""

    def __init__(self, max_batch: int, max_draft: int, vocab: int, dtype: int, device: int = 0):
        self.cfg = Config(max_batch, max_draft, vocab, dtype, device)
        h = ctypes.c_void_p()
        rc = lib().spec_verify_create(ctypes.byref(self.cfg), ctypes.byref(h))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_create")
        self._h = h

    def run(self, args: Args, stream: Optional[int] = None) -> None:
        """Enqueue one step on ``stream`` (a hipStream_t as int; None = torch's current stream)."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream(self.cfg.device).cuda_stream
        rc = lib().spec_verify_run(self._h, ctypes.byref(args), ctypes.c_void_p(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_run")

    def schedule(self, args: SchedArgs, stream: Optional[int] = None) -> None:
        """Enqueue the load-aware admission decision on ``stream``."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream(self.cfg.device).cuda_stream
        rc = lib().spec_verify_schedule(self._h, ctypes.byref(args), ctypes.c_void_p(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_schedule")

    def confidence(self, args: ConfArgs, stream: Optional[int] = None) -> None:
        """Enqueue one step of calibrated, delayed confidences on ``stream``."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream(self.cfg.device).cuda_stream
        rc = lib().spec_verify_confidence(self._h, ctypes.byref(args), ctypes.c_void_p(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_confidence")

    def timing_begin(self, max_calls: int) -> None:
        rc = lib().spec_verify_timing_begin(self._h, int(max_calls))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_timing_begin")

    def timing_end(self):
        n = lib().spec_verify_kernel_count()
        ms = (ctypes.c_double * n)()
        runs = ctypes.c_int32(0)
        rc = lib().spec_verify_timing_end(self._h, ms, n, ctypes.byref(runs))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_timing_end")
        return dict(zip(kernel_names(), list(ms))), int(runs.value)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().spec_verify_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
