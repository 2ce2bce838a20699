"""spec_verify: batched draft verification on AMD Instinct MI355X.

The computation lives in libspec_verify.so (HIP kernels for gfx950 behind the C
ABI in include/spec_verify.h).  ``binding`` marshals arguments to it; ``device``
moves buffers with torch.  There is no CPU path.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
