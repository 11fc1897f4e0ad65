"""MI355X-native action-decoder layer chain (gfx950 HIP kernels behind a C ABI).

``gemm_chains_amd.frt`` is the thin ctypes binding of ``libfrt.so`` (``include/frt.h``);
``gemm_chains_amd.device`` holds small torch helpers that allocate device buffers and
call it; ``gemm_chains_amd.build`` compiles the library for gfx950.
"""
from . import frt  # noqa: F401

__all__ = ["frt"]
