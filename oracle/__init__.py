"""Oracle: a plain, slow, float64 CPU reference of the action-decoder layer chain.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the GPU
library (``gemm_chains_amd``) and imports nothing from it; the GPU library never
imports it.  Inputs come from the seeded generators in ``synth`` (which hold none of
the method's arithmetic) or from the tests themselves.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed forms,
brute force, special cases and library routines (see that file's docstring).
"""
from . import codec, ref  # noqa: F401
from .codec import (bf16_decode, bf16_encode, bf16_round, e4m3_decode,  # noqa: F401
                    e4m3_encode, e4m3_round)
