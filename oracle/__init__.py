"""Oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct CPU
implementation (numpy, fp64 unless a step fixes another precision) used to check
the HIP library. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``w4a4_quantized_gemm_smooth_amd``) never imports it and shares no code with it.

Every function is in :mod:`oracle.svdquant`.
"""
from .svdquant import *  # noqa: F401,F403
