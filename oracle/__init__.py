"""CPU oracle for weight-only int4 (W4A16) quantize-and-pack and mixed-precision matmul.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``gemv_int4_quantize_amd``) never imports it, and this package imports nothing
from the product path: the two share no code.  Inputs come from ``synth``.

Plain, slow and obviously correct: numpy fp32 arithmetic for the quantizer in
the order written in :mod:`oracle.w4a16_ref`, and float64 BLAS products for
the matmul.  Every function cites the page passage it follows.

Pinning status (what checks each function against something other than itself)
is listed at the top of :mod:`oracle.w4a16_ref`.
"""

from .w4a16_ref import *  # noqa: F401,F403
