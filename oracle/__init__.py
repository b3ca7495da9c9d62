"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  Parity of
every function here is pinned by ``tests/test_oracle_pins.py`` (the FP8
decoding by ``tests/test_oracle_fp8.py``).
"""

from .attention import (  # noqa: F401
    backward,
    forward,
    forward_rows,
    head_backward,
    head_forward,
    head_forward_blockwise,
    head_probabilities,
    kv_head,
    merge,
)
from .fp8 import decode_e4m3, dequantize, forward_fp8, forward_rows_fp8  # noqa: F401
