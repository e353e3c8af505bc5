"""CPU oracle (fp64, plain loops) for the group-shared fixed fan-in layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports,
links or runs anything in this package, and this package imports nothing
from the HIP library.
"""

from .oracle import (  # noqa: F401
    build,
    lib_path,
    oracle_bce,
    oracle_bwd_h,
    oracle_bwd_w,
    oracle_fwd,
    oracle_step,
)
