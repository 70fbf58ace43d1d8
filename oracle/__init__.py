"""fp64 CPU convolution oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and shares no code with it.
"""
from .oracle import (  # noqa: F401
    build,
    conv_dgrad,
    conv_fwd,
    conv_wgrad,
    num_threads,
    out_dims,
    set_num_threads,
)
