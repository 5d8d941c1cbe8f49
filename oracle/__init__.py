"""CPU oracle (test infrastructure only).

Plain float64 NumPy restatement of what the block-diffusion decode step and the
dual-stream training attention compute.  Only the tests, the smoke check and
the CPU-baseline leg of the benchmark use it; the GPU library never does.
"""
from .bdiff_oracle import *  # noqa: F401,F403
from .bdiff_oracle import __all__  # noqa: F401
