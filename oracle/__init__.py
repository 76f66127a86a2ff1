"""fp64 CPU oracle for the KDA scan -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never does.
"""
from .kda_oracle import backward, build, forward, library_path, short_conv, short_conv_backward  # noqa: F401
