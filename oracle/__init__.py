"""CPU oracle of the SLA2 forward pass (numpy, fp64): TEST INFRASTRUCTURE.

Only tests/, the package entry point's smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package.  It shares no
code with the HIP path, and the HIP path never calls it.
"""
from . import fp8_e4m3, sla2_oracle  # noqa: F401
