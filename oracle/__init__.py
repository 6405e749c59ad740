"""fp64 CPU oracle for SAS gated block-sparse attention (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import it; the device library never does.
"""
from . import sas_oracle  # noqa: F401
