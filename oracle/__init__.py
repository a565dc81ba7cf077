"""fp64 CPU oracle of the Focus-dLLM sparse attention step.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The HIP library never does.
"""
from . import focus_oracle  # noqa: F401
