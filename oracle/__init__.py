"""CPU float64 oracle for dense attention forward (test infrastructure only).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the GPU path.
"""

from .attention import attention_forward, attention_rows  # noqa: F401
