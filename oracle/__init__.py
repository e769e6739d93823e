"""fp64 CPU oracle of the TokenSelect decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from . import tokenselect_oracle, tolerance  # noqa: F401
