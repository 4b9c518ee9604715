"""fp64 CPU oracle for the WKV operators (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .wkv_oracle import *  # noqa: F401,F403
