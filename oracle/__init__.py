"""CPU oracle for weight-absorbed Multi-head Latent Attention (test infrastructure).

This package is test infrastructure only. The product path never imports,
links or calls it; only the tests, the smoke check and the benchmark's CPU
baseline leg do. It shares no code with the HIP library: its one dependency
on this repository is the seeded input generator in `workloads`.

Everything here is plain float64 numpy written from the pages' definitions.
Each function's pins (tests in tests/test_oracle_pins.py that tie it to
something other than itself: printed values, closed forms, brute force,
invariances) are listed in its docstring.
"""
from .mla_oracle import *  # noqa: F401,F403
