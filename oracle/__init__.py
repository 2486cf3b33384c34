"""CPU fp64 oracle of the affine autoregressive-flow block (test infrastructure
only: imported by the tests, the smoke check and the benchmark's CPU-baseline
leg, never by the product path)."""
from .af_oracle import *  # noqa: F401,F403
from . import af_oracle  # noqa: F401
