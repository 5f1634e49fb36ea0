"""CPU oracle of the tree speculative-decoding hot path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .spec_oracle import *  # noqa: F401,F403
