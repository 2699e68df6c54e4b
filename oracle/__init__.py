"""CPU oracle of the MoE FFN forward pass -- test infrastructure only.

Only the tests, the entry module's smoke check and the benchmark's
cpu_baseline leg import this package; the HIP library never does.
"""
from . import moe_oracle
from .moe_oracle import *  # noqa: F401,F403
