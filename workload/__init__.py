"""Seeded synthetic workloads (control-plane stand-in and bf16 value draws)."""
from .synth import Workload, bf16_bits, build, decode, prefill, rows_values, BF16_POISON  # noqa: F401
from .configs import WORKLOADS, make  # noqa: F401
