"""Seeded synthetic workload inputs (no attention arithmetic here)."""
from .inputs import (WORKLOADS, Workload, Inputs, workload, make_inputs, random_qkv,  # noqa: F401
                     bf16_round, bf16_to_f32)
