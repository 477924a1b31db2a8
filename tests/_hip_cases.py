"""Inputs of the span-search GPU tests, shared with the CPU pin that checks the oracle's
ranking precision on those same inputs.

Workload.k_units is the number of spans k, Workload.block the longest final span.
"""
from __future__ import annotations

import numpy as np

from dsgen import Workload

HIP_CASES = [
    Workload("hip_mha", "bf16", B=2, Hq=4, Hkv=4, d=128, T=5000, r=16, block=8, k_units=32, seed_base=51000),
    Workload("hip_gqa4", "bf16", B=1, Hq=16, Hkv=4, d=128, T=20000, r=16, block=16, k_units=64, seed_base=51100,
             T_cap=20100),
    Workload("hip_f32", "f32", B=1, Hq=2, Hkv=1, d=128, T=3001, r=16, block=4, k_units=40, seed_base=51200,
             fixed_outliers=True),
    Workload("hip_span1", "bf16", B=1, Hq=2, Hkv=2, d=128, T=777, r=16, block=1, k_units=50, seed_base=51300),
    Workload("hip_k1", "bf16", B=1, Hq=8, Hkv=1, d=128, T=4096, r=16, block=64, k_units=1, seed_base=51400),
    Workload("hip_k1024", "bf16", B=1, Hq=2, Hkv=1, d=128, T=65536, r=16, block=16, k_units=1024, seed_base=51500),
    Workload("hip_no_round", "bf16", B=1, Hq=4, Hkv=2, d=128, T=1000, r=16, block=64, k_units=20, seed_base=51600),
    # k <= 64 runs the one-wavefront selection, larger k the block radix selection: both sides of the boundary.
    Workload("hip_k65", "bf16", B=1, Hq=8, Hkv=2, d=128, T=30000, r=16, block=32, k_units=65, seed_base=51700),
    Workload("hip_k64_f32", "f32", B=1, Hq=4, Hkv=2, d=128, T=12345, r=16, block=8, k_units=64, seed_base=51800),
]

# Span counts of the exact-tie cases (one on each side of the two selection kernels' boundary).
TIE_KS = (48, 96)


def ties_case(k: int) -> Workload:
    """K rows repeat with period 5, so many candidates score exactly alike."""
    return Workload(f"hip_ties_k{k}", "bf16", B=1, Hq=4, Hkv=2, d=128, T=9000, r=16, block=16, k_units=k,
                    seed_base=51900 + k)


def tie_periodic_K(K: np.ndarray, T: int) -> np.ndarray:
    """A copy of the stored K whose rows 5 .. T-1 repeat rows 0 .. 4."""
    K = np.ascontiguousarray(K).copy()
    K[:, :, 5:T] = K[:, :, np.arange(5, T) % 5]
    return K
