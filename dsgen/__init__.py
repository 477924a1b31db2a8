"""Seeded synthetic workloads for the Double Sparsity decode step (shapes, seeds, inputs only)."""
from .configs import (Workload, WORKLOADS, WORKLOAD_ORDER, RAGGED_ORDER, THRESHOLD_ORDER, OFFLOAD_ORDER, HIP_ORDER,
                      HEADLINE, get, unit_seed, calib_seed, model_seed, lengths_seed)
from .gen import (f32_to_bf16_bits, bf16_bits_to_f32, to_f64, outlier_channels, gen_unit,
                  gen_cache, gen_calib, storage_dtype, seq_lengths)

__all__ = ["Workload", "WORKLOADS", "WORKLOAD_ORDER", "RAGGED_ORDER", "THRESHOLD_ORDER", "OFFLOAD_ORDER", "HIP_ORDER",
           "HEADLINE", "get", "unit_seed", "calib_seed", "model_seed", "lengths_seed", "seq_lengths", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "to_f64", "outlier_channels", "gen_unit", "gen_cache", "gen_calib", "storage_dtype"]
