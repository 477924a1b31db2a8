"""Seeded synthetic inputs for the Double Sparsity decode step.

Recipe (shared by the HIP path's tests and benchmark and by the oracle's tests):

* q, K, V are i.i.d. N(0, 1) drawn in float32 from one PCG64 stream per
  (sequence b, KV head g) unit, in the order K [T, d], V [T, d], q [G, d].
* A small set of outlier channels is scaled by 6 on q and K (never on V).  The
  set is per KV head and shared by every sequence and by all query heads of
  the group: a static, model-like pattern, which is what the Double Sparsity
  page relies on when it calibrates channel sparsity offline (method details;
  abstract).  The tiny fp32 workload fixes the outliers to channels 0..7.
* bf16 workloads round the float32 draws to bfloat16 with round-to-nearest-even.
  bf16 tensors travel as their raw uint16 bit patterns.
* The offline calibration set is n_calib queries per query head and n_calib
  keys per KV head, drawn the same way from a separate seed, kept in float32.
* Ragged batches draw each sequence's length uniformly from [T // 16, T] on
  their own seed, with sequence 0 at the full T; the cache holds T valid rows
  for every sequence, so rows past a sequence's length are ordinary data that
  a kernel must not use.
* Rows between T and T_cap are filled with NaN, so a kernel that reads past the
  valid tokens poisons its output.

Nothing here computes any part of the method.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import Workload, calib_seed, lengths_seed, model_seed, unit_seed

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


def outlier_channels(w: Workload) -> np.ndarray:
    """[Hkv, n_outliers] int64, ascending: the planted outlier channels per KV head."""
    if w.fixed_outliers:
        return np.tile(np.arange(w.n_outliers, dtype=np.int64), (w.Hkv, 1))
    rng = np.random.Generator(np.random.PCG64(model_seed(w)))
    return np.stack([np.sort(rng.choice(w.d, size=w.n_outliers, replace=False))
                     for _ in range(w.Hkv)]).astype(np.int64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32, copy=False)


def gen_unit(w: Workload, b: int, g: int, outl: np.ndarray | None = None):
    """Stored (K [T, d], V [T, d], q [G, d]) of one (sequence, KV head) unit."""
    if outl is None:
        outl = outlier_channels(w)
    rng = np.random.Generator(np.random.PCG64(unit_seed(w, b, g)))
    K = rng.standard_normal((w.T, w.d), dtype=np.float32)
    V = rng.standard_normal((w.T, w.d), dtype=np.float32)
    q = rng.standard_normal((w.G, w.d), dtype=np.float32)
    ch = outl[g]
    K[:, ch] *= np.float32(w.outlier_scale)
    q[:, ch] *= np.float32(w.outlier_scale)
    return _store(K, w.dtype), _store(V, w.dtype), _store(q, w.dtype)


def storage_dtype(w: Workload):
    return np.uint16 if w.dtype == "bf16" else np.float32


def _pad_value(w: Workload):
    return BF16_NAN if w.dtype == "bf16" else np.float32(np.nan)


def gen_cache(w: Workload, threads: int | None = None):
    """Whole decode batch: q [B, Hq, d], K and V [B, Hkv, T_cap, d] (stored form).

    Units are generated in parallel threads; numpy's generators release the
    GIL while filling, so this scales with cores.
    """
    sd = storage_dtype(w)
    q = np.empty((w.B, w.Hq, w.d), dtype=sd)
    K = np.empty((w.B, w.Hkv, w.cap, w.d), dtype=sd)
    V = np.empty((w.B, w.Hkv, w.cap, w.d), dtype=sd)
    if w.cap > w.T:
        K[:, :, w.T:, :] = _pad_value(w)
        V[:, :, w.T:, :] = _pad_value(w)
    outl = outlier_channels(w)

    def one(unit):
        b, g = divmod(unit, w.Hkv)
        Ku, Vu, qu = gen_unit(w, b, g, outl)
        K[b, g, :w.T] = Ku
        V[b, g, :w.T] = Vu
        q[b, g * w.G:(g + 1) * w.G] = qu

    n = w.B * w.Hkv
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if n == 1 or threads <= 1:
        for u in range(n):
            one(u)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
    return q, K, V


def gen_calib(w: Workload):
    """Offline calibration set: q_cal [n, Hq, d] and k_cal [Hkv, n, d], float32."""
    outl = outlier_channels(w)
    rng = np.random.Generator(np.random.PCG64(calib_seed(w)))
    qc = rng.standard_normal((w.n_calib, w.Hq, w.d), dtype=np.float32)
    kc = rng.standard_normal((w.Hkv, w.n_calib, w.d), dtype=np.float32)
    s = np.float32(w.outlier_scale)
    for g in range(w.Hkv):
        ch = outl[g]
        kc[g][:, ch] *= s
        for h in range(g * w.G, (g + 1) * w.G):
            qc[:, h, ch] *= s
    return qc, kc


def seq_lengths(w: Workload) -> np.ndarray:
    """int32 [B] lengths of a ragged batch: uniform in [T // 16, T], sequence 0 at T."""
    if not w.ragged:
        return np.full(w.B, w.T, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(lengths_seed(w)))
    lens = rng.integers(max(1, w.T // 16), w.T, size=w.B, endpoint=True).astype(np.int32)
    lens[0] = w.T
    return lens
