"""Shared test helpers: device upload of seeded workloads and the parity rules."""
from __future__ import annotations

import numpy as np

import dsgen
import oracle as O

# Output tolerances (max-abs), by element type of q, K, V.
OUT_TOL = {"f32": 1e-5, "bf16": 2e-3}
# Boundary-tie window of the index rule, relative to the k-th largest oracle score.
TIE_REL = 1e-6


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def kth_largest(u: np.ndarray, k: int) -> float:
    return float(np.partition(np.asarray(u, dtype=np.float64), len(u) - k)[len(u) - k])


def check_index_parity(gpu_idx, u_oracle, k, what=""):
    """Kept set must equal the oracle's, except boundary ties: every unit in the
    symmetric difference must score within TIE_REL * |theta| of theta, the
    oracle's k-th largest score (TIE_REL * max|u| when theta is 0)."""
    gpu = np.asarray(gpu_idx, dtype=np.int64)
    u = np.asarray(u_oracle, dtype=np.float64)
    assert gpu.shape == (k,), (what, gpu.shape, k)
    assert np.all(np.diff(gpu) > 0), f"{what}: indices not strictly ascending"
    assert gpu[0] >= 0 and gpu[-1] < len(u), f"{what}: index out of range"
    ref = O.select_topk(u, k)
    diff = np.setxor1d(gpu, ref)
    if len(diff):
        theta = kth_largest(u, k)
        tol = TIE_REL * (abs(theta) if theta != 0 else float(np.max(np.abs(u))))
        bad = diff[np.abs(u[diff] - theta) > tol]
        assert len(bad) == 0, (f"{what}: {len(bad)} kept/dropped units outside the tie window "
                               f"(theta={theta}, tol={tol}, e.g. {bad[:5]} scores {u[bad[:5]]})")
    return len(diff)


def unit_inputs(w: dsgen.Workload, q, K, V, b, g):
    """float64 (q_group [G, d], K [T, d], V [T, d]) of one unit from the stored batch arrays."""
    G = w.G
    return (dsgen.to_f64(q[b, g * G:(g + 1) * G], w.dtype), dsgen.to_f64(K[b, g, :w.T], w.dtype),
            dsgen.to_f64(V[b, g, :w.T], w.dtype))


def check_row(qg, Kf, Vf, ch_g, k, block, T, gpu_out_g, gpu_idx_g, dtype, what, scale=None):
    """Full parity of one (sequence, KV head) row from float64 inputs (qg [G, d], Kf and Vf
    [>= T, d]): the first k index slots by the index rule, any slots after them -1, and the
    output against the oracle's attention over the GPU's kept set.  Returns (tie swaps, error)."""
    if scale is None:
        scale = O.default_scale(Kf.shape[1])
    out_ref, kept_ref, scores = O.decode_unit(qg, Kf, Vf, ch_g, k, block, scale, T)
    idx = np.asarray(gpu_idx_g)
    assert np.all(idx[k:] == -1), f"{what}: index slots past the kept count are not -1"
    swaps = check_index_parity(idx[:k], scores, k, what=what)
    S = O.tokens_of(idx[:k], block, T)
    ref = O.attend(qg, Kf, Vf, S, scale)
    err = float(np.max(np.abs(np.asarray(gpu_out_g) - ref)))
    assert err <= OUT_TOL[dtype], f"{what}: max-abs error {err} > {OUT_TOL[dtype]}"
    if swaps == 0:
        assert float(np.max(np.abs(ref - out_ref))) == 0.0
    return swaps, err


def check_unit(w, q, K, V, ch, b, g, gpu_out, gpu_idx, scale=None):
    """Full parity of one unit of a workload: kept indices by the index rule, output vs the
    oracle's attention over the GPU's kept set.  Returns (tie swaps, max-abs error)."""
    qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
    return check_row(qg, Kf, Vf, ch[g], w.k_units, w.block, w.T, gpu_out[b, g * w.G:(g + 1) * w.G],
                     gpu_idx[b, g], w.dtype, f"unit b={b} g={g}", scale)


def check_threshold_parity(gpu_idx, gpu_count, u_oracle, tau, k_max, what=""):
    """Threshold rule: the GPU's kept set (its first `gpu_count` index slots, -1 after them)
    must equal the oracle's except units whose oracle score lies within TIE_REL of a
    boundary of the rule: tau, or the k_max-th largest score when the cap can bind.
    Returns the number of such boundary swaps."""
    idx = np.asarray(gpu_idx, dtype=np.int64)
    u = np.asarray(u_oracle, dtype=np.float64)
    n = int(gpu_count)
    assert 0 <= n <= k_max and idx.shape == (k_max,), (what, n, idx.shape)
    assert np.all(idx[n:] == -1), f"{what}: slots past the count are not -1"
    got = idx[:n]
    assert np.all(np.diff(got) > 0), f"{what}: indices not strictly ascending"
    assert n == 0 or (got[0] >= 0 and got[-1] < len(u)), f"{what}: index out of range"
    ref = O.select_threshold(u, tau, k_max)
    diff = np.setxor1d(got, ref)
    if len(diff):
        bounds = [tau] if np.isfinite(tau) else []
        if k_max <= len(u):
            theta = kth_largest(u, k_max)
            if not np.isfinite(tau) or theta >= tau - TIE_REL * abs(tau):
                bounds.append(theta)
        ok = np.zeros(len(diff), dtype=bool)
        for b in bounds:
            ok |= np.abs(u[diff] - b) <= TIE_REL * (abs(b) if b != 0 else float(np.max(np.abs(u))))
        assert ok.all(), (f"{what}: {int((~ok).sum())} kept/dropped units away from the rule's boundaries "
                          f"(tau={tau}, e.g. {diff[~ok][:5]} scores {u[diff[~ok][:5]]})")
    return len(diff)


def check_threshold_unit(w, q, K, V, ch, b, g, gpu_out, gpu_idx, gpu_counts, tau, scale=None):
    """Full parity of one unit under the threshold rule: kept set by check_threshold_parity,
    output against the oracle's attention over the GPU's kept set (zero when it is empty).
    Returns (boundary swaps, max-abs error, kept count)."""
    qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
    if scale is None:
        scale = O.default_scale(w.d)
    out_ref, kept_ref, scores = O.decode_unit_threshold(qg, Kf, Vf, ch[g], w.k_units, tau, w.block, scale, w.T)
    n = int(gpu_counts[b, g])
    swaps = check_threshold_parity(gpu_idx[b, g], n, scores, tau, w.k_units, what=f"unit b={b} g={g}")
    S = O.tokens_of(gpu_idx[b, g, :n], w.block, w.T)
    ref = O.attend(qg, Kf, Vf, S, scale) if len(S) else np.zeros((w.G, w.d))
    got = gpu_out[b, g * w.G:(g + 1) * w.G]
    err = float(np.max(np.abs(got - ref)))
    assert err <= OUT_TOL[w.dtype], f"unit b={b} g={g}: max-abs error {err} > {OUT_TOL[w.dtype]}"
    if n == 0:
        assert np.all(got == 0), f"unit b={b} g={g}: nothing kept but the output is not zero"
    if swaps == 0:
        assert float(np.max(np.abs(ref - out_ref))) == 0.0
    return swaps, err, n
