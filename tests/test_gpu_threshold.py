"""GPU parity of the threshold rule (Jenga page, core method item 1) against the CPU oracle.

The decode step keeps, per (sequence, KV head) row, the units whose positive-only
aggregated score reaches tau, at most k_max of them.  Checked through the C ABI:
the positive-only scores on their own (float64 sums rounded once to float32), then
the whole step on small shapes that span several tiles with ragged tails and every
regime of the rule (rows that keep nothing, rows compacted below the cap, rows at
the cap), exact ties at tau on integer data, the two-phase split, tau = -inf / +inf,
and the full-size threshold workload in the benchmark's launch configuration.

Index rule: kept sets equal the oracle's except units within 1e-6 relative of tau
(or of the k_max-th largest score when the cap binds).  Output rule: max-abs error
against the oracle's attention over the GPU's kept set, zero when nothing is kept.
"""
import math

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dsgen
import long_context_sparse_ds_amd as L
import oracle as O
from dsgen import Workload
from _helpers import OUT_TOL, check_threshold_parity, check_threshold_unit, to_device, unit_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L.lib()   # raises if the HIP library is missing


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _setup(w):
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    return q, K, V, ch, qd, Kd, Vd, chd, label


def _oracle_scores(w, q, K, V, ch, b, g):
    qg, Kf, _ = unit_inputs(w, q, K, V, b, g)
    u = O.label_scores_positive(qg, O.label_rows(Kf, ch[g]), ch[g])
    return u if w.block == 1 else O.block_scores(u, w.block)


# (workload, quantile of row (0, 0)'s oracle scores that sets tau)
THRESH_CASES = [
    (Workload("thr_gqa4", "bf16", B=2, Hq=8, Hkv=2, d=128, T=5000, r=16, block=1, k_units=300, seed_base=31000), 0.95),
    (Workload("thr_mha_blk64", "bf16", B=1, Hq=4, Hkv=4, d=128, T=64 * 70 + 13, r=16, block=64, k_units=20,
              seed_base=31100), 0.7),
    (Workload("thr_gqa8_r8", "bf16", B=1, Hq=16, Hkv=2, d=128, T=3000, r=8, block=1, k_units=100, seed_base=31200),
     0.9),
    (Workload("thr_f32", "f32", B=1, Hq=2, Hkv=1, d=128, T=1500, r=16, block=1, k_units=77, seed_base=31300,
              fixed_outliers=True), 0.97),
    (Workload("thr_r12", "bf16", B=1, Hq=4, Hkv=2, d=128, T=2500, r=12, block=1, k_units=100, seed_base=31400),
     0.95),
    (Workload("thr_r32", "bf16", B=1, Hq=4, Hkv=2, d=128, T=4000, r=32, block=1, k_units=150, seed_base=31500),
     0.97),
    (Workload("thr_splits", "bf16", B=1, Hq=4, Hkv=4, d=128, T=16384, r=16, block=1, k_units=1024,
              seed_base=31600), 0.97),
    (Workload("thr_gqa4_blk16", "bf16", B=2, Hq=8, Hkv=2, d=128, T=16 * 500 + 7, r=16, block=16, k_units=64,
              seed_base=31700, T_cap=16 * 500 + 40), 0.85),
]


def _tau_of(w, q, K, V, ch, quant):
    return float(np.quantile(_oracle_scores(w, q, K, V, ch, 0, 0), quant))


@pytest.mark.parametrize("w,quant", THRESH_CASES, ids=[c[0].name for c in THRESH_CASES])
def test_label_scores_positive_match_oracle(w, quant):
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    s = L.ds_label_scores_positive(qd, label, chd, w.T, w.block)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            u = _oracle_scores(w, q, K, V, ch, b, g)
            # double accumulation rounded once to float32: within one float32 rounding
            np.testing.assert_allclose(s[b, g, :len(u)].astype(np.float64), u, rtol=2 ** -23, atol=1e-12)


@pytest.mark.parametrize("w,quant", THRESH_CASES, ids=[c[0].name for c in THRESH_CASES])
def test_decode_threshold_all_units(w, quant):
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    tau = _tau_of(w, q, K, V, ch, quant)
    _say(f"{w.name} tau={tau:.6g} k_max={w.k_units}")
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block)
    torch.cuda.synchronize()
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    counts = []
    for b in range(w.B):
        for g in range(w.Hkv):
            swaps, err, n = check_threshold_unit(w, q, K, V, ch, b, g, out, idx, cnt, tau)
            counts.append(n)
    _say(f"{w.name} kept counts {counts}")


@pytest.mark.parametrize("i", [0, 3, 5], ids=lambda i: THRESH_CASES[i][0].name)
def test_decode_threshold_rebuilds_label_rows(i):
    """The threshold step with the newest 37 label rows rebuilt inside the call, from a
    cache whose rows there hold garbage: the rows come back bit-exact, and indices,
    counts and outputs equal those of the same step on the intact cache (the rebuilt
    rows are scored in the same channel order)."""
    w, quant = THRESH_CASES[i]
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    tau = _tau_of(w, q, K, V, ch, quant)
    ref = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block)
    torch.cuda.synchronize()
    ref = [t.cpu() for t in ref]
    t_app = w.T - 37
    intact = label.clone()
    raw = label.view(torch.int16) if w.dtype == "bf16" else label.view(torch.int32)
    raw[:, :, t_app:w.T].fill_(0x3F00)   # garbage in the rows to be rebuilt
    _say(f"{w.name} tau={tau:.6g} t_append={t_app}")
    got = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block, t_append=t_app)
    torch.cuda.synchronize()
    assert torch.equal(label.view(torch.uint8), intact.view(torch.uint8))
    for a, b in zip(got, ref):
        assert torch.equal(a.cpu().view(torch.int32), b.view(torch.int32))


def test_decode_threshold_regimes_on_one_batch():
    """One batch whose rows fall in all three regimes at one tau: a row that keeps
    nothing, rows compacted below the cap, and a row at the cap."""
    w = Workload("thr_regimes", "bf16", B=4, Hq=8, Hkv=2, d=128, T=6000, r=16, block=1, k_units=200,
                 seed_base=31800)
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    maxima = [float(_oracle_scores(w, q, K, V, ch, b, g).max()) for b in range(w.B) for g in range(w.Hkv)]
    # tau above the smallest row maximum: that row keeps nothing
    tau = min(maxima) * 1.01
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block)
    torch.cuda.synchronize()
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    ns = []
    for b in range(w.B):
        for g in range(w.Hkv):
            ns.append(check_threshold_unit(w, q, K, V, ch, b, g, out, idx, cnt, tau)[2])
    _say(f"tau={tau:.6g} counts {ns}")
    assert min(ns) == 0
    assert max(ns) == w.k_units or any(0 < n < w.k_units for n in ns)


def test_decode_threshold_exact_ties_at_tau():
    """Integer-valued q and K: every score is an exact integer, many equal tau.  A unit
    scoring exactly tau is kept, and with exact arithmetic the kept sets are identical."""
    w = Workload("thr_ints", "bf16", B=1, Hq=4, Hkv=2, d=128, T=3000, r=16, block=1, k_units=2500,
                 seed_base=31900)
    rng = np.random.default_rng(3)
    q = dsgen.f32_to_bf16_bits(rng.integers(-2, 3, size=(w.B, w.Hq, w.d)).astype(np.float32))
    K = dsgen.f32_to_bf16_bits(rng.integers(-2, 3, size=(w.B, w.Hkv, w.T, w.d)).astype(np.float32))
    V = dsgen.f32_to_bf16_bits(rng.standard_normal((w.B, w.Hkv, w.T, w.d)).astype(np.float32))
    ch = np.sort(np.stack([rng.choice(w.d, w.r, replace=False) for _ in range(w.Hkv)]), axis=1).astype(np.int32)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    for tau in (3.0, 8.0, 0.0):
        out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block)
        torch.cuda.synchronize()
        out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
        for g in range(w.Hkv):
            u = _oracle_scores(w, q, K, V, ch, 0, g)
            assert np.all(u == np.round(u))
            want = O.select_threshold(u, tau, w.k_units)
            n = int(cnt[0, g])
            _say(f"tau={tau} g={g}: {n} kept, {int((u == tau).sum())} exactly at tau")
            assert list(idx[0, g, :n]) == list(want) and np.all(idx[0, g, n:] == -1)
            check_threshold_unit(w, q, K, V, ch, 0, g, out, idx, cnt, tau)


def test_decode_threshold_infinite_tau():
    """tau = -inf keeps the k_max largest positive-only scores (the top-k rule on them);
    tau = +inf keeps nothing: counts 0, every slot -1, zero outputs."""
    w = THRESH_CASES[0][0]
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, -math.inf, w.block)
    torch.cuda.synchronize()
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(cnt == w.k_units)
    for b in range(w.B):
        for g in range(w.Hkv):
            check_threshold_unit(w, q, K, V, ch, b, g, out, idx, cnt, -math.inf)
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, math.inf, w.block)
    torch.cuda.synchronize()
    assert torch.all(cnt == 0) and torch.all(idx == -1) and torch.all(out == 0)


def test_decode_threshold_two_phases_match_one_call():
    """ds_decode_score_threshold then ds_decode_select_attend_threshold through one workspace
    give exactly what the one call gives (the same kernels, split in two calls)."""
    w, quant = THRESH_CASES[1]
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    tau = _tau_of(w, q, K, V, ch, quant)
    lab2 = label.clone()
    o1, i1, c1 = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block,
                                                   t_append=w.T - 1)
    ws = L.ds_decode_score_threshold(qd, Kd, lab2, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
    o2, i2, c2 = L.ds_decode_select_attend_threshold(qd, Kd, Vd, w.T, w.k_units, tau, ws, w.block)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(c1, c2) and torch.equal(o1, o2) and torch.equal(label, lab2)


def test_decode_threshold_fused_label_append():
    """Label rows [t_append, T) are rebuilt inside the threshold call (planted garbage is
    overwritten bit-exactly) and the appended tokens are scored from K."""
    w, quant = THRESH_CASES[0]
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    tau = _tau_of(w, q, K, V, ch, quant)
    raw = label.view(torch.int16)
    raw[:, :, w.T - 5:w.T].fill_(0x3F00)
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, tau, w.block,
                                                      t_append=w.T - 5)
    torch.cuda.synchronize()
    assert torch.equal(label, L.ds_build_label_cache(Kd, chd))
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            check_threshold_unit(w, q, K, V, ch, b, g, out, idx, cnt, tau)


@pytest.mark.parametrize("name", dsgen.THRESHOLD_ORDER)
def test_decode_threshold_full_size_workload(name):
    """The threshold workload at full size, called as the benchmark calls it (label row
    T-1 rebuilt in the call): every row's kept set, count and output against the oracle."""
    w = dsgen.get(name)
    q, K, V, ch, qd, Kd, Vd, chd, label = _setup(w)
    out, idx, cnt = L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, label, chd, w.T, w.k_units, w.tau, w.block,
                                                      t_append=w.T - 1)
    torch.cuda.synchronize()
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(np.isfinite(out))

    def row(u):
        b, g = divmod(u, w.Hkv)
        return check_threshold_unit(w, q, K, V, ch, b, g, out, idx, cnt, w.tau)

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        res = list(ex.map(row, range(w.B * w.Hkv)))
    _say(f"{name}: counts {cnt.reshape(-1).tolist()}, boundary swaps {sum(r[0] for r in res)}, "
         f"max-abs err {max(r[1] for r in res):.3g}, empty rows {int((cnt == 0).sum())}")
    del q, K, V
    torch.cuda.empty_cache()
