"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Each stage is checked on its own (label pack bit-exact; scores against the
oracle's float64 scores; selection fed float32 scores bit-exact against the
oracle's selection of the same values; attention fed fixed index sets), then
the whole decode step end to end: on small shapes that span several tiles
with ragged tails, edge cases, and on every unit of the
five full-size workloads in the launch configuration the benchmark times.

Index rule: kept sets equal the oracle's except boundary ties within 1e-6
relative of the oracle's k-th score.  Output rule: max-abs error against the
oracle's attention over the GPU's kept set, 1e-5 (fp32) / 2e-3 (bf16).
"""
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dsgen
import long_context_sparse_ds_amd as L
import oracle as O
from dsgen import Workload
from _helpers import OUT_TOL, check_index_parity, check_row, check_unit, to_device, unit_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L.lib()   # raises if the HIP library is missing


def _say(msg):
    print(f"[case] {msg}", flush=True)


def run_decode(w: Workload, threads=None):
    _say(f"{w.name} {w.dtype} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} cap={w.cap} r={w.r} block={w.block} "
         f"k={w.k_units}")
    q, K, V = dsgen.gen_cache(w, threads)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, w.block)
    torch.cuda.synchronize()
    return q, K, V, ch, out.cpu().numpy(), idx.cpu().numpy()


SMALL = [
    Workload("mha_ragged", "bf16", B=2, Hq=4, Hkv=4, d=128, T=3000, r=16, block=1, k_units=190, seed_base=11000,
             T_cap=3100),
    Workload("gqa8_ragged", "bf16", B=2, Hq=16, Hkv=2, d=128, T=5000, r=8, block=1, k_units=333, seed_base=12000),
    Workload("gqa4_r12", "bf16", B=1, Hq=8, Hkv=2, d=128, T=2500, r=12, block=1, k_units=100, seed_base=13000),
    Workload("gqa3", "bf16", B=1, Hq=6, Hkv=2, d=128, T=777, r=16, block=1, k_units=50, seed_base=13500),
    Workload("f32_gqa2", "f32", B=1, Hq=2, Hkv=1, d=128, T=1500, r=16, block=1, k_units=77, seed_base=14000,
             fixed_outliers=True),
    Workload("f32_r6", "f32", B=2, Hq=2, Hkv=2, d=128, T=900, r=6, block=1, k_units=64, seed_base=14500),
    Workload("block64_partial", "bf16", B=2, Hq=4, Hkv=4, d=128, T=64 * 50 + 17, r=16, block=64, k_units=9,
             seed_base=15000, T_cap=64 * 52),
    Workload("block16_gqa2", "bf16", B=1, Hq=4, Hkv=2, d=128, T=4000, r=16, block=16, k_units=20, seed_base=16000),
    Workload("dense_tokens", "bf16", B=1, Hq=2, Hkv=2, d=128, T=700, r=16, block=1, k_units=700, seed_base=17000),
    Workload("dense_blocks", "bf16", B=1, Hq=2, Hkv=2, d=128, T=64 * 7 + 5, r=16, block=64, k_units=8,
             seed_base=17500),
    Workload("k1", "bf16", B=1, Hq=2, Hkv=2, d=128, T=4097, r=16, block=1, k_units=1, seed_base=18000),
    Workload("T1", "bf16", B=2, Hq=2, Hkv=2, d=128, T=1, r=16, block=1, k_units=1, seed_base=18500, T_cap=64),
    Workload("r_eq_d", "bf16", B=1, Hq=2, Hkv=2, d=128, T=2000, r=128, block=1, k_units=125, seed_base=19000),
    Workload("select_multi_tile", "bf16", B=1, Hq=1, Hkv=1, d=128, T=70001, r=16, block=1, k_units=4000,
             seed_base=19500),
    # Groups of 8 and 16 query heads: several 4-head chunks per row, each a workgroup of its own (fp32, a block
    # variant, and G = 16 on 8 rows, which takes the XCD-grouped grid with four head chunks per row).
    Workload("f32_gqa8", "f32", B=1, Hq=8, Hkv=1, d=128, T=1200, r=16, block=1, k_units=100, seed_base=19600,
             fixed_outliers=True),
    Workload("gqa8_block16", "bf16", B=1, Hq=16, Hkv=2, d=128, T=4000, r=16, block=16, k_units=25, seed_base=19700),
    Workload("gqa16_rows8", "bf16", B=4, Hq=32, Hkv=2, d=128, T=3000, r=8, block=1, k_units=150, seed_base=19800),
    # One head per row, 8 rows (the XCD-grouped grid) and 8 splits per row: a padded cache, a kept count that
    # leaves the last split one token (449 = 7 * 64 + 1), 10 tiles (the 16-tile selection), every token kept.
    Workload("mha_cs_rows8", "bf16", B=2, Hq=4, Hkv=4, d=128, T=6000, r=16, block=1, k_units=512, seed_base=19900,
             T_cap=6100),
    Workload("mha_cs_k449_tiles10", "bf16", B=1, Hq=8, Hkv=8, d=128, T=20000, r=8, block=1, k_units=449,
             seed_base=19910),
    Workload("mha_cs_dense", "bf16", B=1, Hq=8, Hkv=8, d=128, T=500, r=16, block=1, k_units=500, seed_base=19920),
    # 256 rows: one workgroup per row, which builds the row's top-digit histogram itself
    Workload("rows256_one_split", "bf16", B=32, Hq=8, Hkv=8, d=128, T=2500, r=16, block=1, k_units=100,
             seed_base=19950),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_decode_small_all_units(w):
    q, K, V, ch, out, idx = run_decode(w)
    assert np.all(np.isfinite(out))
    for b in range(w.B):
        for g in range(w.Hkv):
            check_unit(w, q, K, V, ch, b, g, out, idx)


def check_all_units(w, q, K, V, ch, out, idx):
    """check_unit on every (sequence, KV head) unit, spread over host threads (numpy's
    conversions, products and sorts release the GIL).  Returns (tie swaps, worst error)."""
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    n = max(1, min(16, len(os.sched_getaffinity(0)), len(units)))
    with ThreadPoolExecutor(n) as ex:
        res = list(ex.map(lambda u: check_unit(w, q, K, V, ch, u[0], u[1], out, idx), units))
    return sum(r[0] for r in res), max(r[1] for r in res)


@pytest.mark.parametrize("name", dsgen.WORKLOAD_ORDER)
def test_decode_full_size_workload(name):
    """The five workloads at full size, in the benchmark's launch configuration: every
    (sequence, KV head) unit's kept set and output against the oracle."""
    w = dsgen.get(name)
    q, K, V, ch, out, idx = run_decode(w)
    assert np.all(np.isfinite(out))
    rows = idx.reshape(-1, w.k_units)
    assert np.all(np.diff(rows, axis=1) > 0) and rows.min() >= 0 and rows.max() < w.n_units
    swaps, err = check_all_units(w, q, K, V, ch, out, idx)
    _say(f"{name}: all {w.B * w.Hkv} units checked, tie swaps {swaps}, max-abs err {err:.3g}")
    del q, K, V
    torch.cuda.empty_cache()


def test_label_pack_bit_exact_and_append_leaves_other_rows():
    w = Workload("pack", "bf16", B=2, Hq=4, Hkv=2, d=128, T=1000, r=16, block=1, k_units=10, seed_base=20000,
                 T_cap=1030)
    q, K, V = dsgen.gen_cache(w)
    ch = np.sort(np.random.default_rng(1).choice(128, (w.Hkv, w.r)), axis=1).astype(np.int32)
    Kd = to_device(K, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = torch.full((w.B, w.Hkv, w.cap, w.r), 0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    label.view(torch.int16).fill_(0x1234)
    L.ds_build_label_cache(Kd, chd, 0, 600, label=label)
    L.ds_build_label_cache(Kd, chd, 600, 601, label=label)   # one appended row
    torch.cuda.synchronize()
    got = label.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(w.B):
        for g in range(w.Hkv):
            want = O.label_rows(K[b, g], ch[g])
            np.testing.assert_array_equal(got[b, g, :601], want[:601])
            assert np.all(got[b, g, 601:] == 0x1234)
    # fp32 cache
    wf = w.with_(dtype="f32", seed_base=20500)
    qf, Kf, Vf = dsgen.gen_cache(wf)
    lab = L.ds_build_label_cache(to_device(Kf, "f32"), chd)
    torch.cuda.synchronize()
    for b in range(w.B):
        for g in range(w.Hkv):
            np.testing.assert_array_equal(lab.cpu().numpy()[b, g, :w.T], O.label_rows(Kf[b, g, :w.T], ch[g]))


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[2], SMALL[4], SMALL[5], SMALL[6], SMALL[7]],
                         ids=lambda w: w.name)
def test_label_scores_match_oracle(w):
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = O.calibrate_channels(qc, kc, w.Hkv, w.r)
    qd, Kd = to_device(q, w.dtype), to_device(K, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    s = L.ds_label_scores(qd, label, chd, w.T, w.block)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            qg, Kf, _ = unit_inputs(w, q, K, V, b, g)
            u = O.label_scores(qg, O.label_rows(Kf, ch[g]), ch[g])
            if w.block > 1:
                u = O.block_scores(u, w.block)
            got = s[b, g, :len(u)].astype(np.float64)
            # double accumulation rounded once to float32: within one float32 rounding
            np.testing.assert_allclose(got, u, rtol=2 ** -23, atol=1e-12)


SELECT_CASES = [
    ("ints_ties", 3, 5000, 700, "ints"),
    ("tiny_n1", 2, 1, 1, "normal"),
    ("n7_all", 1, 7, 7, "normal"),
    ("all_equal", 2, 9000, 1234, "equal"),
    ("signed_zeros", 2, 300, 150, "zeros"),
    ("tile_edge", 2, 4096, 4096, "normal"),
    ("tile_edge_plus1", 2, 4097, 100, "ints"),
    ("long_row", 3, 131072, 8192, "normal"),
    ("long_row_ties", 2, 100003, 6250, "ints"),
    ("negative", 2, 2000, 1999, "negative"),
]


@pytest.mark.parametrize("name,rows,n,k,kind", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_topk_select_bit_exact(name, rows, n, k, kind):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if kind == "ints":
        u = rng.integers(-20, 21, size=(rows, n)).astype(np.float32)
    elif kind == "equal":
        u = np.full((rows, n), 3.5, np.float32)
    elif kind == "zeros":
        u = np.where(rng.random((rows, n)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        u[:, ::7] = 1.0
    elif kind == "negative":
        u = -np.abs(rng.standard_normal((rows, n))).astype(np.float32) * 100
    else:
        u = (rng.standard_normal((rows, n)) * 100).astype(np.float32)
    ld = n + 5
    buf = np.zeros((rows, ld), np.float32)
    buf[:, :n] = u
    idx = L.ds_topk_select(torch.from_numpy(buf).cuda(), n, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for i in range(rows):
        np.testing.assert_array_equal(idx[i], O.select_topk(u[i].astype(np.float64), k), err_msg=f"{name} row {i}")


ATTN_CASES = [
    Workload("attn_mha", "bf16", B=2, Hq=4, Hkv=4, d=128, T=3000, r=16, block=1, k_units=211, seed_base=21000),
    Workload("attn_gqa8", "bf16", B=1, Hq=16, Hkv=2, d=128, T=4000, r=8, block=1, k_units=999, seed_base=22000),
    Workload("attn_f32", "f32", B=1, Hq=2, Hkv=2, d=128, T=1024, r=16, block=1, k_units=64, seed_base=23000),
    Workload("attn_block", "bf16", B=1, Hq=4, Hkv=4, d=128, T=64 * 30 + 9, r=16, block=64, k_units=7,
             seed_base=24000),
]


@pytest.mark.parametrize("w", ATTN_CASES, ids=lambda w: w.name)
def test_sparse_attention_from_fixed_indices(w):
    q, K, V = dsgen.gen_cache(w)
    rng = np.random.default_rng(5)
    idx = np.stack([np.stack([np.sort(rng.choice(w.n_units, w.k_units, replace=False)) for _ in range(w.Hkv)])
                    for _ in range(w.B)]).astype(np.int32)
    if w.block > 1:   # make one row keep the partial last block
        idx[0, 0] = np.append(np.sort(rng.choice(w.n_units - 1, w.k_units - 1, replace=False)), w.n_units - 1)
    out = L.ds_sparse_attn_from_indices(to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype),
                                        torch.from_numpy(idx).cuda(), w.T, w.block)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
            S = O.tokens_of(idx[b, g], w.block, w.T)
            ref = O.attend(qg, Kf, Vf, S, O.default_scale(w.d))
            err = np.max(np.abs(out[b, g * w.G:(g + 1) * w.G] - ref))
            assert err <= OUT_TOL[w.dtype], (b, g, err)


def test_decode_is_deterministic_and_address_independent():
    w = SMALL[1]
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, chd)
    o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units)
    o2, i2 = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units)
    # a copy of the instance at other addresses
    o3, i3 = L.ds_decode_sparse_attn(qd.clone(), Kd.clone(), Vd.clone(), label.clone(), chd.clone(), w.T, w.k_units)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(i1, i3)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(o1.view(torch.int32), o3.view(torch.int32))


def test_decode_scale_argument():
    w = SMALL[0]
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    chd = torch.from_numpy(ch).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, chd)
    out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, scale=0.02)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            check_unit(w, q, K, V, ch, b, g, out, idx, scale=0.02)


def test_workspace_reuse_and_graph_replay_match_eager():
    """One workspace reused across calls (the merge counters reset themselves), and the
    decode step captured in a HIP graph: every replay, with eager work and
    synchronisation in between, must reproduce the eager result bit for bit."""
    w = SMALL[1]   # several splits per row: exercises the cross-split merge
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, chd)
    ref_o, ref_i = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units)
    ws = L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units)
    ws.fill_(0xA5)   # arbitrary contents on entry
    out = torch.empty_like(ref_o)
    idx = torch.empty_like(ref_i)
    for _ in range(3):
        L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, out=out, indices=idx, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i) and torch.equal(out.view(torch.int32), ref_o.view(torch.int32))
    # a different shape through the same workspace in between must not disturb it
    L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T - 100, 50, workspace=ws)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, out=out, indices=idx, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, out=out, indices=idx, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), rep
        assert torch.equal(out.view(torch.int32), ref_o.view(torch.int32)), rep
        # eager work between replays
        o2, _ = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int32), ref_o.view(torch.int32))


APPEND_CASES = [SMALL[0], SMALL[4], SMALL[6],
                # the 37 rebuilt rows straddle two 2048-token score tiles (17 + 20)
                Workload("append_two_tiles", "bf16", B=1, Hq=4, Hkv=2, d=128, T=2068, r=16, block=1, k_units=150,
                         seed_base=19900)]


@pytest.mark.parametrize("w", APPEND_CASES, ids=lambda w: w.name)
def test_decode_fused_label_append(w):
    """Label rows [t_append, T) are rebuilt from K inside the decode call: start from a
    cache whose newest rows hold garbage and check they come back bit-exact and the
    step matches the oracle.  37 rows: more than the score kernel stages per tile, so
    both the staged and the direct K reads are taken."""
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    chd = torch.from_numpy(ch).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, chd)
    t_app = w.T - 37
    raw = label.view(torch.int16) if w.dtype == "bf16" else label.view(torch.int32)
    raw[:, :, t_app:w.T].fill_(0x3F00)   # garbage in the rows to be appended
    out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, w.block, t_append=t_app)
    torch.cuda.synchronize()
    got = label.cpu().view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else label.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            np.testing.assert_array_equal(got[b, g, :w.T], O.label_rows(K[b, g, :w.T], ch[g]))
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            check_unit(w, q, K, V, ch, b, g, out, idx)


FUSED_CASES = [SMALL[0], SMALL[1], SMALL[2], SMALL[4], SMALL[6], SMALL[7], SMALL[8], SMALL[13],
               Workload("many_splits", "bf16", B=1, Hq=2, Hkv=2, d=128, T=30000, r=16, block=1, k_units=9000,
                        seed_base=25000)]


@pytest.mark.parametrize("w", FUSED_CASES, ids=lambda w: w.name)
def test_select_attention_from_oracle_scores(w):
    """Selection + attention fed the oracle's float64 scores rounded to float32: the kept
    set must equal the oracle's selection of those same float32 values exactly, and the
    output must match the oracle's attention over it."""
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = O.calibrate_channels(qc, kc, w.Hkv, w.r)
    ld = -(-w.n_units // 4) * 4
    sc = np.zeros((w.B, w.Hkv, ld), np.float32)
    units = {}
    for b in range(w.B):
        for g in range(w.Hkv):
            qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
            u = O.label_scores(qg, O.label_rows(Kf, ch[g]), ch[g])
            if w.block > 1:
                u = O.block_scores(u, w.block)
            sc[b, g, :len(u)] = u.astype(np.float32)
            units[b, g] = (qg, Kf, Vf)
    out, idx = L.ds_select_attention(to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype),
                                     torch.from_numpy(sc).cuda(), w.T, w.k_units, w.block)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    for (b, g), (qg, Kf, Vf) in units.items():
        want = O.select_topk(sc[b, g, :w.n_units].astype(np.float64), w.k_units)
        np.testing.assert_array_equal(idx[b, g], want, err_msg=f"unit ({b},{g})")
        ref = O.attend(qg, Kf, Vf, O.tokens_of(want, w.block, w.T), O.default_scale(w.d))
        err = float(np.max(np.abs(out[b, g * w.G:(g + 1) * w.G] - ref)))
        assert err <= OUT_TOL[w.dtype], (b, g, err)


def test_alternating_inputs_through_one_workspace():
    """Split states of one call must never leak into the next: two different decode
    inputs alternate through one workspace (cross-split merge every call) and each
    result must equal that input's own reference bit for bit."""
    w = SMALL[1]
    refs, ins = [], []
    for seed in (40000, 41000):
        wi = w.with_(seed_base=seed)
        q, K, V = dsgen.gen_cache(wi)
        qc, kc = dsgen.gen_calib(wi)
        chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, wi.r)).cuda()
        qd, Kd, Vd = to_device(q, wi.dtype), to_device(K, wi.dtype), to_device(V, wi.dtype)
        label = L.ds_build_label_cache(Kd, chd)
        o, i = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, wi.T, wi.k_units)
        torch.cuda.synchronize()
        refs.append((o.clone(), i.clone()))
        ins.append((qd, Kd, Vd, label, chd))
    ws = L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units)
    outs = []
    for rep in range(24):
        qd, Kd, Vd, label, chd = ins[rep % 2]
        outs.append(L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, workspace=ws))
    torch.cuda.synchronize()
    for rep, (o, i) in enumerate(outs):
        ro, ri = refs[rep % 2]
        assert torch.equal(i, ri), rep
        assert torch.equal(o.view(torch.int32), ro.view(torch.int32)), rep


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[4], SMALL[6], SMALL[13],
                               Workload("two_stage_gqa8", "bf16", B=1, Hq=16, Hkv=2, d=128, T=40001, r=8, block=1,
                                        k_units=900, seed_base=29500)], ids=lambda w: w.name)
def test_two_phase_decode_equals_single_call(w):
    """ds_decode_score then ds_decode_select_attend through one workspace must give exactly
    the results of ds_decode_sparse_attn (same kernels), including the fused label append."""
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, chd)
    o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, w.block, t_append=w.T - 3)
    ws = L.ds_decode_score(qd, Kd, label, chd, w.T, w.k_units, w.block, t_append=w.T - 3)
    o2, i2 = L.ds_decode_select_attend(qd, Kd, Vd, w.T, w.k_units, ws, w.block)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def _adversarial_row(kind, n, rng):
    """Finite float32 score rows that stress the selection's digit bounds and tie rule."""
    if kind == "ints":          # heavy exact ties everywhere, also at the k-th score
        return rng.integers(-6, 7, size=n).astype(np.float32)
    if kind == "equal":         # one value: the k lowest ids are kept
        return np.full(n, -2.75, np.float32)
    if kind == "zeros":         # +0.0 / -0.0 are one key; a few positives above them
        u = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        u[::97] = 1.0
        return u
    if kind == "denormal":      # positive and negative subnormals around zero
        mags = rng.integers(1, 1 << 12, size=n).astype(np.uint32)
        signs = np.where(rng.random(n) < 0.5, np.uint32(0x80000000), np.uint32(0))
        return (mags | signs).view(np.float32)
    if kind == "boundaries":    # powers of two and their neighbours: values on the 11-bit digit edges
        sign = np.where(rng.random(n) < 0.3, -1.0, 1.0)
        base = (sign * np.ldexp(1.0, rng.integers(-3, 4, size=n))).astype(np.float32)
        step = rng.integers(-1, 2, size=n)
        up = np.nextafter(base, np.float32(np.inf))
        down = np.nextafter(base, np.float32(-np.inf))
        return np.where(step > 0, up, np.where(step < 0, down, base)).astype(np.float32)
    if kind == "one_digit":     # every score in one top digit: all are candidates
        return (1.0 + rng.random(n) * 0.2).astype(np.float32)
    if kind == "huge":          # magnitudes near the float32 maximum
        return (rng.standard_normal(n) * 1e37).astype(np.float32)
    raise ValueError(kind)


ADV_KINDS = ["ints", "equal", "zeros", "denormal", "boundaries", "one_digit", "huge"]
ADV_SHAPES = [(3000, 1000), (5000, 4999), (16384, 1024), (30000, 9000), (777, 1)]


@pytest.mark.parametrize("kind", ADV_KINDS)
def test_select_attention_adversarial_scores(kind):
    """Selection inside the fused kernel on caller score rows built to sit on digit
    bounds, signed zeros, subnormals and exact ties: kept ids bit-exact against the
    oracle's selection of the same float32 values, outputs against the oracle."""
    for T, k in ADV_SHAPES:
        w = Workload(f"adv_{kind}_{T}", "bf16", B=1, Hq=4, Hkv=2, d=128, T=T, r=16, block=1, k_units=k,
                     seed_base=26000 + T)
        _say(f"{w.name} k={k}")
        q, K, V = dsgen.gen_cache(w)
        rng = np.random.default_rng(zlib.crc32(w.name.encode()))
        ld = -(-T // 4) * 4
        sc = np.zeros((1, 2, ld), np.float32)
        for g in range(2):
            sc[0, g, :T] = _adversarial_row(kind, T, rng)
        out, idx = L.ds_select_attention(to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"),
                                         torch.from_numpy(sc).cuda(), T, k, 1)
        torch.cuda.synchronize()
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        for g in range(2):
            want = O.select_topk(sc[0, g, :T].astype(np.float64), k)
            np.testing.assert_array_equal(idx[0, g], want, err_msg=f"{w.name} g={g}")
            qg, Kf, Vf = unit_inputs(w, q, K, V, 0, g)
            ref = O.attend(qg, Kf, Vf, want, O.default_scale(w.d))
            err = float(np.max(np.abs(out[0, g * 2:(g + 1) * 2] - ref)))
            assert err <= OUT_TOL["bf16"], (w.name, g, err)


def _bf16_ints(arr):
    """Small integers are exact in bfloat16: the bit patterns of those values."""
    return dsgen.f32_to_bf16_bits(np.ascontiguousarray(arr, dtype=np.float32))


@pytest.mark.parametrize("T,k,span", [(20000, 3000, 2), (9000, 4500, 0), (32768, 777, 1)],
                         ids=["ties_20k", "q_zero_9k", "ties_32k"])
def test_decode_integer_scores_exact_ties(T, k, span):
    """The whole decode step (score kernel with its tile histograms, then the fused
    kernel) on q and K with small integer values, so every score is an exact integer
    and the k-th score is shared by many tokens (span 0: q = 0, all scores equal).
    Ties go to the lower token id on both sides, so the kept ids match exactly."""
    B, Hq, Hkv, d, r = 1, 4, 2, 128, 8
    rng = np.random.default_rng(T + span)
    qf = rng.integers(-span, span + 1, size=(B, Hq, d)).astype(np.float32)
    Kf = rng.integers(-2, 3, size=(B, Hkv, T, d)).astype(np.float32)
    Vf = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    ch = np.stack([np.sort(rng.choice(d, r, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    q, K, V = _bf16_ints(qf), _bf16_ints(Kf), _bf16_ints(Vf)
    _say(f"integer scores T={T} k={k} span={span}")
    qd, Kd, Vd = to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, T, k, 1)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    w = Workload("ints", "bf16", B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, r=r, block=1, k_units=k, seed_base=0)
    for g in range(Hkv):
        qg, Kg, Vg = unit_inputs(w, q, K, V, 0, g)
        u = O.label_scores(qg, O.label_rows(Kg, ch[g]), ch[g])
        want = O.select_topk(u, k)
        np.testing.assert_array_equal(idx[0, g], want, err_msg=f"g={g}")
        ref = O.attend(qg, Kg, Vg, want, O.default_scale(d))
        err = float(np.max(np.abs(out[0, g * 2:(g + 1) * 2] - ref)))
        assert err <= OUT_TOL["bf16"], (g, err)


RAGGED_CASES = [
    # (workload shape, per-sequence lengths, rows rebuilt per sequence)
    (Workload("ragged_mha", "bf16", B=4, Hq=2, Hkv=2, d=128, T=5000, r=16, block=1, k_units=300, seed_base=27000),
     [5000, 1, 777, 3001], 1),
    (Workload("ragged_gqa4", "bf16", B=3, Hq=8, Hkv=2, d=128, T=9000, r=8, block=1, k_units=256, seed_base=27100),
     [9000, 2049, 100], 3),
    (Workload("ragged_block64", "bf16", B=3, Hq=2, Hkv=2, d=128, T=64 * 40 + 5, r=16, block=64, k_units=8,
              seed_base=27200), [64 * 40 + 5, 64 * 3 + 1, 10], 2),
    (Workload("ragged_f32", "f32", B=2, Hq=1, Hkv=1, d=128, T=1500, r=16, block=1, k_units=77, seed_base=27300,
              fixed_outliers=True), [1500, 64], 1),
    (Workload("ragged_gqa8", "bf16", B=4, Hq=16, Hkv=2, d=128, T=6000, r=8, block=1, k_units=400, seed_base=27400),
     [6000, 333, 4097, 1], 2),
]


@pytest.mark.parametrize("w,lens,n_append", RAGGED_CASES, ids=[c[0].name for c in RAGGED_CASES])
def test_decode_ragged_lengths(w, lens, n_append):
    """Sequences of unequal lengths in one call: each (sequence, KV head) row is the
    oracle's decode of its own prefix of T_b tokens keeping min(k, its units) units;
    index slots past that are -1; the last n_append label rows of every sequence are
    rebuilt from K (planted garbage is overwritten bit-exactly)."""
    _say(f"{w.name} lens={lens} n_append={n_append} k={w.k_units}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    raw = label.view(torch.int16) if w.dtype == "bf16" else label.view(torch.int32)
    for b, Tb in enumerate(lens):
        raw[b, :, max(Tb - n_append, 0):Tb].fill_(0x3F00)   # garbage where the append must write
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, idx = L.ds_decode_sparse_attn_ragged(qd, Kd, Vd, label, chd, seq, w.T, w.k_units, w.block,
                                              n_append=n_append)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    want_label = L.ds_build_label_cache(Kd, chd)
    torch.cuda.synchronize()
    assert torch.equal(label, want_label), "appended label rows not rebuilt exactly"
    scale = O.default_scale(w.d)
    for b, Tb in enumerate(lens):
        n_b = -(-Tb // w.block)
        k_b = min(w.k_units, n_b)
        for g in range(w.Hkv):
            qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
            out_ref, kept, scores = O.decode_unit(qg, Kf[:Tb], Vf[:Tb], ch[g], k_b, w.block, scale, Tb)
            check_index_parity(idx[b, g, :k_b], scores, k_b, what=f"{w.name} b={b} g={g}")
            assert np.all(idx[b, g, k_b:] == -1), (b, g)
            ref = O.attend(qg, Kf[:Tb], Vf[:Tb], O.tokens_of(idx[b, g, :k_b], w.block, Tb), scale)
            err = float(np.max(np.abs(out[b, g * w.G:(g + 1) * w.G] - ref)))
            assert err <= OUT_TOL[w.dtype], (w.name, b, g, err)


def test_decode_ragged_equal_lengths_match_uniform_call():
    """All sequences at the full length: the ragged call returns exactly the uniform call's results."""
    w = SMALL[1]   # gqa8_ragged: B=2, Hq=16, Hkv=2, T=5000
    _say(f"ragged == uniform on {w.name}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    label = L.ds_build_label_cache(Kd, ch)
    o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, label, ch, w.T, w.k_units, w.block, t_append=w.T - 1)
    seq = torch.full((w.B,), w.T, dtype=torch.int32, device="cuda")
    o2, i2 = L.ds_decode_sparse_attn_ragged(qd, Kd, Vd, label, ch, seq, w.T, w.k_units, w.block, n_append=1)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("case", [RAGGED_CASES[0], RAGGED_CASES[2]], ids=lambda c: c[0].name)
def test_decode_ragged_two_phases_match_one_call(case):
    """ds_decode_score_ragged then ds_decode_select_attend_ragged through one workspace give
    exactly what ds_decode_sparse_attn_ragged gives (the same kernels, split in two calls)."""
    w, lens, n_append = case
    _say(f"ragged two phases on {w.name} lens={lens}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lab1 = L.ds_build_label_cache(Kd, ch)
    lab2 = lab1.clone()
    o1, i1 = L.ds_decode_sparse_attn_ragged(qd, Kd, Vd, lab1, ch, seq, w.T, w.k_units, w.block, n_append=n_append)
    ws = L.ds_decode_score_ragged(qd, Kd, lab2, ch, seq, w.T, w.k_units, w.block, n_append=n_append)
    o2, i2 = L.ds_decode_select_attend_ragged(qd, Kd, Vd, seq, w.T, w.k_units, ws, w.block)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    assert torch.equal(lab1, lab2)


@pytest.mark.parametrize("name", dsgen.RAGGED_ORDER)
def test_decode_ragged_full_size_workload(name):
    """The ragged benchmark batch at full size, called as the benchmark calls it (one label
    row rebuilt per sequence): every (sequence, KV head) row against the oracle over its own
    length (kept count min(k, T_b), -1 after it)."""
    w = dsgen.get(name)
    lens = dsgen.seq_lengths(w)
    _say(f"{w.name} lens={lens.tolist()} k={w.k_units}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    seq = torch.from_numpy(lens).cuda()
    out, idx = L.ds_decode_sparse_attn_ragged(qd, Kd, Vd, label, chd, seq, w.T, w.k_units, w.block, n_append=1)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    assert np.all(np.isfinite(out))

    def row(u):
        b, g = divmod(u, w.Hkv)
        Tb = int(lens[b])
        qg, Kf, Vf = unit_inputs(w, q, K, V, b, g)
        return check_row(qg, Kf, Vf, ch[g], min(w.k_units, -(-Tb // w.block)), w.block, Tb,
                         out[b, g * w.G:(g + 1) * w.G], idx[b, g], w.dtype, f"{w.name} b={b} g={g} T_b={Tb}")

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        res = list(ex.map(row, range(w.B * w.Hkv)))
    _say(f"{name}: all {w.B * w.Hkv} rows checked, tie swaps {sum(r[0] for r in res)}, "
         f"max-abs err {max(r[1] for r in res):.3g}")
    del q, K, V
    torch.cuda.empty_cache()


LONG_ADV_SHAPES = [(70000, 3000), (32868, 500), (65536, 16384)]


@pytest.mark.parametrize("kind", ADV_KINDS)
def test_long_rows_two_stage_selection_adversarial(kind):
    """Rows longer than 32,768 units whose partitions' candidates fit the fused kernel
    (a per-partition top k, then the fused kernel over the candidates): the adversarial
    score rows again, with a last partition shorter than k (32,868 units, k = 500) and
    the largest candidate set (two partitions of k = 16,384).  Kept ids bit-exact
    against the oracle's selection of the same float32 values."""
    for T, k in LONG_ADV_SHAPES:
        w = Workload(f"long_{kind}_{T}", "bf16", B=1, Hq=4, Hkv=2, d=128, T=T, r=16, block=1, k_units=k,
                     seed_base=28000 + T)
        _say(f"{w.name} k={k}")
        q, K, V = dsgen.gen_cache(w)
        rng = np.random.default_rng(zlib.crc32(w.name.encode()))
        ld = -(-T // 4) * 4
        sc = np.zeros((1, 2, ld), np.float32)
        for g in range(2):
            sc[0, g, :T] = _adversarial_row(kind, T, rng)
        out, idx = L.ds_select_attention(to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"),
                                         torch.from_numpy(sc).cuda(), T, k, 1)
        torch.cuda.synchronize()
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        for g in range(2):
            want = O.select_topk(sc[0, g, :T].astype(np.float64), k)
            np.testing.assert_array_equal(idx[0, g], want, err_msg=f"{w.name} g={g}")
            qg, Kf, Vf = unit_inputs(w, q, K, V, 0, g)
            ref = O.attend(qg, Kf, Vf, want, O.default_scale(w.d))
            err = float(np.max(np.abs(out[0, g * 2:(g + 1) * 2] - ref)))
            assert err <= OUT_TOL["bf16"], (w.name, g, err)


@pytest.mark.parametrize("w", [
    Workload("long_gqa4", "bf16", B=1, Hq=8, Hkv=2, d=128, T=70000, r=8, block=1, k_units=2000, seed_base=29000),
    Workload("long_blk2", "bf16", B=1, Hq=2, Hkv=2, d=128, T=2 * 40000 + 1, r=16, block=2, k_units=5000,
             seed_base=29100),
    # groups of 8 and 16 query heads: eight heads per workgroup (matrix cores in bf16, the lane path in fp32)
    Workload("long_gqa8", "bf16", B=2, Hq=16, Hkv=2, d=128, T=70001, r=8, block=1, k_units=2001, seed_base=29200),
    Workload("long_gqa16", "bf16", B=1, Hq=32, Hkv=2, d=128, T=40000, r=8, block=1, k_units=1500, seed_base=29300),
    Workload("long_gqa8_f32", "f32", B=1, Hq=8, Hkv=1, d=128, T=40000, r=16, block=1, k_units=700,
             seed_base=29400),
], ids=lambda w: w.name)
def test_decode_long_rows_two_stage(w):
    """The whole decode step on rows of more than 32,768 units (token-level with GQA groups of 4, 8
    and 16, and 2-token blocks with a partial last block): every unit against the oracle."""
    q, K, V, ch, out, idx = run_decode(w)
    for b in range(w.B):
        for g in range(w.Hkv):
            check_unit(w, q, K, V, ch, b, g, out, idx)


BUCKET_ADV_SHAPES = [(3000, 1000), (16384, 1024), (30000, 9000)]


def _bf16_adversarial_column(kind, n, rng):
    """bf16 bit patterns for one K column (the tokens' scores, up to a factor of 2)."""
    if kind == "one_digit":     # every score in one top digit: all are candidates
        return dsgen.f32_to_bf16_bits((1.0 + rng.random(n) * 0.2).astype(np.float32))
    if kind == "equal":         # one value: the k lowest ids are kept
        return np.full(n, dsgen.f32_to_bf16_bits(np.float32([-2.75]))[0], np.uint16)
    if kind == "zeros":         # +0.0 / -0.0 are one key; a few positives above them
        bits = np.where(rng.random(n) < 0.5, 0x8000, 0x0000).astype(np.uint16)
        bits[::97] = 0x3F80     # 1.0
        return bits
    if kind == "denormal":      # bf16 subnormals of both signs (exponent field 0)
        return (rng.integers(1, 128, size=n) | np.where(rng.random(n) < 0.5, 0x8000, 0)).astype(np.uint16)
    if kind == "boundaries":    # powers of two and their bf16 neighbours: values on the 11-bit digit edges
        sign = np.where(rng.random(n) < 0.3, 0x8000, 0).astype(np.int64)
        expo = rng.integers(124, 131, size=n).astype(np.int64)   # 2^-3 .. 2^3
        base = sign | (expo << 7)
        step = rng.integers(-1, 2, size=n)
        return np.clip(base + step, 0, 0xFFFF).astype(np.uint16)
    if kind == "ints":          # heavy exact ties everywhere, also at the k-th score
        return dsgen.f32_to_bf16_bits(rng.integers(-6, 7, size=n).astype(np.float32))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["one_digit", "equal", "zeros", "denormal", "boundaries", "ints"])
def test_decode_bucketed_adversarial_scores(kind):
    """The whole decode step of rows split over several workgroups (the score kernel's
    sorted tile lists, then the selection from them) on scores built to stress it: q is
    the first unit vector in every head and the label channels are 0..r-1, so a token's
    score is G times K[t, 0], which is set to a bf16 pattern of the given kind (all in one
    top digit, all equal, signed zeros, subnormals, values on digit edges, small
    integers).  Kept ids must equal the oracle's exactly (ties to the lower id), outputs
    within 2e-3."""
    Hq, Hkv, r = 4, 2, 16
    G = Hq // Hkv
    for T, k in BUCKET_ADV_SHAPES:
        rng = np.random.default_rng(zlib.crc32(f"{kind}{T}".encode()))
        w = Workload(f"badv_{kind}_{T}", "bf16", B=1, Hq=Hq, Hkv=Hkv, d=128, T=T, r=r, block=1, k_units=k,
                     seed_base=28000 + T)
        assert L.ds_decode_workspace_bytes(1, Hq, Hkv, 128, T, 1, k) > 0
        _say(f"{w.name} k={k}")
        _, K, V = dsgen.gen_cache(w)
        K = np.ascontiguousarray(K)
        for g in range(Hkv):
            K[0, g, :T, 0] = _bf16_adversarial_column(kind, T, rng)
        qf = np.zeros((1, Hq, 128), np.float32)
        qf[:, :, 0] = 1.0
        q = dsgen.f32_to_bf16_bits(qf)
        ch = np.tile(np.arange(r, dtype=np.int32), (Hkv, 1))
        qd, Kd, Vd = to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
        chd = torch.from_numpy(ch).cuda()
        label = L.ds_build_label_cache(Kd, chd)
        out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, T, k, 1)
        torch.cuda.synchronize()
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        for g in range(Hkv):
            qg, Kg, Vg = unit_inputs(w, q, K, V, 0, g)
            u = O.label_scores(qg, O.label_rows(Kg, ch[g]), ch[g])
            np.testing.assert_array_equal(u, G * Kg[:, 0])   # the construction above
            want = O.select_topk(u, k)
            np.testing.assert_array_equal(idx[0, g], want, err_msg=f"{w.name} g={g}")
            ref = O.attend(qg, Kg, Vg, want, O.default_scale(128))
            err = float(np.max(np.abs(out[0, g * G:(g + 1) * G] - ref)))
            assert err <= OUT_TOL["bf16"], (w.name, g, err)


def _bf16_patterns_with_digit(digit, lo, hi):
    """bf16 bit patterns (uint16) whose float value x lies in [lo, hi) and whose float32 sort key
    (sign flipped for x >= 0, every bit flipped for x < 0) has top 11 bits equal to digit."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    bits = pats << 16
    x = bits.view(np.float32)
    key = np.where(bits >> 31 == 0, bits | 0x80000000, ~bits & 0xFFFFFFFF).astype(np.uint32)
    ok = np.isfinite(x) & (x >= lo) & (x < hi) & ((key >> 21) == digit)
    return pats[ok].astype(np.uint16)


def test_bucket_top_digit_at_wavefront_seams():
    """Rows split over 8 workgroups (the sorted-list selection) whose k-th largest score sits in
    a digit between two wavefronts of the selection's digit scan (digit 1920 - 128 w, tested
    from the edge lanes' counts), with many exact ties at the threshold: q is one-hot on the
    first label channel, so a token's score is its K value there.  Seam w = 3 holds [2, 2.5),
    seam w = 11 holds (-2, -1.75].  The kept set must equal the oracle's exactly (ties go to
    the lowest token ids on both sides), and each output must match the oracle's attention."""
    B, H, T, r, k, d = 1, 8, 6000, 16, 512, 128
    rng = np.random.default_rng(20251)
    ch = np.stack([np.sort(rng.choice(d, r, replace=False)) for _ in range(H)]).astype(np.int32)
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    bf = lambda a: (f32(a).view(np.uint32) >> 16).astype(np.uint16)   # truncation to bf16 patterns
    K = bf(rng.normal(0.0, 0.1, (B, H, T, d)))
    V = bf(rng.normal(0.0, 1.0, (B, H, T, d)))
    q = np.zeros((B, H, d), dtype=np.uint16)
    one = bf([1.0])[0]
    seams = {3: ((2.5, 16.0), (2.0, 2.5), (-2.0, 2.0)), 11: ((-1.74, 4.0), (-2.0, -1.74), (-8.0, -2.0))}
    for g in range(H):
        w = 3 if g % 2 == 0 else 11
        (a_lo, a_hi), (s_lo, s_hi), (b_lo, b_hi) = seams[w]
        c0 = ch[g, 0]
        q[0, g, c0] = one
        inside = _bf16_patterns_with_digit(1920 - 128 * w, s_lo, s_hi)
        assert len(inside) >= 8, (w, len(inside))
        n_above, n_in = 300 + 7 * g, 400
        perm = rng.permutation(T)
        col = bf(rng.uniform(b_lo, b_hi, T))
        col[perm[:n_above]] = bf(rng.uniform(a_lo, a_hi, n_above))
        col[perm[n_above:n_above + n_in]] = rng.choice(inside, n_in)
        K[0, g, :, c0] = col
    qd, Kd, Vd = to_device(q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(Kd, chd)
    out, idx = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, T, k)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    for g in range(H):
        qg = dsgen.to_f64(q[0, g:g + 1], "bf16")
        Kf, Vf = dsgen.to_f64(K[0, g], "bf16"), dsgen.to_f64(V[0, g], "bf16")
        u = Kf[:, ch[g, 0]]
        theta = np.sort(u)[::-1][k - 1]
        key_digit = (np.float32(theta).view(np.uint32) ^ (0x80000000 if theta >= 0 else 0xFFFFFFFF)) >> 21
        assert key_digit in (1920 - 128 * 3, 1920 - 128 * 11), (g, theta, key_digit)
        assert np.sum(u == theta) > 1, (g, "the threshold should be tied")
        np.testing.assert_array_equal(idx[0, g], O.select_topk(u, k), err_msg=f"head {g}")
        check_row(qg, Kf, Vf, ch[g], k, 1, T, out[0, g:g + 1], idx[0, g], "bf16", f"head {g}")
