"""GPU parity of the offloaded-KV decode step (K and V in pinned host memory).

ds_decode_sparse_attn_offload runs the kernels of ds_decode_sparse_attn with K and V
read across the host link, so its indices and outputs must equal, bit for bit, those
of the same call on device-resident K and V; the oracle checks a sample of units too.
Covered: the fused path (token-level and 64-token blocks, GQA, T_cap > T, appended
label rows read from host K), its one-pass form (256 one-split rows), the separate path
for rows of more than 32,768 units, the full-size offload workload, and the rejection
of device-resident K/V.
"""
import ctypes

import numpy as np
import pytest
import torch

import dsgen
import long_context_sparse_ds_amd as L
import oracle as O
from dsgen import Workload
from _helpers import check_unit, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L.lib()   # raises if the HIP library is missing


def _say(msg):
    print(f"[case] {msg}", flush=True)


def bits(t):
    """Raw bit patterns, so NaN padding rows compare equal."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def to_pinned(arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
        else torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.pin_memory()


OFFLOAD_CASES = [
    Workload("off_mha", "bf16", B=2, Hq=4, Hkv=4, d=128, T=3000, r=16, block=1, k_units=190, seed_base=41000,
             T_cap=3100),
    Workload("off_gqa4_blk64", "bf16", B=1, Hq=8, Hkv=2, d=128, T=64 * 70 + 13, r=16, block=64, k_units=20,
             seed_base=41100),
    Workload("off_f32", "f32", B=1, Hq=2, Hkv=1, d=128, T=1500, r=16, block=1, k_units=77, seed_base=41200,
             fixed_outliers=True),
    Workload("off_long_rows", "bf16", B=1, Hq=2, Hkv=2, d=128, T=40000, r=16, block=1, k_units=600,
             seed_base=41300),
    # 256 rows of one split each: the one-pass kernel, reading K (for the rebuilt rows) and V from the host
    Workload("off_one_pass", "bf16", B=64, Hq=4, Hkv=4, d=128, T=1500, r=8, block=1, k_units=60, seed_base=41400),
]


@pytest.mark.parametrize("w", OFFLOAD_CASES, ids=[w.name for w in OFFLOAD_CASES])
def test_offload_matches_device_resident(w):
    _say(f"{w.name} T={w.T} block={w.block} k={w.k_units}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    chd = torch.from_numpy(ch).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    Kh, Vh = to_pinned(K, w.dtype), to_pinned(V, w.dtype)
    lab_dev = L.ds_build_label_cache(Kd, chd)
    lab_off = lab_dev.clone()
    raw = lab_off.view(torch.int16) if w.dtype == "bf16" else lab_off.view(torch.int32)
    raw[:, :, w.T - 3:w.T].fill_(0x3F00)   # the append must rebuild these rows from host K
    o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, lab_dev, chd, w.T, w.k_units, w.block, t_append=w.T - 3)
    o2, i2 = L.ds_decode_sparse_attn_offload(qd, Kh, Vh, lab_off, chd, w.T, w.k_units, w.block, t_append=w.T - 3)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2), "kept sets differ between host and device K/V"
    assert torch.equal(o1, o2), "outputs differ between host and device K/V"
    assert torch.equal(bits(lab_dev), bits(lab_off)), "label rows appended from host K differ"
    out, idx = o2.cpu().numpy(), i2.cpu().numpy()
    for b, g in {(0, 0), (w.B - 1, w.Hkv - 1)}:
        check_unit(w, q, K, V, ch, b, g, out, idx)


def test_offload_phases_with_host_kv_match_one_call():
    """The two phases run on their own with host K/V (how the benchmark times them) give
    the one call's results."""
    w = OFFLOAD_CASES[0]
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd = to_device(q, w.dtype), to_device(K, w.dtype)
    Kh, Vh = to_pinned(K, w.dtype), to_pinned(V, w.dtype)
    lab1 = L.ds_build_label_cache(Kd, chd)
    lab2 = lab1.clone()
    o1, i1 = L.ds_decode_sparse_attn_offload(qd, Kh, Vh, lab1, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
    ws = L.ds_decode_score(qd, Kh, lab2, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
    o2, i2 = L.ds_decode_select_attend(qd, Kh, Vh, w.T, w.k_units, ws, w.block)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(bits(lab1), bits(lab2))


def test_offload_rejects_device_kv():
    """Device-resident K or V passed to the offload call is an argument error, raised
    before any launch."""
    w = OFFLOAD_CASES[0]
    q, K, V = dsgen.gen_cache(w)
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    Vh = to_pinned(V, w.dtype)
    ch = torch.zeros((w.Hkv, w.r), dtype=torch.int32, device="cuda")
    label = torch.zeros((w.B, w.Hkv, w.cap, w.r), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda")
    ws = L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.lib().ds_decode_sparse_attn_offload(p(qd), p(Kd), p(Vh), p(label), p(ch), w.r, L.DS_DTYPE_BF16, w.B,
                                               w.Hq, w.Hkv, w.d, w.cap, w.T, w.T, w.block, w.k_units, 0.0, p(out),
                                               p(idx), p(ws), ws.numel(), None)
    assert st == L.DS_ERR_INVALID_ARGUMENT and "pinned host" in L.ds_last_error()
    with pytest.raises(ValueError):
        L.ds_decode_sparse_attn_offload(qd, Kd, Vd, label, ch, w.T, w.k_units, w.block)


@pytest.mark.parametrize("name", dsgen.OFFLOAD_ORDER)
def test_offload_full_size_workload(name):
    """The offload workload at full size, called as the benchmark calls it: equal to the
    device-resident call bit for bit, and the oracle checks two units."""
    w = dsgen.get(name)
    _say(f"{name}: B={w.B} H={w.Hq}/{w.Hkv} T={w.T} block={w.block} k={w.k_units}")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    chd = torch.from_numpy(ch).cuda()
    qd = to_device(q, w.dtype)
    Kh, Vh = to_pinned(K, w.dtype), to_pinned(V, w.dtype)
    Kd = Kh.cuda()
    lab = L.ds_build_label_cache(Kd, chd)
    lab2 = lab.clone()
    o2, i2 = L.ds_decode_sparse_attn_offload(qd, Kh, Vh, lab2, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
    torch.cuda.synchronize()
    Vd = Vh.cuda()
    o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, lab, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)
    out, idx = o2.cpu().numpy(), i2.cpu().numpy()
    for b, g in ((0, 0), (w.B - 1, w.Hkv - 1)):
        swaps, err = check_unit(w, q, K, V, ch, b, g, out, idx)
        _say(f"{name} unit ({b},{g}): tie swaps {swaps}, max-abs err {err:.3g}")
    del q, K, V, Kd, Vd
    torch.cuda.empty_cache()
