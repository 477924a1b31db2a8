"""The no-allocation decode entry point (ds_decode_sparse_attn_noalloc) against the workspace
form (ds_decode_sparse_attn), through the C ABI.

Both run the same kernels, the first with the library's static device scratch as its
workspace, so indices and outputs must be identical bit for bit.  Two calls in a row share
the scratch, the second with a smaller shape (fewer rows, splits and tiles), so that state
left by the first call (merge tickets, split states, scores) cannot leak into the second.
A third call repeats the first shape after the smaller one.  The oracle also checks every
row of each call (index rule and output tolerance).
"""
import numpy as np
import pytest
import torch

import dsgen
import long_context_sparse_ds_amd as L
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


BIG = dsgen.get(dsgen.HEADLINE)
SMALL = Workload("noalloc_small", "bf16", B=2, Hq=8, Hkv=4, d=128, T=3000, r=16, block=1, k_units=150,
                 seed_base=61000, T_cap=3100)


def _setup(w):
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    dev = [to_device(a, w.dtype) for a in (q, K, V)]
    chd = torch.from_numpy(ch).cuda()
    label = L.ds_build_label_cache(dev[1], chd)
    return (q, K, V, ch), (*dev, chd, label)


def test_noalloc_matches_workspace_form_on_consecutive_calls():
    host, dev = {}, {}
    for w in (BIG, SMALL):
        host[w.name], dev[w.name] = _setup(w)
    torch.cuda.synchronize()
    for w in (BIG, SMALL, BIG):
        _say(f"noalloc {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} k={w.k_units} "
             f"workspace {L.ds_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units)} bytes")
        qd, Kd, Vd, chd, label = dev[w.name]
        o1, i1 = L.ds_decode_sparse_attn(qd, Kd, Vd, label, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
        o2, i2 = L.ds_decode_sparse_attn_noalloc(qd, Kd, Vd, label, chd, w.T, w.k_units, w.block, t_append=w.T - 1)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), f"{w.name}: indices differ in {(i1 != i2).sum().item()} slots"
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), f"{w.name}: outputs differ"
        q, K, V, ch = host[w.name]
        out, idx = o2.cpu().numpy(), i2.cpu().numpy()
        for b in range(w.B):
            for g in range(w.Hkv):
                check_unit(w, q, K, V, ch, b, g, out, idx)
        _say(f"noalloc {w.name}: identical to the workspace form; every row matches the oracle")
