"""Every decode path captured in a HIP graph reproduces its eager result bit for bit.

The benchmark times graph-replayed steps, and the split merge relies on tickets that
the kernels reset themselves, so each path (unequal lengths, the threshold rule, the
two-stage selection of long rows, the span search, offloaded K/V, the one-pass kernel) is
captured once and replayed several times, with eager calls and synchronisation in between,
each replay checked against the eager call on the same inputs.
"""
import numpy as np
import pytest
import torch

import dsgen
import long_context_sparse_ds_amd as L
from dsgen import Workload
from _helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L.lib()   # raises if the HIP library is missing


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _inputs(w):
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    chd = torch.from_numpy(L.ds_calibrate_channels(qc, kc, w.r)).cuda()
    qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    return qd, Kd, Vd, chd, L.ds_build_label_cache(Kd, chd)


def _path(name):
    """(call(outputs) -> None writing into preallocated outputs, outputs) for one path."""
    if name == "ragged":
        w = Workload("g_ragged", "bf16", B=3, Hq=8, Hkv=2, d=128, T=9000, r=8, block=1, k_units=256, seed_base=61000)
        qd, Kd, Vd, chd, lab = _inputs(w)
        seq = torch.tensor([9000, 2049, 100], dtype=torch.int32, device="cuda")
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    idx=torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda"),
                    ws=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units))
        return (lambda o: L.ds_decode_sparse_attn_ragged(qd, Kd, Vd, lab, chd, seq, w.T, w.k_units, w.block,
                                                         n_append=1, out=o["out"], indices=o["idx"],
                                                         workspace=o["ws"])), outs
    if name == "threshold":
        w = Workload("g_thr", "bf16", B=2, Hq=8, Hkv=2, d=128, T=64 * 70 + 13, r=16, block=64, k_units=20,
                     seed_base=61100)
        qd, Kd, Vd, chd, lab = _inputs(w)
        s = L.ds_label_scores_positive(qd, lab, chd, w.T, w.block)
        tau = float(torch.quantile(s[0, 0, :-(-w.T // 64)], 0.7))
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    idx=torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda"),
                    cnt=torch.empty((w.B, w.Hkv), dtype=torch.int32, device="cuda"),
                    ws=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units))
        return (lambda o: L.ds_decode_sparse_attn_threshold(qd, Kd, Vd, lab, chd, w.T, w.k_units, tau, w.block,
                                                            out=o["out"], indices=o["idx"], counts=o["cnt"],
                                                            workspace=o["ws"], t_append=w.T - 1)), outs
    if name == "long_rows":
        w = Workload("g_long", "bf16", B=1, Hq=8, Hkv=2, d=128, T=70000, r=8, block=1, k_units=2000, seed_base=61200)
        qd, Kd, Vd, chd, lab = _inputs(w)
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    idx=torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda"),
                    ws=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units))
        return (lambda o: L.ds_decode_sparse_attn(qd, Kd, Vd, lab, chd, w.T, w.k_units, w.block, out=o["out"],
                                                  indices=o["idx"], workspace=o["ws"], t_append=w.T - 1)), outs
    if name == "span_search":
        w = Workload("g_hip", "bf16", B=2, Hq=16, Hkv=4, d=128, T=20000, r=16, block=16, k_units=64,
                     seed_base=61300)
        q, K, V = dsgen.gen_cache(w)
        qd, Kd, Vd = to_device(q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
        n = L.lib().ds_hip_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.T, w.k_units, w.block)
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    spans=torch.empty((w.B, w.Hkv, w.k_units, 2), dtype=torch.int32, device="cuda"),
                    ws=torch.empty(n, dtype=torch.uint8, device="cuda"))
        return (lambda o: L.ds_decode_hip_attn(qd, Kd, Vd, w.T, w.k_units, w.block, out=o["out"],
                                               spans=o["spans"], workspace=o["ws"])), outs
    if name == "offload":
        w = Workload("g_off", "bf16", B=2, Hq=4, Hkv=4, d=128, T=3000, r=16, block=1, k_units=190, seed_base=61400)
        qd, Kd, Vd, chd, lab = _inputs(w)
        Kh, Vh = Kd.cpu().pin_memory(), Vd.cpu().pin_memory()
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    idx=torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda"),
                    ws=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units))
        return (lambda o: L.ds_decode_sparse_attn_offload(qd, Kh, Vh, lab, chd, w.T, w.k_units, w.block,
                                                          out=o["out"], indices=o["idx"], workspace=o["ws"],
                                                          t_append=w.T - 1)), outs
    if name == "one_pass":
        w = Workload("g_one", "bf16", B=64, Hq=4, Hkv=4, d=128, T=2500, r=16, block=1, k_units=100, seed_base=61500)
        assert L.ds_decode_is_one_pass(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units, w.r)
        qd, Kd, Vd, chd, lab = _inputs(w)
        outs = dict(out=torch.empty((w.B, w.Hq, w.d), device="cuda"),
                    idx=torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device="cuda"),
                    ws=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units))
        return (lambda o: L.ds_decode_sparse_attn(qd, Kd, Vd, lab, chd, w.T, w.k_units, w.block, out=o["out"],
                                                  indices=o["idx"], workspace=o["ws"], t_append=w.T - 1)), outs
    raise ValueError(name)


PATHS = ["ragged", "threshold", "long_rows", "span_search", "offload", "one_pass"]


@pytest.mark.parametrize("name", PATHS)
def test_graph_replay_matches_eager(name):
    call, outs = _path(name)
    result_keys = [k for k in outs if k != "ws"]
    call(outs)
    torch.cuda.synchronize()
    ref = {k: outs[k].clone() for k in result_keys}
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(outs)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call(outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in result_keys:
            outs[k].zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in result_keys:
            assert torch.equal(_bits(outs[k]), _bits(ref[k])), (name, k, rep)
        call(outs)   # eager work between replays
        torch.cuda.synchronize()
        for k in result_keys:
            assert torch.equal(_bits(outs[k]), _bits(ref[k])), (name, k, "eager", rep)
