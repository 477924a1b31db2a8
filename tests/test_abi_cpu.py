"""Boundary tests that need no GPU: the library loads, exports every declared
symbol, rejects bad arguments before any HIP call, sizes workspaces, and its
CPU calibration agrees with the oracle.  Device pointers passed here are fake
(never dereferenced): every call below fails validation first."""
import ctypes
import math

import numpy as np
import pytest

import dsgen
import long_context_sparse_ds_amd as L
import oracle as O

FAKE = 4096          # 256-byte aligned fake device address
MISALIGNED = 4096 + 8


def test_library_exports_every_header_symbol():
    names = L.header_symbols()
    assert {"ds_calibrate_channels", "ds_build_label_cache", "ds_decode_sparse_attn",
            "ds_decode_workspace_bytes", "ds_last_error"} <= set(names)
    handle = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert L.ds_version().startswith("dsparse")


def _decode(**kw):
    a = dict(q=FAKE, K=FAKE, V=FAKE, label=FAKE, ch=FAKE, r=16, dt=L.DS_DTYPE_BF16, B=1, Hq=32, Hkv=32, d=128,
             T_cap=16384, T=16384, t_append=None, block=1, k=1024, scale=0.0, out=FAKE, idx=FAKE, ws=FAKE, ws_bytes=0,
             stream=None)
    a.update(kw)
    if a["t_append"] is None:
        a["t_append"] = a["T"]
    return L.lib().ds_decode_sparse_attn(a["q"], a["K"], a["V"], a["label"], a["ch"], a["r"], a["dt"], a["B"],
                                         a["Hq"], a["Hkv"], a["d"], a["T_cap"], a["T"], a["t_append"], a["block"],
                                         a["k"], a["scale"], a["out"], a["idx"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), L.DS_ERR_INVALID_ARGUMENT, "null"),
    (dict(ws=None), L.DS_ERR_INVALID_ARGUMENT, "null"),
    (dict(dt=7), L.DS_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(d=64), L.DS_ERR_UNSUPPORTED, "d = 64"),
    (dict(Hq=30, Hkv=8), L.DS_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(B=0), L.DS_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(r=0), L.DS_ERR_INVALID_ARGUMENT, "r <= d"),
    (dict(r=129), L.DS_ERR_INVALID_ARGUMENT, "r <= d"),
    (dict(T=0), L.DS_ERR_INVALID_ARGUMENT, "T <= T_cap"),
    (dict(T=20000), L.DS_ERR_INVALID_ARGUMENT, "T <= T_cap"),
    (dict(k=0), L.DS_ERR_INVALID_ARGUMENT, "k_units"),
    (dict(k=16385), L.DS_ERR_INVALID_ARGUMENT, "k_units"),
    (dict(t_append=16385), L.DS_ERR_INVALID_ARGUMENT, "t_append"),
    (dict(t_append=-1), L.DS_ERR_INVALID_ARGUMENT, "t_append"),
    (dict(block=3), L.DS_ERR_INVALID_ARGUMENT, "power of two"),
    (dict(block=128), L.DS_ERR_INVALID_ARGUMENT, "power of two"),
    (dict(block=64, k=257), L.DS_ERR_INVALID_ARGUMENT, "k_units"),
    (dict(K=MISALIGNED), L.DS_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(ws=FAKE + 16), L.DS_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(ws_bytes=100), L.DS_ERR_WORKSPACE_TOO_SMALL, "workspace"),
])
def test_decode_rejects_bad_arguments(kw, status, needle):
    assert _decode(**kw) == status
    assert needle in L.ds_last_error()


def test_workspace_size_is_consistent_and_checked():
    n = L.ds_decode_workspace_bytes(1, 32, 32, 128, 16384, 1, 1024)
    assert n % 256 == 0 and n >= 32 * 16384 * 4
    assert _decode(ws_bytes=n - 1) == L.DS_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(L.DsError):
        L.ds_decode_workspace_bytes(1, 32, 32, 128, 16384, 1, 0)
    # sized independently of dtype and r, grows with the batch
    assert L.ds_decode_workspace_bytes(16, 32, 32, 128, 32768, 1, 2048) > n


def test_other_entry_points_validate_first():
    lib = L.lib()
    assert lib.ds_build_label_cache(FAKE, L.DS_DTYPE_BF16, 1, 1, 100, 128, FAKE, 16, 50, 40, FAKE, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "t_begin" in L.ds_last_error()
    assert lib.ds_build_label_cache(FAKE, L.DS_DTYPE_BF16, 1, 1, 100, 96, FAKE, 16, 0, 1, FAKE, None) \
        == L.DS_ERR_UNSUPPORTED
    assert lib.ds_build_label_cache(FAKE, L.DS_DTYPE_BF16, 1, 1, 1 << 31, 128, FAKE, 16, 0, 1, FAKE, None) \
        == L.DS_ERR_UNSUPPORTED
    assert "T_cap" in L.ds_last_error()
    assert lib.ds_build_label_cache(FAKE, L.DS_DTYPE_BF16, 300, 300, 100, 128, FAKE, 16, 0, 1, FAKE, None) \
        == L.DS_ERR_UNSUPPORTED
    assert lib.ds_topk_select(FAKE, 4, 100, 100, 101, FAKE, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_topk_select(FAKE, 4, 100, 50, 10, FAKE, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_label_scores(FAKE, FAKE, FAKE, 16, L.DS_DTYPE_F32, 1, 1, 1, 128, 1024, 1024, 1, FAKE, 1022,
                               None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_sparse_attn_from_indices(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 100, 100, 1, 10, FAKE,
                                           0.0, FAKE, FAKE, 10, None) == L.DS_ERR_WORKSPACE_TOO_SMALL
    assert lib.ds_select_attention(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 100, 100, 1, 10, FAKE, 128, 0.0,
                                   FAKE, FAKE, FAKE, 10, None) == L.DS_ERR_WORKSPACE_TOO_SMALL
    assert lib.ds_select_attention(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 100, 100, 1, 10, FAKE, 98, 0.0,
                                   FAKE, FAKE, FAKE, 1 << 20, None) == L.DS_ERR_INVALID_ARGUMENT
    # ragged decode: seq_lens, n_append and the fused-path limit are checked on the host
    ws = L.ds_decode_workspace_bytes(2, 4, 4, 128, 1000, 1, 50)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 2, 4, 4, 128, 1000, 1000)
    assert lib.ds_decode_sparse_attn_ragged(*args, None, 1, 1, 50, 0.0, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "seq_lens" in L.ds_last_error()
    assert lib.ds_decode_sparse_attn_ragged(*args, FAKE, -1, 1, 50, 0.0, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "n_append" in L.ds_last_error()
    big = L.ds_decode_workspace_bytes(1, 1, 1, 128, 40000, 1, 50)
    assert lib.ds_decode_sparse_attn_ragged(FAKE, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 1, 1, 1, 128, 40000,
                                            40000, FAKE, 1, 1, 50, 0.0, FAKE, FAKE, FAKE, big, None) \
        == L.DS_ERR_UNSUPPORTED
    assert lib.ds_decode_sparse_attn_ragged(*args, FAKE, 1, 1, 1001, 0.0, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    # the ragged phases validate the same way
    sargs = (FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 2, 4, 4, 128, 1000, 1000)
    assert lib.ds_decode_score_ragged(*sargs, None, 1, 1, 50, FAKE, ws, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_score_ragged(*sargs, FAKE, -2, 1, 50, FAKE, ws, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_score_ragged(*sargs, FAKE, 1, 1, 50, FAKE, 10, None) == L.DS_ERR_WORKSPACE_TOO_SMALL
    aargs = (FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 2, 4, 4, 128, 1000, 1000)
    assert lib.ds_decode_select_attend_ragged(*aargs, None, 1, 50, 0.0, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_select_attend_ragged(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 1, 1, 128, 40000, 40000, FAKE, 1,
                                              50, 0.0, FAKE, FAKE, FAKE, big, None) == L.DS_ERR_UNSUPPORTED
    assert lib.ds_decode_select_attend_ragged(*aargs, FAKE, 1, 50, 0.0, None, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    # threshold rule: counts, tau, the group size and the fused-path limit are checked on the host
    ws8 = L.ds_decode_workspace_bytes(2, 8, 2, 128, 1000, 1, 50)
    targs = (FAKE, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 2, 8, 2, 128, 1000, 1000, 999, 1, 50)
    assert lib.ds_decode_sparse_attn_threshold(*targs, 1.0, 0.0, FAKE, FAKE, None, FAKE, ws8, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "counts" in L.ds_last_error()
    assert lib.ds_decode_sparse_attn_threshold(*targs, float("nan"), 0.0, FAKE, FAKE, FAKE, FAKE, ws8, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "NaN" in L.ds_last_error()
    ws16 = L.ds_decode_workspace_bytes(2, 32, 2, 128, 1000, 1, 50)
    assert lib.ds_decode_sparse_attn_threshold(FAKE, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 2, 32, 2, 128, 1000,
                                               1000, 999, 1, 50, 1.0, 0.0, FAKE, FAKE, FAKE, FAKE, ws16, None) \
        == L.DS_ERR_UNSUPPORTED
    ws_g8 = L.ds_decode_workspace_bytes(2, 16, 2, 128, 1000, 1, 50)
    assert lib.ds_decode_sparse_attn_threshold(FAKE, FAKE, FAKE, FAKE, FAKE, 65, L.DS_DTYPE_BF16, 2, 16, 2, 128,
                                               1000, 1000, 999, 1, 50, 1.0, 0.0, FAKE, FAKE, FAKE, FAKE, ws_g8, None) \
        == L.DS_ERR_UNSUPPORTED
    assert "512" in L.ds_last_error()
    big = L.ds_decode_workspace_bytes(1, 1, 1, 128, 40000, 1, 50)
    assert lib.ds_decode_sparse_attn_threshold(FAKE, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 1, 1, 1, 128,
                                               40000, 40000, 40000, 1, 50, 1.0, 0.0, FAKE, FAKE, FAKE, FAKE, big,
                                               None) == L.DS_ERR_UNSUPPORTED
    assert lib.ds_decode_score_threshold(FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 2, 32, 2, 128, 1000, 1000,
                                         1000, 1, 50, FAKE, ws16, None) == L.DS_ERR_UNSUPPORTED
    assert lib.ds_decode_select_attend_threshold(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 2, 8, 2, 128, 1000, 1000, 1, 50,
                                                 1.0, 0.0, FAKE, FAKE, None, FAKE, ws8, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_label_scores_positive(FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 1, 16, 1, 128, 1024, 1024, 1, FAKE,
                                        1024, None) == L.DS_ERR_UNSUPPORTED
    assert lib.ds_label_scores_positive(FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, 1, 8, 1, 128, 1024, 1024, 1, FAKE,
                                        1022, None) == L.DS_ERR_INVALID_ARGUMENT
    # offloaded K/V: null pointers fail first; a pointer HIP does not know is rejected before any launch
    oargs = (16, L.DS_DTYPE_BF16, 2, 4, 4, 128, 1000, 1000, 999, 1, 50, 0.0)
    assert lib.ds_decode_sparse_attn_offload(FAKE, None, FAKE, FAKE, FAKE, *oargs, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_sparse_attn_offload(FAKE, FAKE, FAKE, FAKE, FAKE, *oargs, FAKE, FAKE, FAKE, ws, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert "K" in L.ds_last_error()
    # hierarchical span search: capacity, workspace and argument checks on the host
    assert lib.ds_hip_token_capacity(1 << 20, 64, 64) == 64 * 64
    assert lib.ds_hip_token_capacity(1000, 20, 64) == 1000      # no round: every token
    assert lib.ds_hip_token_capacity(10, 3, 2) == 6
    assert lib.ds_hip_token_capacity(10, 0, 2) == 0 and lib.ds_hip_token_capacity(10, 11, 2) == 0
    assert lib.ds_hip_workspace_bytes(1, 4, 4, 128, 1000, 2000, 8) == 0
    assert lib.ds_hip_workspace_bytes(1, 4, 4, 96, 1000, 20, 8) == 0
    hws = lib.ds_hip_workspace_bytes(1, 4, 4, 128, 1000, 20, 8)
    assert hws > 0
    hargs = (FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 1000, 1000)
    assert lib.ds_decode_hip_attn(*hargs, 20, 8, 0.0, FAKE, None, FAKE, hws, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_hip_attn(*hargs, 1025, 8, 0.0, FAKE, FAKE, FAKE, hws, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_hip_attn(*hargs, 20, 0, 0.0, FAKE, FAKE, FAKE, hws, None) == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_decode_hip_attn(*hargs, 20, 8, 0.0, FAKE, FAKE, FAKE, hws - 1, None) \
        == L.DS_ERR_WORKSPACE_TOO_SMALL
    assert lib.ds_decode_hip_attn(FAKE, FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 64, 1000, 1000, 20, 8, 0.0, FAKE, FAKE,
                                  FAKE, hws, None) == L.DS_ERR_UNSUPPORTED
    assert lib.ds_hip_search(FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 1000, 1000, 20, 8, FAKE, None, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_hip_search(FAKE, FAKE, L.DS_DTYPE_BF16, 1, 4, 4, 128, 1000, 1001, 20, 8, FAKE, FAKE, None) \
        == L.DS_ERR_INVALID_ARGUMENT
    # a valid call afterwards clears the message
    L.ds_decode_workspace_bytes(1, 1, 1, 128, 10, 1, 1)
    assert L.ds_last_error() == ""


def test_calibrate_rejects_bad_arguments():
    lib = L.lib()
    q = np.zeros((4, 2, 8), np.float32)
    k = np.zeros((1, 4, 8), np.float32)
    out = np.full((1, 3), -7, np.int32)
    assert lib.ds_calibrate_channels(None, 4, k.ctypes.data, 4, 2, 1, 8, 3, out.ctypes.data) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_calibrate_channels(q.ctypes.data, 4, k.ctypes.data, 4, 3, 2, 8, 3, out.ctypes.data) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert lib.ds_calibrate_channels(q.ctypes.data, 4, k.ctypes.data, 4, 2, 1, 8, 9, out.ctypes.data) \
        == L.DS_ERR_INVALID_ARGUMENT
    assert list(out[0]) == [-7, -7, -7]   # untouched on failure


@pytest.mark.parametrize("name", dsgen.WORKLOAD_ORDER)
def test_calibrate_matches_oracle_on_workloads(name):
    w = dsgen.get(name)
    qc, kc = dsgen.gen_calib(w)
    np.testing.assert_array_equal(L.ds_calibrate_channels(qc, kc, w.r), O.calibrate_channels(qc, kc, w.Hkv, w.r))


def test_calibrate_matches_oracle_on_ties_and_small_shapes():
    rng = np.random.default_rng(11)
    for (n_q, Hq, Hkv, d, n_k) in [(3, 4, 2, 8, 5), (7, 6, 3, 16, 2), (1, 1, 1, 128, 1)]:
        qc = rng.integers(-2, 3, size=(n_q, Hq, d)).astype(np.float32)   # integer data: exact ties
        kc = rng.integers(-2, 3, size=(Hkv, n_k, d)).astype(np.float32)
        for r in sorted({1, d // 3 + 1, d}):
            np.testing.assert_array_equal(L.ds_calibrate_channels(qc, kc, r), O.calibrate_channels(qc, kc, Hkv, r))


def _noalloc(B=1, Hq=32, Hkv=32, T=16384, k=1024, block=1, q=FAKE):
    return L.lib().ds_decode_sparse_attn_noalloc(q, FAKE, FAKE, FAKE, FAKE, 16, L.DS_DTYPE_BF16, B, Hq, Hkv, 128, T, T,
                                                 T, block, k, 0.0, FAKE, FAKE, None)


def test_noalloc_scratch_size_matches_header():
    import re
    with open(L._binding.HEADER) as f:
        m = re.search(r"#define\s+DS_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.DS_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_shapes_beyond_its_scratch_before_any_hip_call():
    # 512 rows of 32,768 scores need 64 MiB of workspace: more than the static scratch.
    assert L.ds_decode_workspace_bytes(16, 32, 32, 128, 32768, 1, 2048) > L.DS_NOALLOC_SCRATCH_BYTES
    assert _noalloc(B=16, T=32768, k=2048) == L.DS_ERR_WORKSPACE_TOO_SMALL
    assert "static device scratch" in L.ds_last_error()
    # argument checks come first, as for the workspace form
    assert _noalloc(q=None) == L.DS_ERR_INVALID_ARGUMENT
    assert _noalloc(k=0) == L.DS_ERR_INVALID_ARGUMENT
    # the headline shape fits
    assert L.ds_decode_workspace_bytes(1, 32, 32, 128, 16384, 1, 1024) <= L.DS_NOALLOC_SCRATCH_BYTES
