"""ctypes binding of libdsparse.so.

Argument marshalling only: every step runs in the library's HIP kernels (or,
for the offline calibration, its C++ code).  torch supplies device memory and
the current HIP stream.  If the library is missing, every call raises: there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# DSPARSE_LIB selects another build of the same library (the host-sanitizer build of build.py).
LIB_PATH = os.environ.get("DSPARSE_LIB") or os.path.join(PKG, "libdsparse.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ds.h")

DS_OK = 0
DS_ERR_INVALID_ARGUMENT = 1
DS_ERR_UNSUPPORTED = 2
DS_ERR_WORKSPACE_TOO_SMALL = 3
DS_ERR_HIP = 4
DS_DTYPE_F32 = 0
DS_DTYPE_BF16 = 1

_c_i32, _c_i64, _c_size, _c_vp, _c_f32 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_float)

_SIGNATURES = {
    "ds_last_error": (ctypes.c_char_p, []),
    "ds_version": (ctypes.c_char_p, []),
    "ds_calibrate_channels": (_c_i32, [_c_vp, _c_i64, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp]),
    "ds_build_label_cache": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_vp, _c_i32, _c_i64, _c_i64,
                                      _c_vp, _c_vp]),
    "ds_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i64]),
    "ds_decode_is_one_pass": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i64, _c_i32, _c_i32]),
    "ds_decode_sparse_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                       _c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64, _c_f32, _c_vp, _c_vp, _c_vp,
                                       _c_size, _c_vp]),
    "ds_decode_sparse_attn_noalloc": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                               _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64, _c_f32, _c_vp,
                                               _c_vp, _c_vp]),
    "ds_decode_sparse_attn_ragged": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                              _c_i32, _c_i32, _c_i64, _c_i64, _c_vp, _c_i32, _c_i32, _c_i64, _c_f32,
                                              _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_decode_score": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                 _c_i64, _c_i64, _c_i32, _c_i64, _c_vp, _c_size, _c_vp]),
    "ds_decode_select_attend": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64,
                                         _c_i32, _c_i64, _c_f32, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_decode_score_ragged": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_i64, _c_i64, _c_vp, _c_i32, _c_i32, _c_i64, _c_vp, _c_size, _c_vp]),
    "ds_decode_select_attend_ragged": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                                _c_i64, _c_vp, _c_i32, _c_i64, _c_f32, _c_vp, _c_vp, _c_vp, _c_size,
                                                _c_vp]),
    "ds_decode_sparse_attn_threshold": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64, _c_f32,
                                                 _c_f32, _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_decode_score_threshold": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64, _c_vp, _c_size, _c_vp]),
    "ds_decode_select_attend_threshold": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                   _c_i64, _c_i64, _c_i32, _c_i64, _c_f32, _c_f32, _c_vp, _c_vp,
                                                   _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_label_scores_positive": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                          _c_i64, _c_i32, _c_vp, _c_i64, _c_vp]),
    "ds_decode_sparse_attn_offload": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                               _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64, _c_f32, _c_vp,
                                               _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_decode_hip_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64,
                                    _c_i32, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_hip_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32]),
    "ds_hip_token_capacity": (_c_i64, [_c_i64, _c_i64, _c_i64]),
    "ds_hip_search": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32,
                               _c_vp, _c_vp, _c_vp]),
    "ds_select_attention": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64,
                                     _c_i32, _c_i64, _c_vp, _c_i64, _c_f32, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ds_label_scores": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64,
                                 _c_i32, _c_vp, _c_i64, _c_vp]),
    "ds_topk_select": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "ds_sparse_attn_from_indices": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                             _c_i64, _c_i32, _c_i64, _c_vp, _c_f32, _c_vp, _c_vp, _c_size, _c_vp]),
}

_lib = None


class DsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ds status {status}: {message}")
        self.status = status


def header_symbols() -> list[str]:
    """Every function the C header declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(ds_\w+)\s*\(", text, flags=re.M)))


def lib() -> ctypes.CDLL:
    """Load libdsparse.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_ds_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def ds_last_error() -> str:
    return lib().ds_last_error().decode()


def ds_version() -> str:
    return lib().ds_version().decode()


def _check(status: int):
    if status != DS_OK:
        raise DsError(status, ds_last_error())


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DS_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DS_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _host(t, name):
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _kv(t, name):
    """K or V: a device tensor, or a pinned host tensor (offloaded cache)."""
    return _dev(t, name) if t.is_cuda else _host(t, name)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- entry points

def ds_calibrate_channels(q_cal: np.ndarray, k_cal: np.ndarray, r: int) -> np.ndarray:
    """Offline calibration on the CPU.  q_cal [n_q, Hq, d], k_cal [Hkv, n_k, d] -> int32 [Hkv, r]."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    n_q, Hq, d = q.shape
    Hkv, n_k, d2 = k.shape
    if d2 != d:
        raise ValueError("q_cal and k_cal disagree on d")
    out = np.empty((Hkv, r), dtype=np.int32)
    _check(lib().ds_calibrate_channels(q.ctypes.data, n_q, k.ctypes.data, n_k, Hq, Hkv, d, r, out.ctypes.data))
    return out


def ds_build_label_cache(K, channels, t_begin: int = 0, t_end: int | None = None, label=None, stream=None):
    """Pack label[b, g, t, :] = K[b, g, t, channels[g]] for t in [t_begin, t_end).  Returns label."""
    torch = _torch()
    B, Hkv, T_cap, d = K.shape
    r = channels.shape[1]
    if t_end is None:
        t_end = T_cap
    if label is None:
        label = torch.empty((B, Hkv, T_cap, r), dtype=K.dtype, device=K.device)
    if channels.dtype != torch.int32 or label.dtype != K.dtype or tuple(label.shape) != (B, Hkv, T_cap, r):
        raise ValueError("channels must be int32 [Hkv, r]; label must match K's dtype and be [B, Hkv, T_cap, r]")
    _check(lib().ds_build_label_cache(_dev(K, "K"), _dtype_code(K), B, Hkv, T_cap, d, _dev(channels, "channels"), r,
                                      t_begin, t_end, _dev(label, "label"), _stream(stream)))
    return label


def ds_decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, T: int, block: int, k_units: int) -> int:
    n = lib().ds_decode_workspace_bytes(B, Hq, Hkv, d, T, block, k_units)
    if n == 0:
        raise DsError(DS_ERR_INVALID_ARGUMENT, ds_last_error())
    return n


def ds_decode_is_one_pass(B: int, Hq: int, Hkv: int, d: int, T: int, block: int, k_units: int, r: int,
                          dtype: str = "bf16") -> bool:
    """Whether the one-call decode step runs this shape as a single kernel (host only)."""
    v = lib().ds_decode_is_one_pass(B, Hq, Hkv, d, T, block, k_units, r,
                                    DS_DTYPE_BF16 if dtype == "bf16" else DS_DTYPE_F32)
    if v < 0:
        raise DsError(DS_ERR_INVALID_ARGUMENT, ds_last_error())
    return bool(v)


def alloc_workspace(B, Hq, Hkv, d, T, block, k_units, device="cuda"):
    torch = _torch()
    return torch.empty(ds_decode_workspace_bytes(B, Hq, Hkv, d, T, block, k_units), dtype=torch.uint8, device=device)


def ds_decode_sparse_attn(q, K, V, label, channels, T: int, k_units: int, block: int = 1, scale: float = 0.0,
                          out=None, indices=None, workspace=None, stream=None, t_append: int | None = None):
    """One Double Sparsity decode step.  Returns (out fp32 [B, Hq, d], indices int32 [B, Hkv, k_units]).

    t_append < T first rebuilds label rows [t_append, T) from K inside the call."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    dt = _dtype_code(q)
    if K.dtype != q.dtype or V.dtype != q.dtype or label.dtype != q.dtype:
        raise ValueError("q, K, V and label must share one dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_units, q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_sparse_attn(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dev(label, "label"),
                                       _dev(channels, "channels"), r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block,
                                       k_units, scale, _dev(out, "out"), _dev(indices, "indices"),
                                       _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))
    return out, indices


DS_NOALLOC_SCRATCH_BYTES = 32 << 20


def ds_decode_sparse_attn_noalloc(q, K, V, label, channels, T: int, k_units: int, block: int = 1, scale: float = 0.0,
                                  out=None, indices=None, stream=None, t_append: int | None = None):
    """ds_decode_sparse_attn with the library's static device scratch as its workspace (the call
    allocates nothing on the device; pass out and indices to allocate nothing here either).
    Returns (out fp32 [B, Hq, d], indices int32 [B, Hkv, k_units])."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    dt = _dtype_code(q)
    if K.dtype != q.dtype or V.dtype != q.dtype or label.dtype != q.dtype:
        raise ValueError("q, K, V and label must share one dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_sparse_attn_noalloc(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dev(label, "label"),
                                               _dev(channels, "channels"), r, dt, B, Hq, Hkv, d, T_cap, T, t_append,
                                               block, k_units, scale, _dev(out, "out"), _dev(indices, "indices"),
                                               _stream(stream)))
    return out, indices


def ds_decode_sparse_attn_threshold(q, K, V, label, channels, T: int, k_max: int, tau: float, block: int = 1,
                                    scale: float = 0.0, out=None, indices=None, counts=None, workspace=None,
                                    stream=None, t_append: int | None = None):
    """The decode step with the threshold rule (positive-only head aggregation, keep the units scoring
    >= tau, at most k_max).  Returns (out fp32 [B, Hq, d], indices int32 [B, Hkv, k_max] with -1 past
    each row's count, counts int32 [B, Hkv])."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    dt = _dtype_code(q)
    if K.dtype != q.dtype or V.dtype != q.dtype or label.dtype != q.dtype:
        raise ValueError("q, K, V and label must share one dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=q.device)
    if counts is None:
        counts = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_max, q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_sparse_attn_threshold(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dev(label, "label"),
                                                 _dev(channels, "channels"), r, dt, B, Hq, Hkv, d, T_cap, T,
                                                 t_append, block, k_max, tau, scale, _dev(out, "out"),
                                                 _dev(indices, "indices"), _dev(counts, "counts"),
                                                 _dev(workspace, "workspace"),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices, counts


def ds_decode_score_threshold(q, K, label, channels, T: int, k_max: int, block: int = 1, workspace=None,
                              stream=None, t_append: int | None = None):
    """First phase of ds_decode_sparse_attn_threshold (label-row append and positive-only scores into the
    workspace).  Returns workspace."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_max, q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_score_threshold(_dev(q, "q"), _dev(K, "K"), _dev(label, "label"),
                                           _dev(channels, "channels"), r, _dtype_code(q), B, Hq, Hkv, d, T_cap, T,
                                           t_append, block, k_max, _dev(workspace, "workspace"),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace


def ds_decode_select_attend_threshold(q, K, V, T: int, k_max: int, tau: float, workspace, block: int = 1,
                                      scale: float = 0.0, out=None, indices=None, counts=None, stream=None):
    """Second phase of ds_decode_sparse_attn_threshold, from a workspace ds_decode_score_threshold filled.
    Returns (out, indices, counts)."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=q.device)
    if counts is None:
        counts = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
    _check(lib().ds_decode_select_attend_threshold(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(q), B, Hq,
                                                   Hkv, d, T_cap, T, block, k_max, tau, scale, _dev(out, "out"),
                                                   _dev(indices, "indices"), _dev(counts, "counts"),
                                                   _dev(workspace, "workspace"),
                                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices, counts


def ds_decode_sparse_attn_offload(q, K, V, label, channels, T: int, k_units: int, block: int = 1, scale: float = 0.0,
                                  out=None, indices=None, workspace=None, stream=None, t_append: int | None = None):
    """The decode step with K and V in pinned host memory (everything else on the device).
    Returns (out fp32 [B, Hq, d], indices int32 [B, Hkv, k_units])."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    dt = _dtype_code(q)
    if K.dtype != q.dtype or V.dtype != q.dtype or label.dtype != q.dtype:
        raise ValueError("q, K, V and label must share one dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_units, q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_sparse_attn_offload(_dev(q, "q"), _host(K, "K"), _host(V, "V"), _dev(label, "label"),
                                               _dev(channels, "channels"), r, dt, B, Hq, Hkv, d, T_cap, T, t_append,
                                               block, k_units, scale, _dev(out, "out"), _dev(indices, "indices"),
                                               _dev(workspace, "workspace"),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices


def ds_hip_token_capacity(T: int, k_spans: int, span: int) -> int:
    cap = lib().ds_hip_token_capacity(T, k_spans, span)
    if cap == 0:
        raise DsError(DS_ERR_INVALID_ARGUMENT, ds_last_error())
    return cap


def ds_decode_hip_attn(q, K, V, T: int, k_spans: int, span: int, scale: float = 0.0, out=None, spans=None,
                       workspace=None, stream=None):
    """Decode with the hierarchical span search.  Returns (out fp32 [B, Hq, d], spans int32 [B, Hkv, k_spans, 2])."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    if K.dtype != q.dtype or V.dtype != q.dtype:
        raise ValueError("q, K and V must share one dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if spans is None:
        spans = torch.empty((B, Hkv, k_spans, 2), dtype=torch.int32, device=q.device)
    if workspace is None:
        n = lib().ds_hip_workspace_bytes(B, Hq, Hkv, d, T, k_spans, span)
        if n == 0:
            raise DsError(DS_ERR_INVALID_ARGUMENT, ds_last_error())
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(lib().ds_decode_hip_attn(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(q), B, Hq, Hkv, d, T_cap,
                                    T, k_spans, span, scale, _dev(out, "out"), _dev(spans, "spans"),
                                    _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return out, spans


def ds_hip_search(q, K, T: int, k_spans: int, span: int, spans=None, tokens=None, stream=None):
    """Steps 0-2 of ds_decode_hip_attn.  Returns (spans [B, Hkv, k_spans, 2], tokens [B, Hkv, capacity])."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    cap = ds_hip_token_capacity(T, k_spans, span)
    if spans is None:
        spans = torch.empty((B, Hkv, k_spans, 2), dtype=torch.int32, device=q.device)
    if tokens is None:
        tokens = torch.empty((B, Hkv, cap), dtype=torch.int32, device=q.device)
    _check(lib().ds_hip_search(_dev(q, "q"), _dev(K, "K"), _dtype_code(q), B, Hq, Hkv, d, T_cap, T, k_spans, span,
                               _dev(spans, "spans"), _dev(tokens, "tokens"), _stream(stream)))
    return spans, tokens


def ds_decode_sparse_attn_ragged(q, K, V, label, channels, seq_lens, T_max: int, k_units: int, block: int = 1,
                                 n_append: int = 1, scale: float = 0.0, out=None, indices=None, workspace=None,
                                 stream=None):
    """The decode step for sequences of unequal lengths: seq_lens is a device int32 [B] tensor.
    Returns (out fp32 [B, Hq, d], indices int32 [B, Hkv, k_units], -1 past each row's kept count)."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    dt = _dtype_code(q)
    if K.dtype != q.dtype or V.dtype != q.dtype or label.dtype != q.dtype:
        raise ValueError("q, K, V and label must share one dtype")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T_max, block, k_units, q.device)
    _check(lib().ds_decode_sparse_attn_ragged(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dev(label, "label"),
                                              _dev(channels, "channels"), r, dt, B, Hq, Hkv, d, T_cap, T_max,
                                              _dev(seq_lens, "seq_lens"), n_append, block, k_units, scale,
                                              _dev(out, "out"), _dev(indices, "indices"), _dev(workspace, "workspace"),
                                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices


def ds_decode_score(q, K, label, channels, T: int, k_units: int, block: int = 1, workspace=None, stream=None,
                    t_append: int | None = None):
    """First phase of ds_decode_sparse_attn (label-row append and scores into the workspace).  Returns workspace."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_units, q.device)
    if t_append is None:
        t_append = T
    _check(lib().ds_decode_score(_dev(q, "q"), _kv(K, "K"), _dev(label, "label"), _dev(channels, "channels"), r,
                                 _dtype_code(q), B, Hq, Hkv, d, T_cap, T, t_append, block, k_units,
                                 _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))
    return workspace


def ds_decode_select_attend(q, K, V, T: int, k_units: int, workspace, block: int = 1, scale: float = 0.0, out=None,
                            indices=None, stream=None):
    """Second phase of ds_decode_sparse_attn, from a workspace ds_decode_score filled.  Returns (out, indices)."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    _check(lib().ds_decode_select_attend(_dev(q, "q"), _kv(K, "K"), _kv(V, "V"), _dtype_code(q), B, Hq, Hkv, d,
                                         T_cap, T, block, k_units, scale, _dev(out, "out"), _dev(indices, "indices"),
                                         _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))
    return out, indices


def _check_seq_lens(seq_lens, B):
    torch = _torch()
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")


def ds_decode_score_ragged(q, K, label, channels, seq_lens, T_max: int, k_units: int, block: int = 1,
                           n_append: int = 1, workspace=None, stream=None):
    """First phase of ds_decode_sparse_attn_ragged (label-row rebuild and scores into the workspace).
    Returns workspace."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    r = channels.shape[1]
    _check_seq_lens(seq_lens, B)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T_max, block, k_units, q.device)
    _check(lib().ds_decode_score_ragged(_dev(q, "q"), _dev(K, "K"), _dev(label, "label"), _dev(channels, "channels"),
                                        r, _dtype_code(q), B, Hq, Hkv, d, T_cap, T_max, _dev(seq_lens, "seq_lens"),
                                        n_append, block, k_units, _dev(workspace, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace


def ds_decode_select_attend_ragged(q, K, V, seq_lens, T_max: int, k_units: int, workspace, block: int = 1,
                                   scale: float = 0.0, out=None, indices=None, stream=None):
    """Second phase of ds_decode_sparse_attn_ragged, from a workspace ds_decode_score_ragged filled.
    Returns (out, indices)."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    _check_seq_lens(seq_lens, B)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    _check(lib().ds_decode_select_attend_ragged(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(q), B, Hq,
                                                Hkv, d, T_cap, T_max, _dev(seq_lens, "seq_lens"), block, k_units,
                                                scale, _dev(out, "out"), _dev(indices, "indices"),
                                                _dev(workspace, "workspace"),
                                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices


def ds_select_attention(q, K, V, scores, T: int, k_units: int, block: int = 1, scale: float = 0.0, out=None,
                        indices=None, workspace=None, stream=None):
    """Selection + attention from a score tensor as ds_label_scores returns it.  Returns (out, indices)."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((B, Hkv, k_units), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_units, q.device)
    _check(lib().ds_select_attention(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(q), B, Hq, Hkv, d, T_cap,
                                     T, block, k_units, _dev(scores, "scores"), scores.shape[-1], scale,
                                     _dev(out, "out"), _dev(indices, "indices"), _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, indices


def ds_label_scores(q, label, channels, T: int, block: int = 1, scores=None, stream=None):
    """Approximate scores only: float32 [B, Hkv, ld] with the first ceil(T/block) entries of each row valid."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, r = label.shape
    n_units = -(-T // block)
    ld = -(-n_units // 4) * 4
    if scores is None:
        scores = torch.empty((B, Hkv, ld), dtype=torch.float32, device=q.device)
    ld = scores.shape[-1]
    _check(lib().ds_label_scores(_dev(q, "q"), _dev(label, "label"), _dev(channels, "channels"), r, _dtype_code(q), B,
                                 Hq, Hkv, d, T_cap, T, block, _dev(scores, "scores"), ld, _stream(stream)))
    return scores


def ds_label_scores_positive(q, label, channels, T: int, block: int = 1, scores=None, stream=None):
    """Positive-only aggregated scores (the threshold rule's step 1), laid out as ds_label_scores."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, r = label.shape
    n_units = -(-T // block)
    ld = -(-n_units // 4) * 4
    if scores is None:
        scores = torch.empty((B, Hkv, ld), dtype=torch.float32, device=q.device)
    ld = scores.shape[-1]
    _check(lib().ds_label_scores_positive(_dev(q, "q"), _dev(label, "label"), _dev(channels, "channels"), r,
                                          _dtype_code(q), B, Hq, Hkv, d, T_cap, T, block, _dev(scores, "scores"), ld,
                                          _stream(stream)))
    return scores


def ds_topk_select(scores, n: int, k: int, idx=None, stream=None):
    """Top-k per row of a float32 [..., ld] score tensor (first n entries of each row).  Returns int32 [..., k]."""
    torch = _torch()
    ld = scores.shape[-1]
    rows = scores.numel() // ld
    if idx is None:
        idx = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    _check(lib().ds_topk_select(_dev(scores, "scores"), rows, n, ld, k, _dev(idx, "idx"), _stream(stream)))
    return idx


def ds_sparse_attn_from_indices(q, K, V, indices, T: int, block: int = 1, scale: float = 0.0, out=None,
                                workspace=None, stream=None):
    """Attention over given kept units only.  Returns out fp32 [B, Hq, d]."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = K.shape
    k_units = indices.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, d, T, block, k_units, q.device)
    _check(lib().ds_sparse_attn_from_indices(_dev(q, "q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(q), B, Hq, Hkv,
                                             d, T_cap, T, block, k_units, _dev(indices, "indices"), scale,
                                             _dev(out, "out"), _dev(workspace, "workspace"),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return out
