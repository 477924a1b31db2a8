"""Per-phase timelines of the decode step's kernels, from their clock stamps.

    python -m long_context_sparse_ds_amd.build --stamps
    python -m long_context_sparse_ds_amd.stamps --workload llama7b_16k

Runs the one-call decode step (ds_decode_sparse_attn) of a workload on the
benchmark's synthetic inputs through the stamped build of the library
(libdsparse_stamps.so beside the library: the same kernels, compiled with DS_STAMPS so that
thread 0 of every workgroup stores the shader clock at each phase boundary; see
csrc/stamps.h).  Several input copies rotate so that a step does not find the
previous one's rows in the caches.  For each stamped kernel of the step it
prints the median, 10th and 90th percentile over the launch's workgroups of
every stamp, in shader-clock cycles from the workgroup's own start, then the
launch's span and the gap before it on the 100 MHz constant clock.  A stamp
taken by thread 0 shows when wavefront 0 got there; after a barrier, when the
whole workgroup had.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import _binding as B
from .build import LIB_STAMPS

# Stamp slots of each stamped source file, in the order a workgroup passes them.
PHASES = {
    "score": {2: "q and channel table in", 3: "wavefront 0: label rows in, scored", 4: "tile histogram",
              5: "bin starts", 6: "bin starts in LDS", 7: "tile sorted in LDS", 8: "list stores issued"},
    "select": {2: "partition scored", 3: "partition threshold", 4: "candidates' histogram stored",
               5: "candidates emitted"},
    "bucket": {2: "prefix words, list heads in", 3: "d0", 4: "tiles' slices", 5: "candidates classified",
               6: "radix passes, join", 7: "position scan", 8: "split's kept list in LDS",
               9: "wavefront 0: gather, lane-group merge", 10: "all states in LDS", 11: "combine weights",
               12: "state stored", 13: "stores completed", 14: "ticket", 15: "splits merged"},
    "selattn": {16: "one pass: label rows scored", 2: "scores, top-digit counts in", 3: "d0",
                4: "units classified", 5: "first candidate pass", 6: "second candidate pass", 7: "threshold",
                8: "kept units classified", 9: "kept list in LDS", 10: "slots mapped to units",
                11: "indices written", 12: "wavefront 0: gather", 13: "output or state stored", 14: "ticket",
                15: "splits merged"},
}
ORDER = ["score", "select", "bucket", "selattn"]
SLOTS, WGS = 32, 4096


def _load(path: str) -> ctypes.CDLL:
    h = ctypes.CDLL(path)
    for name, (res, args) in B._SIGNATURES.items():
        if hasattr(h, name):
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
    for name in PHASES:
        getattr(h, f"ds_stamps_dump_{name}").argtypes = [ctypes.c_void_p]
    return h


def timeline(workload: str, copies: int = 4, reps: int = 5) -> str:
    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import dsgen

    if not os.path.exists(LIB_STAMPS):
        raise RuntimeError(f"{LIB_STAMPS} is missing: python -m long_context_sparse_ds_amd.build --stamps")
    h = _load(LIB_STAMPS)
    w = dsgen.get(workload)
    if w.ragged or w.tau is not None or w.hip or w.offload:
        raise ValueError("stamps: the uniform top-k step only")
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = B.ds_calibrate_channels(qc, kc, w.r)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if w.dtype == "bf16" else a)
        return t.to(dev).view(tdt)

    chd = torch.from_numpy(ch).to(dev)
    insts = []
    for _ in range(copies):
        it = {"q": up(q), "K": up(K), "V": up(V)}
        it["label"] = B.ds_build_label_cache(it["K"], chd)
        insts.append(it)
    wsb = h.ds_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units)
    for it in insts:
        it["ws"] = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    idx = torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    vp = ctypes.c_void_p
    dt = 1 if w.dtype == "bf16" else 0

    def step(it):
        st = h.ds_decode_sparse_attn(vp(it["q"].data_ptr()), vp(it["K"].data_ptr()), vp(it["V"].data_ptr()),
                                     vp(it["label"].data_ptr()), vp(chd.data_ptr()), w.r, dt, w.B, w.Hq, w.Hkv,
                                     w.d, w.cap, w.T, w.T - 1, w.block, w.k_units, 0.0, vp(out.data_ptr()),
                                     vp(idx.data_ptr()), vp(it["ws"].data_ptr()), wsb, vp(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(h.ds_last_error().decode())

    for i in range(2 * copies):   # warm-up
        step(insts[i % copies])
    torch.cuda.synchronize()
    got = {name: [] for name in PHASES}
    buf = np.zeros(WGS * SLOTS, dtype=np.uint64)
    for rep in range(reps):
        for name in PHASES:
            if getattr(h, f"ds_stamps_clear_{name}")() != 0:
                raise RuntimeError("stamp buffer clear failed")
        step(insts[rep % copies])
        torch.cuda.synchronize()
        for name in PHASES:
            if getattr(h, f"ds_stamps_dump_{name}")(buf.ctypes.data) != 0:
                raise RuntimeError("stamp buffer read failed")
            a = buf.reshape(WGS, SLOTS).astype(np.int64)
            ran = a[:, 1] > 0
            if ran.any():
                got[name].append(a[ran].copy())
    lines = [f"workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} r={w.r} block={w.block} "
             f"k={w.k_units} {w.dtype}; {reps} steps, stamps of every workgroup"]
    prev_end = None
    for name in ORDER:
        if not got[name]:
            continue
        a = np.concatenate(got[name])
        wgs = len(a) // len(got[name])
        lines.append(f"\n{name} ({wgs} workgroups per launch): cycles from the workgroup's start")
        for slot, label in PHASES[name].items():
            v = a[:, slot] - a[:, 1]
            v = v[(a[:, slot] > 0) & (v >= 0)]
            if len(v):
                lines.append(f"  {slot:2d} {label:40s} median {np.median(v):8.0f}  p10 {np.percentile(v, 10):8.0f}"
                             f"  p90 {np.percentile(v, 90):8.0f}  ({len(v)} stamps)")
        spans, gaps = [], []
        for r in got[name]:
            ends = r[:, 31][r[:, 31] > 0]
            if len(ends):
                spans.append((ends.max() - r[:, 0].min()) / 100.0)
        lines.append(f"  launch span (first start to last end): median {np.median(spans):.2f} us")
        if prev_end is not None:
            for r, e in zip(got[name], prev_end):
                gaps.append((r[:, 0].min() - e) / 100.0)
            lines.append(f"  gap after the previous kernel's last workgroup: median {np.median(gaps):.2f} us")
        prev_end = [r[:, 31][r[:, 31] > 0].max() for r in got[name]]
    return "\n".join(lines)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="llama7b_16k")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    print(timeline(args.workload, args.copies, args.reps), flush=True)


if __name__ == "__main__":
    main()
