"""Benchmark of the Double Sparsity sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b_16k]

A step is one pass of the whole per-step path over one decode batch: one
ds_decode_sparse_attn call that appends the newest token's label row (row
T-1, rebuilt from K inside the call), scores every token from the label
cache, selects the top-k and runs attention over the kept K/V rows (with the
cross-split merge).  A ragged workload (--workload ragged_16k) runs
ds_decode_sparse_attn_ragged instead: each sequence is scored, selected and
attended over its own length.  The threshold workload (--workload
jenga_gqa_32k) runs ds_decode_sparse_attn_threshold: positive-only head
aggregation, block max, and every block scoring at least tau kept (at most
k_max); its kept-token count, and so its byte count, comes from the call's own
counts.  The span-search workload (--workload hip_1m) runs ds_decode_hip_attn
over one million tokens: the search phase is ds_hip_search, the attention phase
ds_sparse_attn_from_indices over its token list.  The offload workload (--workload offload_256k) keeps K and V in pinned
host memory and runs ds_decode_sparse_attn_offload; its roofline is the host
link, against a measured pinned-to-device copy.  Offline calibration is outside the step.  Steps rotate
over N independent copies of the cache ("layers") so the per-step working set
cannot be served from the 256 MB Infinity Cache.  K steps are captured into
HIP graphs and replayed; the timed region is bracketed by device
synchronisation and HIP events on the replay stream.

Per-kernel durations come from the stage entry points (same kernels), each
replayed from its own graph over the rotating instances; the dominant one
gives the roofline object.  A shape that the one-call step runs in one pass
(ds_decode_is_one_pass: one kernel scores, selects and attends) has that
kernel as its roofline, timed the same way; its phase entry points still run
the two-kernel form and are reported beside it.  The CPU baseline times the float64 oracle on a
bounded sample of the same workload with a process pool.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import dsgen  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "sparse decode attention µs/step + achieved HBM GB/s (T=16K, 32 heads, bf16)"
MALL_BYTES = 256 * 2 ** 20
# The two phases of the span-search step, timed through ds_hip_search and ds_sparse_attn_from_indices.
PHASE_NAMES = {"decode_score": "hip_search", "decode_select_attend": "attention_from_indices"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The sources that build each timed stage's kernels and plan their launches: a recorded counter reading stays
# valid while these files are unchanged (the other kernels' sources do not enter its digest).
STAGE_SOURCES = {
    "decode_score": ("ds_api.hip", "ds_common.h", "stamps.h", "label_dot.h", "score.hip", "select_dev.h",
                     "select.hip"),
    "decode_select_attend": ("ds_api.hip", "ds_common.h", "stamps.h", "label_dot.h", "select_dev.h", "fused_dev.h",
                             "select.hip", "selattn.hip", "bucket.hip", "attn.hip"),
    "decode_step_one_pass": ("ds_api.hip", "ds_common.h", "stamps.h", "label_dot.h", "select_dev.h", "fused_dev.h",
                             "selattn.hip"),
    "hip_search": ("ds_api.hip", "ds_common.h", "stamps.h", "hip_search.hip"),
    "attention_from_indices": ("ds_api.hip", "ds_common.h", "stamps.h", "attn.hip"),
}


def kernel_sources_digest(stage: str) -> str:
    """Digest of the sources of one stage's kernels and their launch plan."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_sparse_ds_amd", "csrc")
    for name in STAGE_SOURCES[stage]:
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, stage: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a copy kernel) and
    recorded in profiles/, or None when no record matches the current sources of that stage's kernels."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_traffic.md")
    if not os.path.exists(path) or stage not in STAGE_SOURCES:
        return None
    digest = kernel_sources_digest(stage)
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                kv = dict(item.split("=", 1) for item in line.split(":", 1)[1].split())
                if kv.get("stage") == stage and kv.get("sources") == digest:
                    return int(kv["bytes"])
    return None


def hip_rounds(w: dsgen.Workload) -> int:
    """Rounds of the span search: halvings of ceil(T / k) until it is at most the final span length."""
    n, r = -(-w.T // w.k_units), 0
    while n > w.block:
        n, r = -(-n // 2), r + 1
    return r


def algorithmic_bytes(w: dsgen.Workload, lens=None, kept=None) -> dict:
    """Bytes the method must move per step (score workspace, split partials and
    the label build are excluded).  lens: per-sequence lengths of a ragged batch.
    kept: (kept tokens, kept units) summed over the rows, for the threshold rule,
    whose kept counts depend on the data."""
    e = w.elem_bytes
    if w.hip:
        # kept = (kept tokens, representative tokens scored), summed over the rows
        kept_tokens, scored = kept if kept is not None else (w.B * w.Hkv * w.k_units * w.block,
                                                             w.B * w.Hkv * w.k_units * (1 + hip_rounds(w)))
        parts = {"search_keys": scored * w.d * e, "kv_gather": 2 * kept_tokens * w.d * e,
                 "q": w.B * w.Hq * w.d * e, "out": 4 * w.B * w.Hq * w.d, "spans": 8 * w.B * w.Hkv * w.k_units}
        parts["step"] = sum(parts.values())
        return parts
    if lens is None:
        lens = [w.T] * w.B
    tokens = sum(int(t) for t in lens)
    if kept is None:
        kept_tokens = w.Hkv * sum(min(w.k_units * w.block, int(t)) for t in lens)
        kept_units = w.Hkv * sum(min(w.k_units, -(-int(t) // w.block)) for t in lens)
    else:
        kept_tokens, kept_units = kept
    parts = {
        "label_scan": w.Hkv * tokens * w.r * e,
        "kv_gather": 2 * kept_tokens * w.d * e,
        "q": w.B * w.Hq * w.d * e,
        "out": 4 * w.B * w.Hq * w.d,
        "indices": 4 * kept_units,
        "label_append": 2 * w.B * w.Hkv * w.r * e,   # read r channels of K row T-1, write one label row
    }
    if w.ragged:
        parts["seq_lens"] = 4 * w.B
    if w.tau is not None:
        parts["counts"] = 4 * w.B * w.Hkv
    parts["step"] = sum(parts.values())
    return parts


def default_instances(w: dsgen.Workload) -> int:
    per = algorithmic_bytes(w)["step"]
    n = max(1, math.ceil(2 * MALL_BYTES / per))
    inst_bytes = 2 * w.B * w.Hkv * w.cap * w.d * w.elem_bytes
    cap = max(1, int(60e9 // max(inst_bytes, 1)))
    return int(min(n, 32, cap))


# ---------------------------------------------------------------- CPU baseline (oracle)

_ORACLE_UNITS = None


def _oracle_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_task(i):
    import oracle as O
    qg, Kf, Vf, ch, k, block, T, tau = _ORACLE_UNITS[i]
    if ch is None:   # span search: k spans, final span length `block`
        O.decode_unit_hip(qg, Kf, Vf, k, block, None, T)
    elif tau is None:
        O.decode_unit(qg, Kf, Vf, ch, k, block, None, T)
    else:
        O.decode_unit_threshold(qg, Kf, Vf, ch, k, tau, block, None, T)
    return i


def cpu_baseline(w, q, K, V, ch, seconds: float, lens):
    """Wall time of the oracle's decode step on the host cores, over a bounded sample."""
    global _ORACLE_UNITS
    import multiprocessing as mp
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    # A sample of whole units; at most 64 units (about 2 GB of float64 inputs at T=16K).  A ragged batch
    # samples the same number of heads from every sequence, so the sample's mean unit stands for the batch's.
    if w.ragged:
        per = max(1, min(w.Hkv, 64 // w.B))
        sample = [(b, g) for b in range(w.B) for g in range(per)]
    elif w.hip:
        sample = units[:4]   # float64 copies of million-token rows: 2 GB per unit
    else:
        sample = units[:64]
    G = w.G

    def unit(b, g):
        Tb = int(lens[b])
        k_b = min(w.k_units, -(-Tb // w.block))
        return (dsgen.to_f64(q[b, g * G:(g + 1) * G], w.dtype), dsgen.to_f64(K[b, g, :Tb], w.dtype),
                dsgen.to_f64(V[b, g, :Tb], w.dtype), None if w.hip else ch[g], w.k_units if w.hip else k_b,
                w.block, Tb, w.tau)

    _ORACLE_UNITS = [unit(b, g) for b, g in sample]
    cores = max(1, min(16, len(os.sched_getaffinity(0)), len(sample)))
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_oracle_init) as pool:
        pool.map(_oracle_task, range(len(sample)))   # warm
        reps, t0 = 0, time.perf_counter()
        while True:
            pool.map(_oracle_task, range(len(sample)))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                break
    _ORACLE_UNITS = None
    per_unit_s = el / (reps * len(sample))
    step_s = per_unit_s * len(units)
    return {"step_s": step_s, "cores": cores, "reps": reps, "sample_units": len(sample), "units": len(units),
            "elapsed_s": el}


# ---------------------------------------------------------------- GPU

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default=dsgen.HEADLINE, choices=dsgen.WORKLOAD_ORDER + dsgen.RAGGED_ORDER + dsgen.THRESHOLD_ORDER +
                    dsgen.OFFLOAD_ORDER + dsgen.HIP_ORDER)
    ap.add_argument("--instances", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--phases-only", action="store_true",
                    help="time only the step's own two phases, not the isolated reference stages (for counter runs)")
    ap.add_argument("--sources-digest", choices=sorted(STAGE_SOURCES),
                    help="print the source digest of one stage's kernels (the key of its traffic records) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times and exit (reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    if args.sources_digest:
        print(kernel_sources_digest(args.sources_digest))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this single-GPU build has no multi-GPU path "
              "(each GPU would run the same kernels on its own share of (sequence, KV head) rows).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_ds_amd as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 10}), flush=True)
        return
    L.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = dsgen.get(args.workload)
    lens = dsgen.seq_lengths(w)
    ab = algorithmic_bytes(w, lens)
    n_inst = args.instances or default_instances(w)
    log(f"workload {w.name}: {w}" + (f", lengths {lens.tolist()}" if w.ragged else ""))
    log(f"algorithmic bytes/step {ab['step']}, instances {n_inst}")

    t0 = time.perf_counter()
    q, K, V = dsgen.gen_cache(w)
    qc, kc = dsgen.gen_calib(w)
    ch = L.ds_calibrate_channels(qc, kc, w.r)
    log(f"generated inputs in {time.perf_counter() - t0:.1f}s")

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q0, K0, V0 = up(q), up(K), up(V)
    chd = torch.from_numpy(ch).to(dev)
    seq = torch.from_numpy(lens).to(dev)
    # full label build, timed on its own (prefill cost, not part of the step); the span search uses none
    lab0, label_build_us = None, None
    if not w.hip:
        lab0 = L.ds_build_label_cache(K0, chd)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        L.ds_build_label_cache(K0, chd, label=lab0)
        ev1.record()
        torch.cuda.synchronize()
        label_build_us = ev0.elapsed_time(ev1) * 1e3

    if w.offload:
        # K and V live in pinned host memory; the device keeps q, the label cache and the outputs.
        def pinned_copy(t):
            return torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t)
        K0, V0 = pinned_copy(K0), pinned_copy(V0)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    inst = []
    for i in range(n_inst):
        if i == 0:
            qi, Ki, Vi, li = q0, K0, V0, lab0
        elif w.offload:
            qi, Ki, Vi, li = q0.clone(), pinned_copy(K0), pinned_copy(V0), lab0.clone()
        else:
            qi, Ki, Vi, li = q0.clone(), K0.clone(), V0.clone(), (lab0.clone() if lab0 is not None else None)
        extra = {}
        if w.hip:
            ws = torch.empty(L.lib().ds_hip_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.T, w.k_units, w.block),
                             dtype=torch.uint8, device=dev)
            cap = L.ds_hip_token_capacity(w.T, w.k_units, w.block)
            extra = dict(spans=torch.empty((w.B, w.Hkv, w.k_units, 2), dtype=torch.int32, device=dev),
                         tokens=torch.empty((w.B, w.Hkv, cap), dtype=torch.int32, device=dev),
                         ws_attn=L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, 1, cap, dev))
        else:
            ws = L.alloc_workspace(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units, dev)
        out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        idx = torch.empty((w.B, w.Hkv, w.k_units), dtype=torch.int32, device=dev)
        cnt = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
        inst.append(dict(q=qi, K=Ki, V=Vi, label=li, ws=ws, out=out, idx=idx, cnt=cnt, **extra))
    del q, K, V
    torch.cuda.synchronize()
    log(f"{n_inst} instances resident ({torch.cuda.memory_allocated() / 2 ** 30:.1f} GiB)")

    def step(i):
        it = inst[i % n_inst]
        if w.hip:
            L.ds_decode_hip_attn(it["q"], it["K"], it["V"], w.T, w.k_units, w.block, out=it["out"],
                                 spans=it["spans"], workspace=it["ws"])
        elif w.ragged:
            L.ds_decode_sparse_attn_ragged(it["q"], it["K"], it["V"], it["label"], chd, seq, w.T, w.k_units,
                                           w.block, n_append=1, out=it["out"], indices=it["idx"],
                                           workspace=it["ws"])
        elif w.tau is not None:
            L.ds_decode_sparse_attn_threshold(it["q"], it["K"], it["V"], it["label"], chd, w.T, w.k_units, w.tau,
                                              w.block, out=it["out"], indices=it["idx"], counts=it["cnt"],
                                              workspace=it["ws"], t_append=w.T - 1)
        elif w.offload:
            L.ds_decode_sparse_attn_offload(it["q"], it["K"], it["V"], it["label"], chd, w.T, w.k_units, w.block,
                                            out=it["out"], indices=it["idx"], workspace=it["ws"], t_append=w.T - 1)
        else:
            L.ds_decode_sparse_attn(it["q"], it["K"], it["V"], it["label"], chd, w.T, w.k_units, w.block,
                                    out=it["out"], indices=it["idx"], workspace=it["ws"], t_append=w.T - 1)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if w.hip:
        # Kept tokens from the call's own spans (the tests check them against the oracle).
        step(0)
        torch.cuda.synchronize()
        sp = inst[0]["spans"].cpu().numpy()
        kept_tokens = int((sp[..., 1] - sp[..., 0]).sum())
        ab = algorithmic_bytes(w, None, (kept_tokens, w.B * w.Hkv * w.k_units * (1 + hip_rounds(w))))
        log(f"span search: {hip_rounds(w)} rounds, {kept_tokens} tokens kept; algorithmic bytes/step {ab['step']}")
    if w.tau is not None:
        # The threshold rule keeps a data-dependent number of units: count the kept
        # tokens from the call's own output (the tests check it against the oracle).
        step(0)
        torch.cuda.synchronize()
        cnt0 = inst[0]["cnt"].cpu().numpy()
        idx0 = inst[0]["idx"].cpu().numpy()
        kept_tokens = 0
        for b in range(w.B):
            for g in range(w.Hkv):
                ids = idx0[b, g, :int(cnt0[b, g])].astype(np.int64)
                kept_tokens += int(np.minimum(w.block, w.T - ids * w.block).sum())
        ab = algorithmic_bytes(w, lens, (kept_tokens, int(cnt0.sum())))
        log(f"threshold rule: kept units per row {cnt0.reshape(-1).tolist()}, {kept_tokens} tokens; "
            f"algorithmic bytes/step {ab['step']}")

    def capture(n_steps, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn(0)   # eager run on the capture stream (lazy init)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n_steps):
                    fn(i)
        torch.cuda.synchronize()
        return g

    rot = capture(n_inst, step)
    rem = args.steps % n_inst
    rem_graph = capture(rem, step) if rem else None
    warm_graph = capture(args.warmup, step) if args.warmup else None

    with torch.cuda.stream(stream):
        if warm_graph is not None:
            warm_graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_host0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps // n_inst):
            rot.replay()
        if rem_graph is not None:
            rem_graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t_host1 = time.perf_counter()
    ms_total = e0.elapsed_time(e1)
    us_step = ms_total * 1e3 / args.steps
    log(f"graph replay: {us_step:.2f} us/step over {args.steps} steps (host wall {(t_host1 - t_host0) * 1e3:.2f} ms)")

    # eager (host-launched) steps, for reference
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        e0.record(stream)
        n_eager = min(args.steps, 4 * n_inst)
        for i in range(n_eager):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    us_step_eager = e0.elapsed_time(e1) * 1e3 / n_eager

    # ---- per-kernel durations via the stage entry points, graph-replayed over the instances
    scores_buf = [torch.empty((w.B, w.Hkv, -(-w.n_units // 64) * 64), dtype=torch.float32, device=dev)
                  for _ in range(n_inst)]

    def st_append(i):
        it = inst[i % n_inst]
        L.ds_build_label_cache(it["K"], chd, w.T - 1, w.T, label=it["label"])

    def st_scores(i):
        it = inst[i % n_inst]
        L.ds_label_scores(it["q"], it["label"], chd, w.T, w.block, scores=scores_buf[i % n_inst])

    def st_decode_score(i):
        it = inst[i % n_inst]
        if w.hip:
            L.ds_hip_search(it["q"], it["K"], w.T, w.k_units, w.block, spans=it["spans"], tokens=it["tokens"])
        elif w.ragged:
            L.ds_decode_score_ragged(it["q"], it["K"], it["label"], chd, seq, w.T, w.k_units, w.block, n_append=1,
                                     workspace=it["ws"])
        elif w.tau is not None:
            L.ds_decode_score_threshold(it["q"], it["K"], it["label"], chd, w.T, w.k_units, w.block,
                                        workspace=it["ws"], t_append=w.T - 1)
        else:
            L.ds_decode_score(it["q"], it["K"], it["label"], chd, w.T, w.k_units, w.block, workspace=it["ws"],
                              t_append=w.T - 1)

    def st_decode_select_attend(i):
        it = inst[i % n_inst]
        if w.hip:
            L.ds_sparse_attn_from_indices(it["q"], it["K"], it["V"], it["tokens"], w.T, 1, out=it["out"],
                                          workspace=it["ws_attn"])
        elif w.ragged:
            L.ds_decode_select_attend_ragged(it["q"], it["K"], it["V"], seq, w.T, w.k_units, it["ws"], w.block,
                                             out=it["out"], indices=it["idx"])
        elif w.tau is not None:
            L.ds_decode_select_attend_threshold(it["q"], it["K"], it["V"], w.T, w.k_units, w.tau, it["ws"], w.block,
                                                out=it["out"], indices=it["idx"], counts=it["cnt"])
        else:
            L.ds_decode_select_attend(it["q"], it["K"], it["V"], w.T, w.k_units, it["ws"], w.block,
                                      out=it["out"], indices=it["idx"])

    def st_select(i):
        it = inst[i % n_inst]
        L.ds_topk_select(scores_buf[i % n_inst], w.n_units, w.k_units, idx=it["idx"])

    def st_attn(i):
        it = inst[i % n_inst]
        L.ds_sparse_attn_from_indices(it["q"], it["K"], it["V"], it["idx"], w.T, w.block, out=it["out"],
                                      workspace=it["ws"])

    kernel_us = {}
    # The decode step's two phases (its own kernels), then isolated stages for reference
    # (uniform-length top-k stages, so not for a ragged batch or the threshold rule).  A
    # one-pass step is one kernel: the step itself is timed as its own stage.
    one_pass = (not w.hip and w.tau is None and
                L.ds_decode_is_one_pass(w.B, w.Hq, w.Hkv, w.d, w.T, w.block, w.k_units, w.r, w.dtype))
    stages = [("decode_score", st_decode_score), ("decode_select_attend", st_decode_select_attend)]
    if one_pass:
        stages = [("decode_step_one_pass", step)] + stages
    if not w.ragged and w.tau is None and not w.offload and not w.hip and not args.phases_only:
        stages += [("label_append", st_append), ("scores", st_scores), ("select", st_select),
                   ("attention_from_indices", st_attn)]
    elif w.tau is not None and not args.phases_only:
        # The separate attention kernel over the step's own kept blocks (slots past a row's count are -1).
        stages += [("attention_from_indices", st_attn)]
    for name, fn in stages:
        g = capture(n_inst, fn)
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.kernel_reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        kernel_us[name] = e0.elapsed_time(e1) * 1e3 / (args.kernel_reps * n_inst)
        del g
    log("per-stage us: " + ", ".join(f"{k}={v:.2f}" for k, v in kernel_us.items()))

    if w.hip:
        # the search (representative K rows, q, spans) and the attention over the kept tokens (reading
        # their int32 ids)
        kept_tok = ab["kv_gather"] // (2 * w.d * w.elem_bytes)
        stage_bytes = {"decode_score": ab["search_keys"] + ab["q"] + ab["spans"],
                       "decode_select_attend": ab["kv_gather"] + ab["q"] + ab["out"] + 4 * kept_tok}
    else:
        stage_bytes = {
            "decode_score": ab["label_scan"] + ab["q"] + ab["label_append"] + ab.get("seq_lens", 0),
            "decode_select_attend": ab["kv_gather"] + ab["q"] + ab["indices"] + ab["out"] + ab.get("seq_lens", 0) +
            ab.get("counts", 0),
            "label_append": ab["label_append"],
            "scores": ab["label_scan"] + ab["q"],
            "select": ab["indices"],
            "attention_from_indices": ab["kv_gather"] + ab["q"] + ab["indices"] + ab["out"],
            "decode_step_one_pass": ab["step"],
        }
    # the decode step's kernels: the one-pass kernel, or the score pass and selection + attention
    dominant = ("decode_step_one_pass" if one_pass else
                max(("decode_score", "decode_select_attend"), key=lambda k: kernel_us[k]))
    dom_gbs = stage_bytes[dominant] / (kernel_us[dominant] * 1e-6) / 1e9

    gbs = ab["step"] / (us_step * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us_step / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "T": w.T, "r": w.r,
                   "block": w.block, "k_units": w.k_units, "instances": n_inst, "launch": "hip graph replay",
                   "parallelism": "single GPU", **({"seq_lens": lens.tolist()} if w.ragged else {}),
                   **({"rule": "threshold", "tau": w.tau} if w.tau is not None else {}),
                   **({"kv_location": "pinned host memory"} if w.offload else {}),
                   **({"rule": "hierarchical span search", "k_spans": w.k_units, "span": w.block,
                       "rounds": hip_rounds(w)} if w.hip else {})},
        "us_per_step": round(us_step, 3),
        "one_pass": bool(one_pass),
        "us_per_step_eager": round(us_step_eager, 3),
        "algorithmic_bytes_per_step": ab["step"],
        "step_roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
        "label_build_us": round(label_build_us, 2) if label_build_us is not None else None,
        "stage_us": {PHASE_NAMES.get(k, k) if w.hip else k: round(v, 3) for k, v in kernel_us.items()},
        "roofline": {"bound": "hbm", "kernel": PHASE_NAMES.get(dominant, dominant) if w.hip else dominant, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, PHASE_NAMES.get(dominant, dominant) if w.hip else dominant),
                     "bytes_per_launch": stage_bytes[dominant], "avg_launch_us": round(kernel_us[dominant], 3)},
    }

    if w.offload:
        # The host link: kept K/V bytes per select-attend launch against a plain pinned-to-device copy.
        src = torch.empty(2 ** 30, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            dst.copy_(src, non_blocking=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(5):
                dst.copy_(src, non_blocking=True)
            e1.record(stream)
            torch.cuda.synchronize()
        h2d_gbs = 5 * 2 ** 30 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        link_gbs = ab["kv_gather"] / (kernel_us["decode_select_attend"] * 1e-6) / 1e9
        result["host_link"] = {"kv_bytes_per_step": ab["kv_gather"], "achieved_gbs": round(link_gbs, 2),
                               "pinned_to_device_copy_gbs": round(h2d_gbs, 2),
                               "frac_of_copy": round(link_gbs / h2d_gbs, 4)}
        result["roofline"].update({"bound": "host_link", "achieved": round(link_gbs, 2), "peak": round(h2d_gbs, 2),
                                   "frac": round(link_gbs / h2d_gbs, 4), "traffic": None,
                                   "peak_kind": "measured pinned-to-device copy (1 GiB)"})
        log(f"host link: {link_gbs:.1f} GB/s of kept K/V rows; pinned-to-device copy {h2d_gbs:.1f} GB/s")

    if not args.no_cpu and args.cpu_seconds > 0:
        q, K, V = dsgen.gen_cache(w)
        cb = cpu_baseline(w, q, K, V, ch, args.cpu_seconds, lens)
        cpu_us = cb["step_s"] * 1e6
        result["cpu_baseline"] = {
            "value": round(ab["step"] / cb["step_s"] / 1e9, 4), "unit": "GB/s", "us_per_step": round(cpu_us, 1),
            "cores": cb["cores"], "kind": "oracle",
            "sample": (f"float64 numpy oracle decode of {cb['sample_units']} of {cb['units']} (sequence, KV head) "
                       f"units, {cb['reps']} repetitions in {cb['elapsed_s']:.1f}s over a pool of {cb['cores']} "
                       f"single-threaded workers (the pool is capped at 16 workers, one per host core the "
                       f"process may use, and at the sample's unit count); scaled to the whole step")}
        result["gpu_over_cpu"] = round(cpu_us / us_step, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
