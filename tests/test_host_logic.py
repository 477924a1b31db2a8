"""Host-side logic on the CPU: the benchmark's byte accounting for every kind of
workload, the span search's round count (against the oracle's own stopping rule),
the seeded generators, the workspace sizes of the library's plans, and a lane-by-lane
model of the span search's one-wavefront selection network.  No GPU."""
import math
import os
import sys

import numpy as np
import pytest

import dsgen
import long_context_sparse_ds_amd as L
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_headline_bytes_match_the_definition():
    """label scan + kept K/V rows + q + fp32 out + indices + the appended label row."""
    w = dsgen.get("llama7b_16k")
    ab = bench.algorithmic_bytes(w)
    assert ab["label_scan"] == 32 * 16384 * 16 * 2
    assert ab["kv_gather"] == 2 * 32 * 1024 * 128 * 2
    assert ab["q"] == 32 * 128 * 2 and ab["out"] == 4 * 32 * 128 and ab["indices"] == 4 * 32 * 1024
    assert ab["label_append"] == 2 * 32 * 16 * 2
    assert ab["step"] == sum(v for k, v in ab.items() if k != "step") == 33_712_128


def test_block_workload_bytes_count_whole_blocks():
    w = dsgen.get("block64_256k")
    ab = bench.algorithmic_bytes(w)
    assert ab["kv_gather"] == 2 * 32 * 64 * 64 * 128 * 2
    assert ab["indices"] == 4 * 32 * 64


def test_ragged_bytes_use_each_sequence_length():
    w = dsgen.get("ragged_16k")
    lens = dsgen.seq_lengths(w)
    ab = bench.algorithmic_bytes(w, lens)
    assert ab["label_scan"] == w.Hkv * int(lens.sum()) * w.r * 2
    assert ab["kv_gather"] == 2 * w.Hkv * sum(min(w.k_units, int(t)) for t in lens) * w.d * 2
    assert ab["seq_lens"] == 4 * w.B
    short = w.with_(T=5000)
    ab2 = bench.algorithmic_bytes(short, np.array([5000, 300], dtype=np.int32))
    assert ab2["kv_gather"] == 2 * short.Hkv * (1024 + 300) * short.d * 2   # a short sequence keeps all it has


def test_threshold_bytes_follow_the_kept_counts():
    w = dsgen.get("jenga_gqa_32k")
    ab = bench.algorithmic_bytes(w, None, (123_264, 1_926))
    assert ab["kv_gather"] == 2 * 123_264 * 128 * 2 and ab["indices"] == 4 * 1_926
    assert ab["counts"] == 4 * w.B * w.Hkv


@pytest.mark.parametrize("T,k,span", [(1 << 20, 64, 64), (1000, 20, 64), (10, 3, 2), (97, 5, 3), (4096, 32, 16),
                                      (777, 50, 1), (65536, 1024, 16)])
def test_span_search_round_count_matches_the_oracle(T, k, span):
    """The host's round count (halvings of ceil(T / k) down to `span`) is at least the
    number of rounds the oracle runs, and the extra rounds change nothing: running the
    oracle's rule for exactly that many rounds ends with no span longer than `span`."""
    w = dsgen.Workload("r", "bf16", B=1, Hq=1, Hkv=1, d=128, T=T, r=16, block=span, k_units=k, seed_base=1, hip=True)
    rounds = bench.hip_rounds(w)
    longest = max((i + 1) * T // k - i * T // k for i in range(k))
    for _ in range(rounds):
        longest = longest if longest <= span else -(-longest // 2)
    assert longest <= span
    cap = L.ds_hip_token_capacity(T, k, span)
    assert cap == (k * span if rounds > 0 else T)
    if rounds > 0:
        assert k * span < T   # a round runs only when the spans cannot cover every token


def test_span_search_oracle_never_needs_more_rounds_than_the_host():
    rng = np.random.default_rng(3)
    for T, k, span in ((97, 5, 3), (1000, 16, 8), (300, 7, 2)):
        K = rng.standard_normal((T, 8))
        q = rng.standard_normal((2, 8))
        w = dsgen.Workload("r", "bf16", B=1, Hq=2, Hkv=1, d=8, T=T, r=4, block=span, k_units=k, seed_base=1)
        spans = O.hip_search(q, K, T, k, span)
        assert max(e - s for s, e in spans) <= span
        assert bench.hip_rounds(w) >= math.ceil(math.log2(max(1, -(-T // k) / span)))


def test_generators_are_deterministic_and_lengths_in_range():
    w = dsgen.get("ragged_16k")
    a, b = dsgen.seq_lengths(w), dsgen.seq_lengths(w)
    assert np.array_equal(a, b) and a[0] == w.T and a.min() >= w.T // 16 and a.max() <= w.T
    assert np.array_equal(dsgen.seq_lengths(dsgen.get("llama7b_16k")), [16384])
    small = dsgen.Workload("g", "bf16", B=2, Hq=4, Hkv=2, d=128, T=300, r=16, block=1, k_units=10, seed_base=77,
                           T_cap=320)
    q1, K1, V1 = dsgen.gen_cache(small)
    q2, K2, V2 = dsgen.gen_cache(small, threads=1)
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2) and np.array_equal(q1, q2)
    assert np.all(K1[:, :, 300:] == np.uint16(0x7FC0))   # NaN padding past T


def test_workspace_grows_with_the_two_stage_candidates():
    """Rows over 32,768 units whose candidates fit the fused kernel reserve candidate
    buffers; shapes beyond that fall back to the streaming path and still size cleanly."""
    small = L.ds_decode_workspace_bytes(1, 4, 2, 128, 70000, 1, 2000)
    assert small > 0
    cand = 2 * (3 * 2000) * (4 + 4)   # scores and ids of 3 partitions x k per row, 2 rows
    assert small >= cand
    stream = L.ds_decode_workspace_bytes(1, 4, 2, 128, 70000, 1, 20000)   # 3 * 20000 > 32768
    assert stream > 0


# ---------------------------------------------------------------------------
# The span search's one-wavefront selection (k <= 64 spans), modelled lane by
# lane: 64 lanes hold two keys each (element t * 64 + lane is item t), a bitonic
# network sorts them in descending order (partner of element j at distance D is
# j ^ D: in the lane at D = 64, across lanes below), the k-th largest key is
# read from lane k - 1, and ballots (counts of lanes below) give the ties to
# keep and every kept candidate's ascending position.  The model must keep the
# k largest keys with ties to the lower candidate id, candidate c = 2 lane + item.

def _wave_sort_desc(x):
    size = 2
    while size <= 128:
        dist = size // 2
        while dist > 0:
            if dist == 64:
                for ln in range(64):
                    a, b = x[0][ln], x[1][ln]
                    x[0][ln], x[1][ln] = max(a, b), min(a, b)
            else:
                new = [[0] * 64 for _ in range(2)]
                for t in range(2):
                    for ln in range(64):
                        j = t * 64 + ln
                        p = x[t][ln ^ dist]
                        take_max = ((j & size) == 0) == ((j & dist) == 0)
                        new[t][ln] = max(x[t][ln], p) if take_max else min(x[t][ln], p)
                x = new
            dist //= 2
        size *= 2
    return x


def _wave_select(keys, k):
    o = [[keys[2 * ln + t] for ln in range(64)] for t in range(2)]
    x = _wave_sort_desc([row[:] for row in o])
    flat = [x[j // 64][j % 64] for j in range(128)]
    assert flat == sorted(flat, reverse=True)
    thr = x[0][k - 1]

    def below(mask, ln):
        return bin(mask & ((1 << ln) - 1)).count("1")

    def ballot(pred):
        return sum(1 << ln for ln in range(64) if pred(ln))

    n_gt = bin(ballot(lambda ln: o[0][ln] > thr)).count("1") + bin(ballot(lambda ln: o[1][ln] > thr)).count("1")
    eq_take = k - n_gt
    e = [ballot(lambda ln, t=t: o[t][ln] == thr) for t in range(2)]
    kept = [[False] * 64 for _ in range(2)]
    for ln in range(64):
        eb0 = below(e[0], ln) + below(e[1], ln)
        eb1 = eb0 + (o[0][ln] == thr)
        kept[0][ln] = o[0][ln] > thr or (o[0][ln] == thr and eb0 < eq_take)
        kept[1][ln] = o[1][ln] > thr or (o[1][ln] == thr and eb1 < eq_take)
    p = [ballot(lambda ln, t=t: kept[t][ln]) for t in range(2)]
    out = [None] * k
    for ln in range(64):
        p0 = below(p[0], ln) + below(p[1], ln)
        if kept[0][ln]:
            out[p0] = 2 * ln
        if kept[1][ln]:
            out[p0 + kept[0][ln]] = 2 * ln + 1
    return out


@pytest.mark.parametrize("mode", ["distinct", "few_values", "all_equal"])
def test_one_wavefront_selection_model_keeps_the_top_k_ties_to_the_lower_id(mode):
    rng = np.random.default_rng({"distinct": 1, "few_values": 2, "all_equal": 3}[mode])
    for _ in range(300):
        k = int(rng.integers(1, 65))
        # every span has its left child (even id); some have a right child
        valid = [c % 2 == 0 and c < 2 * k or (c % 2 == 1 and c < 2 * k and rng.random() < 0.7) for c in range(128)]
        if mode == "distinct":
            keys = [int(rng.integers(0x00800000, 0xFF7FFFFF)) if v else 0 for v in valid]
        elif mode == "few_values":
            keys = [0x40000000 + int(rng.integers(0, 6)) if v else 0 for v in valid]
        else:
            keys = [0x3F800000 if v else 0 for v in valid]
        want = sorted(sorted((c for c in range(128) if valid[c]), key=lambda c: (-keys[c], c))[:k])
        assert _wave_select(keys, k) == want


def test_one_pass_is_taken_exactly_for_rows_one_workgroup_handles_alone():
    """The one-call decode step runs as one kernel for token-level rows with a single
    split and head chunk and 16- or 32-byte label rows, and as two kernels otherwise."""
    assert L.ds_decode_is_one_pass(16, 32, 32, 128, 32768, 1, 2048, 8)            # batched_32k: 512 rows
    assert L.ds_decode_is_one_pass(256, 32, 32, 128, 16384, 1, 1024, 16)          # 8,192 rows, r = 16
    assert L.ds_decode_is_one_pass(64, 256, 64, 128, 4096, 1, 200, 8)             # groups of 4: one chunk
    assert L.ds_decode_is_one_pass(128, 2, 2, 128, 5000, 1, 200, 4, "f32")        # fp32, 16-byte rows
    assert not L.ds_decode_is_one_pass(1, 32, 32, 128, 16384, 1, 1024, 16)        # 32 rows: eight splits each
    assert not L.ds_decode_is_one_pass(16, 32, 32, 128, 32768, 64, 32, 8)         # blocks
    assert not L.ds_decode_is_one_pass(16, 32, 32, 128, 32768, 1, 2048, 12)       # 24-byte label rows
    assert not L.ds_decode_is_one_pass(64, 512, 64, 128, 4096, 1, 100, 8)         # groups of 8: two head chunks
    assert not L.ds_decode_is_one_pass(64, 32, 32, 128, 131072, 1, 2048, 8)       # past the fused kernel's rows
    with pytest.raises(L.DsError):
        L.ds_decode_is_one_pass(1, 32, 32, 128, 16384, 1, 1024, 0)


def test_one_pass_needs_groups_of_one_two_or_four_heads():
    """Groups of 3 heads run as three one-head chunks, so they keep the two kernels."""
    assert L.ds_decode_is_one_pass(128, 8, 4, 128, 4096, 1, 100, 8)       # G = 2
    assert not L.ds_decode_is_one_pass(128, 12, 4, 128, 4096, 1, 100, 8)  # G = 3
