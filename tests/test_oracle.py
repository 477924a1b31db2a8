"""Pins for the CPU oracle (no GPU).

Each check ties an oracle function to something other than itself: brute force
with exact (fsum) sums on tiny inputs, a library routine (torch's fp64
scaled_dot_product_attention), closed forms, invariants, planted structure in
the synthetic workloads, and a hand-worked fixture.  The mutation tests at the
end plant plausible mistakes in a copy of the oracle and check that some pin
catches each one.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import dsgen
import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _ns(**override):
    ns = types.SimpleNamespace(**{k: getattr(O, k) for k in O.__all__})
    for k, v in override.items():
        setattr(ns, k, v)
    return ns


# ---------------------------------------------------------------- brute force helpers

def brute_rank_select(u, k):
    """Index t is kept iff fewer than k indices beat it (larger, or equal with a lower id)."""
    n = len(u)
    keep = []
    for t in range(n):
        beat = sum(1 for s in range(n) if u[s] > u[t] or (u[s] == u[t] and s < t))
        if beat < k:
            keep.append(t)
    return keep


def brute_importance(q_cal, k_cal, g, G):
    n_q, Hq, d = q_cal.shape
    n_k = k_cal.shape[1]
    out = []
    for c in range(d):
        tot = math.fsum(abs(float(q_cal[n, h, c])) * abs(float(k_cal[g, m, c]))
                        for n in range(n_q) for h in range(g * G, (g + 1) * G) for m in range(n_k))
        out.append(tot / (n_q * G * n_k))
    return out


def brute_label_score(q_group, K, ch, t):
    return math.fsum(float(q_group[h, c]) * float(K[t, c]) for h in range(q_group.shape[0]) for c in ch)


# ---------------------------------------------------------------- checks (shared with mutation tests)

def check_calibration_brute(ns, seed=0):
    rng = np.random.default_rng(seed)
    n_q, n_k, Hq, Hkv, d = 5, 7, 4, 2, 9
    q = rng.standard_normal((n_q, Hq, d))
    k = rng.standard_normal((Hkv, n_k, d))
    G = Hq // Hkv
    for r in (1, 3, 9):
        got = ns.calibrate_channels(q, k, Hkv, r)
        for g in range(Hkv):
            want = brute_rank_select(brute_importance(q, k, g, G), r)
            assert list(got[g]) == want, (r, g, list(got[g]), want)


def check_calibration_ties(ns):
    q = np.ones((3, 2, 8))
    k = np.ones((1, 4, 8))
    for r in (1, 5, 8):
        assert list(ns.calibrate_channels(q, k, 1, r)[0]) == list(range(r))
    # channels 2 and 6 tie for the top; 0 and 4 tie for third
    k2 = np.ones((1, 4, 8))
    k2[0, :, 2] = k2[0, :, 6] = 5.0
    k2[0, :, 0] = k2[0, :, 4] = 3.0
    assert list(ns.calibrate_channels(q, k2, 1, 3)[0]) == [0, 2, 6]


def check_label_gather(ns):
    K = np.arange(70, dtype=np.float64).reshape(7, 10)
    ch = np.array([1, 4, 9])
    L = ns.label_rows(K, ch)
    for t in range(7):
        for j, c in enumerate(ch):
            assert L[t, j] == 10 * t + c


def check_scores_brute(ns, seed=1):
    rng = np.random.default_rng(seed)
    G, d, T = 3, 16, 20
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    for ch in (np.arange(d), np.array([0, 5, 6, 11]), np.array([15])):
        u = ns.label_scores(q, ns.label_rows(K, ch), ch)
        want = [brute_label_score(q, K, ch, t) for t in range(T)]
        np.testing.assert_allclose(u, want, rtol=0, atol=1e-12)


def check_block_max_brute(ns, seed=2):
    rng = np.random.default_rng(seed)
    for T, b in ((100, 64), (128, 64), (7, 3), (5, 1)):
        u = rng.standard_normal(T)
        got = ns.block_scores(u, b)
        want = []
        for s in range(0, T, b):
            m = -math.inf
            for t in range(s, min(s + b, T)):
                m = u[t] if u[t] > m else m
            want.append(m)
        assert list(got) == want


def check_select_brute(ns, seed=3):
    rng = np.random.default_rng(seed)
    for n in (1, 2, 17, 40):
        u = rng.integers(-3, 4, size=n).astype(np.float64)   # many exact ties
        for k in sorted({1, n // 3 + 1, n // 2 + 1, n}):
            assert list(ns.select_topk(u, k)) == brute_rank_select(list(u), k), (n, k)


def _sdpa(q_group, K, V, S, scale):
    """torch's fp64 scaled_dot_product_attention with a boolean mask keeping S."""
    G, d = q_group.shape
    T = K.shape[0]
    mask = torch.zeros((1, 1, 1, T), dtype=torch.bool)
    mask[..., torch.as_tensor(np.asarray(S))] = True
    qt = torch.as_tensor(q_group, dtype=torch.float64).reshape(1, G, 1, d)
    kt = torch.as_tensor(K, dtype=torch.float64).reshape(1, 1, T, d).expand(1, G, T, d).contiguous()
    vt = torch.as_tensor(V, dtype=torch.float64).reshape(1, 1, T, d).expand(1, G, T, d).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.reshape(G, d).numpy()


def check_attend_sdpa(ns, seed=4):
    rng = np.random.default_rng(seed)
    G, d, T = 4, 32, 50
    q = rng.standard_normal((G, d)) * 2
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    for S in (np.arange(T), np.array([3]), np.sort(rng.choice(T, 13, replace=False))):
        np.testing.assert_allclose(ns.attend(q, K, V, S, scale), _sdpa(q, K, V, S, scale),
                                   rtol=0, atol=1e-12)


def check_split_merge(ns, seed=5):
    rng = np.random.default_rng(seed)
    G, d, T = 2, 8, 40
    q = rng.standard_normal((G, d)) * 3
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    S = np.sort(rng.choice(T, 23, replace=False))
    whole = ns.attend(q, K, V, S, 0.5)
    for parts in (1, 2, 5, 23):
        cuts = np.sort(rng.choice(np.arange(1, len(S)), parts - 1, replace=False)) if parts > 1 else []
        pieces = np.split(S, cuts)
        merged = ns.merge_partials([ns.attend_partial(q, K, V, p, 0.5) for p in pieces])
        np.testing.assert_allclose(merged, whole, rtol=0, atol=1e-12)


def check_golden(ns):
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        gold = json.load(f)
    cal = gold["calibration"]
    qc = np.array(cal["q_cal"], dtype=np.float64)
    kc = np.array(cal["k_cal"], dtype=np.float64)
    for r, want in cal["expected"].items():
        assert list(ns.calibrate_channels(qc, kc, 1, int(r))[0]) == want
    dec = gold["decode"]
    K = np.array(dec["K"], dtype=np.float64)
    V = np.array(dec["V"], dtype=np.float64)
    ch = np.array(dec["channels"])
    scale = 1 / math.sqrt(dec["d"])
    T = K.shape[0]
    for case in dec["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        u = ns.label_scores(q, ns.label_rows(K, ch), ch)
        if case["block"] == 1:
            kept = ns.select_topk(u, case["k_units"])
            S = kept
        else:
            kept = ns.select_topk(ns.block_scores(u, case["block"]), case["k_units"])
            S = ns.blocks_to_tokens(kept, case["block"], T)
        assert list(kept) == case["kept"], case["why"]
        np.testing.assert_allclose(ns.attend(q, K, V, S, scale), np.array(case["out"]),
                                   rtol=0, atol=1e-12, err_msg=case["why"])


def brute_positive_score(q_group, K, ch, t):
    return math.fsum(max(0.0, math.fsum(float(q_group[h, c]) * float(K[t, c]) for c in ch))
                     for h in range(q_group.shape[0]))


def brute_threshold_select(u, tau, k):
    """Units at or above tau; past k of them, the ones fewer than k passing units beat."""
    passing = [t for t in range(len(u)) if u[t] >= tau]
    if len(passing) <= k:
        return passing
    keep = []
    for t in passing:
        beat = sum(1 for s in passing if u[s] > u[t] or (u[s] == u[t] and s < t))
        if beat < k:
            keep.append(t)
    return keep


def check_positive_scores_brute(ns, seed=7):
    rng = np.random.default_rng(seed)
    G, d, T = 3, 16, 25
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    for ch in (np.arange(d), np.array([0, 5, 6, 11]), np.array([15])):
        u = ns.label_scores_positive(q, ns.label_rows(K, ch), ch)
        want = [brute_positive_score(q, K, ch, t) for t in range(T)]
        np.testing.assert_allclose(u, want, rtol=0, atol=1e-12)


def check_threshold_select_brute(ns, seed=8):
    rng = np.random.default_rng(seed)
    for n in (1, 2, 17, 40):
        u = rng.integers(-3, 4, size=n).astype(np.float64)   # many exact ties, and scores equal to tau
        for tau in (-math.inf, -3.0, -0.5, 0.0, 1.0, 2.5, 3.0, 4.0):
            for k in sorted({1, n // 3 + 1, n // 2 + 1, n, n + 3}):
                got = list(ns.select_threshold(u, tau, k))
                assert got == brute_threshold_select(list(u), tau, k), (n, tau, k, got)


def _golden_threshold():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        gold = json.load(f)
    dec = gold["decode"]
    return (gold["threshold"], np.array(dec["K"], dtype=np.float64), np.array(dec["V"], dtype=np.float64),
            np.array(dec["channels"]), 1 / math.sqrt(dec["d"]))


def check_golden_threshold(ns):
    """The threshold cases, step by step through the namespace's functions."""
    gold, K, V, ch, scale = _golden_threshold()
    T = K.shape[0]
    for case in gold["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        u = ns.label_scores_positive(q, ns.label_rows(K, ch), ch)
        scores = u if case["block"] == 1 else ns.block_scores(u, case["block"])
        assert list(scores) == case["scores"], case["why"]
        kept = ns.select_threshold(scores, case["tau"], case["k_max"])
        assert list(kept) == case["kept"], case["why"]
        if case["out"] is not None:
            S = ns.tokens_of(kept, case["block"], T)
            out = ns.attend(q, K, V, S, scale) if len(S) else np.zeros((q.shape[0], K.shape[1]))
            np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12, err_msg=case["why"])


def check_golden_threshold_unit(ns):
    """The same cases through the one-call decode of a unit."""
    gold, K, V, ch, scale = _golden_threshold()
    for case in gold["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        out, kept, scores = ns.decode_unit_threshold(q, K, V, ch, case["k_max"], case["tau"], case["block"], scale)
        assert list(kept) == case["kept"] and list(scores) == case["scores"], case["why"]
        assert np.all(np.isfinite(out)), case["why"]
        if case["out"] is not None:
            np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12, err_msg=case["why"])


def _hip_K(case):
    """K [T, 4] from the fixture's column formulas of the token position t."""
    T = case["T"]
    t = np.arange(T, dtype=np.float64)
    forms = {"t": t, "-t": -t, "-2t": -2 * t, "-|t-37|": -np.abs(t - 37)}
    K = np.zeros((T, 4))
    for col, f in case["K_col"].items():
        K[:, int(col)] = forms[f]
    return K


def check_golden_hip(ns):
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        gold = json.load(f)["hierarchical"]
    for case in gold["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        got = [list(sp) for sp in ns.hip_search(q, _hip_K(case), case["T"], case["k"], case["span"])]
        assert got == case["spans"], (case["why"], got)


def check_hip_structure(ns, seed=13):
    """Random inputs: k disjoint ascending spans, each inside one of the first even spans, none
    longer than `span` (or the first spans themselves when no round runs), and rising scores
    keep the k rightmost spans of the last level when T, k and span are powers of two."""
    rng = np.random.default_rng(seed)
    for T, k, span, G in ((97, 5, 3, 2), (1000, 16, 8, 1), (4096, 32, 16, 4), (64, 64, 1, 1)):
        q = rng.standard_normal((G, 8))
        K = rng.standard_normal((T, 8))
        spans = ns.hip_search(q, K, T, k, span)
        assert len(spans) == k
        first = [(i * T // k, (i + 1) * T // k) for i in range(k)]
        no_round = max(e - s for s, e in first) <= span
        for i, (s, e) in enumerate(spans):
            assert 0 <= s < e <= T and (i == 0 or spans[i - 1][1] <= s)
            assert any(fs <= s and e <= fe for fs, fe in first)
            assert (s, e) in first if no_round else e - s <= span
    for T, k, span in ((256, 4, 8), (1024, 8, 4)):
        K = np.zeros((T, 2))
        K[:, 0] = np.cumsum(rng.random(T) + 0.1)   # strictly rising scores
        spans = ns.hip_search(np.array([[1.0, 0.0]]), K, T, k, span)
        assert spans == [(T - (k - i) * span, T - (k - i - 1) * span) for i in range(k)]


# ---------------------------------------------------------------- pins

def test_calibration_matches_all_pairs_brute_force():
    check_calibration_brute(O)


def test_calibration_ties_go_to_lower_channel():
    check_calibration_ties(O)


@pytest.mark.parametrize("name", dsgen.WORKLOAD_ORDER)
def test_calibration_recovers_planted_outliers(name):
    """The planted x6 channels dominate mean|q_c|*mean|k_c| by a wide margin, so r >= 8
    label channels must contain them and r == 8 must equal them."""
    w = dsgen.get(name)
    qc, kc = dsgen.gen_calib(w)
    ch = O.calibrate_channels(qc, kc, w.Hkv, w.r)
    planted = dsgen.outlier_channels(w)
    for g in range(w.Hkv):
        assert set(planted[g]) <= set(ch[g])
        assert list(ch[g]) == sorted(ch[g])
        if w.r == w.n_outliers:
            assert list(ch[g]) == list(planted[g])


def test_label_is_identity_gather():
    check_label_gather(O)


def test_label_scores_match_exact_brute_force():
    check_scores_brute(O)


def test_label_scores_channel_order_and_head_additivity():
    rng = np.random.default_rng(6)
    G, d, T = 4, 24, 33
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    ch = np.array([2, 3, 7, 19, 20])
    u = O.label_scores(q, O.label_rows(K, ch), ch)
    perm = ch[[3, 0, 4, 1, 2]]
    np.testing.assert_allclose(O.label_scores(q, O.label_rows(K, perm), perm), u, rtol=0, atol=1e-12)
    # GQA: the group's score is the sum of the single-head (MHA, G = 1) scores
    heads = sum(O.label_scores(q[h:h + 1], O.label_rows(K, ch), ch) for h in range(G))
    np.testing.assert_allclose(heads, u, rtol=0, atol=1e-12)


def test_block_max_matches_brute_force():
    check_block_max_brute(O)


def test_select_matches_rank_counting_with_ties():
    check_select_brute(O)


def test_r_equals_d_selects_exact_topk_of_true_scores():
    """With every channel as a label channel, identification is exact: the kept set is the
    top-k of the true q.k (summed over the group), by exact brute force."""
    rng = np.random.default_rng(7)
    G, d, T, k = 2, 16, 60, 9
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    _, kept, _ = O.decode_unit(q, K, V, np.arange(d), k)
    true = [math.fsum(float(q[h, c]) * float(K[t, c]) for h in range(G) for c in range(d)) for t in range(T)]
    assert list(kept) == brute_rank_select(true, k)


def test_k_equals_T_is_dense_attention():
    rng = np.random.default_rng(8)
    G, d, T = 3, 32, 64
    q = rng.standard_normal((G, d)) * 2
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    out, kept, _ = O.decode_unit(q, K, V, np.array([0, 1, 2, 3]), T)
    assert list(kept) == list(range(T))
    np.testing.assert_allclose(out, _sdpa(q, K, V, np.arange(T), 1 / math.sqrt(d)), rtol=0, atol=1e-12)


def test_attention_matches_torch_sdpa():
    check_attend_sdpa(O)


def test_weights_sum_to_one_and_output_is_convex_combination():
    rng = np.random.default_rng(9)
    G, d, T = 4, 16, 80
    q = rng.standard_normal((G, d)) * 4
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    S = np.sort(rng.choice(T, 20, replace=False))
    w = O.attention_weights(q, K, S, 0.25)
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    out = O.attend(q, K, V, S, 0.25)
    lo, hi = V[S].min(axis=0), V[S].max(axis=0)
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)


def test_block_variant_special_cases():
    rng = np.random.default_rng(10)
    G, d, T = 2, 16, 100
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    ch = np.array([1, 5, 9])
    # block = 1 is the token variant
    o1, k1, s1 = O.decode_unit(q, K, V, ch, 10, block=1)
    np.testing.assert_array_equal(O.block_scores(s1, 1), s1)
    np.testing.assert_array_equal(O.select_topk(O.block_scores(s1, 1), 10), k1)
    # keeping every block is dense attention, including the partial last block (100 = 64 + 36)
    od, kd, sd = O.decode_unit(q, K, V, ch, 2, block=64)
    assert list(kd) == [0, 1] and len(sd) == 2
    np.testing.assert_allclose(od, _sdpa(q, K, V, np.arange(T), 0.25), rtol=0, atol=1e-12)
    assert list(O.blocks_to_tokens(np.array([1]), 64, T)) == list(range(64, 100))


def test_split_merge_is_partition_invariant():
    check_split_merge(O)


def test_hand_worked_fixture():
    check_golden(O)


def test_decode_unit_on_workload_slice():
    """One full-length unit of the headline workload: the kept set has k distinct ascending
    ids, and exact identification (r = d) keeps more of the true top-k than the r = 16 labels,
    which in turn beat the k/T recall of random pruning by a wide margin."""
    w = dsgen.get("llama7b_16k")
    K, V, q = dsgen.gen_unit(w, 0, 3)
    K, V, q = dsgen.to_f64(K, w.dtype), dsgen.to_f64(V, w.dtype), dsgen.to_f64(q, w.dtype)
    qc, kc = dsgen.gen_calib(w)
    ch = O.calibrate_channels(qc, kc, w.Hkv, w.r)[3]
    out, kept, u = O.decode_unit(q, K, V, ch, w.k_units)
    assert len(kept) == w.k_units and np.all(np.diff(kept) > 0)
    _, exact, _ = O.decode_unit(q, K, V, np.arange(w.d), w.k_units)
    recall = len(set(kept) & set(exact)) / w.k_units
    assert recall > 4 * w.k_units / w.T
    assert np.all(np.isfinite(out))


def test_positive_scores_match_exact_brute_force():
    check_positive_scores_brute(O)


def test_positive_scores_bounds_and_special_cases():
    """u+ is at least the signed group score and at least every single head's clipped score;
    with one query head it is the clipped signed score; with every head's score of one sign it
    is the signed score (all positive) or zero (all negative)."""
    rng = np.random.default_rng(9)
    G, d, T = 4, 20, 30
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    ch = np.array([1, 2, 3, 8, 13, 19])
    L = O.label_rows(K, ch)
    up = O.label_scores_positive(q, L, ch)
    assert np.all(up >= O.label_scores(q, L, ch) - 1e-12) and np.all(up >= 0)
    for h in range(G):
        assert np.all(up >= np.maximum(O.label_scores(q[h:h + 1], L, ch), 0) - 1e-12)
    np.testing.assert_allclose(O.label_scores_positive(q[:1], L, ch), np.maximum(O.label_scores(q[:1], L, ch), 0),
                               rtol=0, atol=1e-12)
    qa, Ka = np.abs(q), np.abs(K)
    La = O.label_rows(Ka, ch)
    np.testing.assert_allclose(O.label_scores_positive(qa, La, ch), O.label_scores(qa, La, ch), rtol=0, atol=1e-12)
    assert np.all(O.label_scores_positive(-qa, La, ch) == 0)


def test_threshold_select_matches_brute_force_with_ties():
    check_threshold_select_brute(O)


def test_threshold_select_special_cases():
    """tau below every score is plain top-k; tau above every score keeps nothing; a cap at or
    above the unit count keeps exactly the units at or above tau; with no cap, raising tau
    never adds a unit."""
    rng = np.random.default_rng(10)
    u = rng.standard_normal(200)
    for k in (1, 17, 200):
        assert list(O.select_threshold(u, -math.inf, k)) == list(O.select_topk(u, k))
        assert len(O.select_threshold(u, u.max() + 1, k)) == 0
    for tau in (-1.0, 0.0, 0.7):
        assert list(O.select_threshold(u, tau, 200)) == list(np.flatnonzero(u >= tau))
    prev = set(range(200))
    for tau in np.linspace(-3, 3, 25):
        cur = set(O.select_threshold(u, tau, 200))
        assert cur <= prev
        prev = cur


def test_threshold_hand_worked_fixture():
    check_golden_threshold(O)
    check_golden_threshold_unit(O)


def test_threshold_decode_reduces_to_topk_on_positive_scores():
    """With tau = -inf the threshold decode is the top-k decode run on the positive-only scores."""
    rng = np.random.default_rng(11)
    G, d, T = 4, 32, 300
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    ch = np.array([0, 3, 9, 10, 22, 31])
    for block, k in ((1, 40), (16, 5)):
        out, kept, scores = O.decode_unit_threshold(q, K, V, ch, k, -math.inf, block)
        u = O.label_scores_positive(q, O.label_rows(K, ch), ch)
        U = u if block == 1 else O.block_scores(u, block)
        want = O.select_topk(U, k)
        assert list(kept) == list(want)
        np.testing.assert_allclose(out, O.attend(q, K, V, O.tokens_of(want, block, T), O.default_scale(d)),
                                   rtol=0, atol=1e-12)


def test_hip_search_hand_worked_fixture():
    check_golden_hip(O)


def test_hip_search_structure_and_monotone_closed_form():
    check_hip_structure(O)


def check_hip_near_tie(ns):
    """Two first tokens scoring 2^24 and 2^24 + 1 (equal once rounded to float32): the search ranks
    the exact scores, so the higher one wins although the other starts lower."""
    K = np.zeros((4, 4))
    K[0, 0], K[2, 0] = 2.0 ** 24, 2.0 ** 24 + 1
    assert [tuple(sp) for sp in ns.hip_search(np.array([[1.0, 0.0, 0.0, 0.0]]), K, 4, 1, 2)] == [(2, 4)]


def test_hip_search_ranks_exact_scores():
    check_hip_near_tie(O)


def check_group_scores(ns, seed=14):
    """Group score = the sum over heads of q_h . K_t in float64, within a few float64 roundings of
    the exact sum (brute force with fsum)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((3, 16))
    K = rng.standard_normal((40, 16))
    toks = [0, 5, 39, 17]
    got = np.asarray(ns.group_token_scores(q, K, toks))
    assert got.dtype == np.float64
    for t, v in zip(toks, got):
        terms = [float(q[h, c]) * float(K[t, c]) for h in range(3) for c in range(16)]
        bound = 64 * 2.0 ** -53 * math.fsum(abs(x) for x in terms)
        assert abs(float(v) - math.fsum(terms)) <= bound, (t, v)


def test_hip_group_scores_are_the_float64_dot():
    check_group_scores(O)


def test_hip_decode_without_rounds_is_dense_attention():
    """When the first k spans are no longer than `span`, every token is kept: dense attention."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((2, 32))
    K = rng.standard_normal((100, 32))
    V = rng.standard_normal((100, 32))
    out, spans = O.decode_unit_hip(q, K, V, 10, 10)
    np.testing.assert_allclose(out, O.attend(q, K, V, np.arange(100), O.default_scale(32)), rtol=0, atol=1e-12)
    assert list(O.spans_to_tokens(spans)) == list(range(100))


# ---------------------------------------------------------------- planted mistakes

def _mut_calib_sum_not_product(q_cal, k_cal, Hkv, r):
    q = np.asarray(q_cal, np.float64); k = np.asarray(k_cal, np.float64)
    G = q.shape[1] // Hkv
    out = np.empty((Hkv, r), np.int32)
    for g in range(Hkv):
        s = np.abs(q[:, g * G:(g + 1) * G]).mean(axis=(0, 1)) + np.abs(k[g]).mean(axis=0)
        out[g] = np.sort(np.argsort(-s, kind="stable")[:r])
    return out


def _mut_calib_ties_high(q_cal, k_cal, Hkv, r):
    q = np.asarray(q_cal, np.float64); k = np.asarray(k_cal, np.float64)
    G = q.shape[1] // Hkv
    out = np.empty((Hkv, r), np.int32)
    for g in range(Hkv):
        s = np.abs(q[:, g * G:(g + 1) * G]).mean(axis=(0, 1)) * np.abs(k[g]).mean(axis=0)
        d = len(s)
        order = d - 1 - np.argsort(-s[::-1], kind="stable")
        out[g] = np.sort(order[:r])
    return out


def _mut_label_wrong_index(K, ch):
    return np.asarray(K)[:, np.asarray(ch) - 1]


def _mut_scores_one_head(q_group, L, ch):
    return np.asarray(L, np.float64) @ np.asarray(q_group, np.float64)[0, np.asarray(ch)]


def _mut_scores_dropped_term(q_group, L, ch):
    qs = np.asarray(q_group, np.float64)[:, np.asarray(ch)]
    return (np.asarray(L, np.float64)[:, :-1] @ qs[:, :-1].T).sum(axis=1) if len(ch) > 1 else \
        (np.asarray(L, np.float64) @ qs.T).sum(axis=1) * 0


def _mut_block_mean(u, block):
    u = np.asarray(u, np.float64)
    nb = -(-len(u) // block)
    return np.array([u[i * block:(i + 1) * block].mean() for i in range(nb)])


def _mut_select_ties_high(u, k):
    u = np.asarray(u, np.float64)
    order = len(u) - 1 - np.argsort(-u[::-1], kind="stable")
    return np.sort(order[:k])


def _mut_select_smallest(u, k):
    return np.sort(np.argsort(np.asarray(u), kind="stable")[:k])


def _mut_attend_no_scale(q_group, K, V, S, scale):
    return O.attend(q_group, K, V, S, 1.0)


def _mut_attend_transposed(q_group, K, V, S, scale):
    z = np.asarray(q_group) @ np.asarray(V)[S].T * scale     # K and V swapped
    w = np.exp(z - z.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(K)[S]


def _mut_merge_no_rescale(parts):
    l = sum(p[1] for p in parts)
    return sum(p[2] for p in parts) / l[:, None]


def _mut_pos_signed(q_group, L, ch):
    return O.label_scores(q_group, L, ch)


def _mut_pos_clip_after_sum(q_group, L, ch):
    return np.maximum(O.label_scores(q_group, L, ch), 0.0)


def _mut_pos_abs(q_group, L, ch):
    qs = np.asarray(q_group, np.float64)[:, np.asarray(ch)]
    return np.abs(np.asarray(L, np.float64) @ qs.T).sum(axis=1)


def _mut_thr_strict(u, tau, k_max):
    u = np.asarray(u, np.float64)
    p = np.flatnonzero(u > tau)
    return p if len(p) <= k_max else np.sort(p[np.argsort(-u[p], kind="stable")][:k_max])


def _mut_thr_cap_lowest_ids(u, tau, k_max):
    p = np.flatnonzero(np.asarray(u, np.float64) >= tau)
    return p[:k_max]


def _mut_thr_cap_ties_high(u, tau, k_max):
    u = np.asarray(u, np.float64)
    p = np.flatnonzero(u >= tau)
    if len(p) <= k_max:
        return p
    rev = p[::-1]
    return np.sort(rev[np.argsort(-u[rev], kind="stable")][:k_max])


def _mut_thr_no_cap(u, tau, k_max):
    return np.flatnonzero(np.asarray(u, np.float64) >= tau)


def _mut_thr_topk_only(u, tau, k_max):
    return O.select_topk(u, min(k_max, len(u)))


def _mut_unit_empty_nan(q_group, K, V, ch, k_max, tau, block=1, scale=None, T=None):
    K = np.asarray(K, np.float64)
    T = K.shape[0] if T is None else T
    scale = O.default_scale(K.shape[1]) if scale is None else scale
    u = O.label_scores_positive(q_group, O.label_rows(K[:T], ch), ch)
    scores = u if block == 1 else O.block_scores(u, block)
    kept = O.select_threshold(scores, tau, k_max)
    S = O.tokens_of(kept, block, T)
    G = np.asarray(q_group).shape[0]
    out = O.attend(q_group, K[:T], np.asarray(V)[:T], S, scale) if len(S) else np.full((G, K.shape[1]), np.nan)
    return out, kept, scores


def _hip_variant(ties_high=False, floor_left=False, last_rep=False, extra=0, early_stop=False, f32=False):
    def search(q_group, K, T, k, span):
        spans = [(i * T // k, (i + 1) * T // k) for i in range(k)]
        rep = (lambda s, e: e - 1) if last_rep else (lambda s, e: s)
        while any(e - s > (2 * span if early_stop else span) for s, e in spans):
            cand = []
            for s, e in spans:
                if e - s > span:
                    m = s + ((e - s) // 2 if floor_left else (e - s + 1) // 2)
                    cand += [(s, m), (m, e)]
                else:
                    cand.append((s, e))
            keys = np.asarray(O.group_token_scores(q_group, K, [rep(s, e) for s, e in cand]),
                              dtype=np.float32 if f32 else np.float64).astype(np.float64)
            idx = np.arange(len(cand))
            order = (idx[::-1][np.argsort(-keys[::-1], kind="stable")] if ties_high
                     else np.argsort(-keys, kind="stable"))
            spans = [cand[i] for i in np.sort(order[:k + extra])]
        return spans
    return search


def _mut_hip_one_head(q_group, K, tokens):
    return O.group_token_scores(np.asarray(q_group)[:1], K, tokens)


MUTANTS = [
    ("hip_search", _hip_variant(ties_high=True), check_golden_hip),
    ("hip_search", _hip_variant(floor_left=True), check_golden_hip),
    ("hip_search", _hip_variant(last_rep=True), check_golden_hip),
    ("hip_search", _hip_variant(extra=1), check_hip_structure),
    ("hip_search", _hip_variant(early_stop=True), check_hip_structure),
    ("hip_search", _hip_variant(f32=True), check_hip_near_tie),
    ("group_token_scores", _mut_hip_one_head, check_group_scores),
    ("label_scores_positive", _mut_pos_signed, check_positive_scores_brute),
    ("label_scores_positive", _mut_pos_clip_after_sum, check_positive_scores_brute),
    ("label_scores_positive", _mut_pos_abs, check_positive_scores_brute),
    ("select_threshold", _mut_thr_strict, check_threshold_select_brute),
    ("select_threshold", _mut_thr_cap_lowest_ids, check_threshold_select_brute),
    ("select_threshold", _mut_thr_cap_ties_high, check_threshold_select_brute),
    ("select_threshold", _mut_thr_no_cap, check_threshold_select_brute),
    ("select_threshold", _mut_thr_topk_only, check_threshold_select_brute),
    ("decode_unit_threshold", _mut_unit_empty_nan, check_golden_threshold_unit),
    ("calibrate_channels", _mut_calib_sum_not_product, check_calibration_brute),
    ("calibrate_channels", _mut_calib_ties_high, check_calibration_ties),
    ("label_rows", _mut_label_wrong_index, check_label_gather),
    ("label_scores", _mut_scores_one_head, check_scores_brute),
    ("label_scores", _mut_scores_dropped_term, check_scores_brute),
    ("block_scores", _mut_block_mean, check_block_max_brute),
    ("select_topk", _mut_select_ties_high, check_select_brute),
    ("select_topk", _mut_select_smallest, check_select_brute),
    ("attend", _mut_attend_no_scale, check_attend_sdpa),
    ("attend", _mut_attend_transposed, check_attend_sdpa),
    ("merge_partials", _mut_merge_no_rescale, check_split_merge),
]


@pytest.mark.parametrize("fn,mutant,check", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(fn, mutant, check):
    with pytest.raises(AssertionError):
        check(_ns(**{fn: mutant}))


GOLDEN_MUTANTS = [
    ("calibrate_channels", _mut_calib_sum_not_product),
    ("calibrate_channels", _mut_calib_ties_high),
    ("label_rows", _mut_label_wrong_index),
    ("label_scores", _mut_scores_one_head),
    ("label_scores", _mut_scores_dropped_term),
    ("block_scores", _mut_block_mean),
    ("select_topk", _mut_select_ties_high),
    ("select_topk", _mut_select_smallest),
    ("attend", _mut_attend_transposed),
]


THRESHOLD_GOLDEN_MUTANTS = [
    ("label_scores_positive", _mut_pos_signed),
    ("label_scores_positive", _mut_pos_clip_after_sum),
    ("label_scores_positive", _mut_pos_abs),
    ("select_threshold", _mut_thr_strict),
    ("select_threshold", _mut_thr_cap_lowest_ids),
    ("select_threshold", _mut_thr_cap_ties_high),
    ("select_threshold", _mut_thr_no_cap),
    ("select_threshold", _mut_thr_topk_only),
    ("block_scores", _mut_block_mean),
]


@pytest.mark.parametrize("fn,mutant", THRESHOLD_GOLDEN_MUTANTS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in THRESHOLD_GOLDEN_MUTANTS])
def test_threshold_fixture_catches_planted_mistake(fn, mutant):
    with pytest.raises(AssertionError):
        check_golden_threshold(_ns(**{fn: mutant}))


@pytest.mark.parametrize("fn,mutant", GOLDEN_MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in GOLDEN_MUTANTS])
def test_hand_worked_fixture_catches_planted_mistake(fn, mutant):
    with pytest.raises(AssertionError):
        check_golden(_ns(**{fn: mutant}))
