"""The span-search oracle's ranking precision against the GPU kernel's, on every input of the
span-search GPU tests (CPU only).

The oracle ranks the float64 group scores (HiP page, abstract: the top-k keys of the query);
the kernel ranks its double sums rounded to float32.  These tests show that on the GPU tests'
inputs the two precisions cannot choose different spans:

* a round tracer re-walks the oracle's search (its candidates and float64 scores), and must end
  on the oracle's spans;
* at every round's cut, every candidate either scores exactly the k-th largest score theta or
  lies outside the boundary-tie window |s - theta| <= 1e-6 |theta|.  Float32 rounding moves a
  score by at most 2^-24 relative, keeps exact ties exact, and so keeps every such cut;
* the oracle's search with its scores rounded to float32 gives the same spans.

The GPU tests then demand exact equality of the spans with the float64 oracle.
"""
import numpy as np
import pytest

import dsgen
import oracle as O
from _helpers import TIE_REL
from _hip_cases import HIP_CASES, TIE_KS, tie_periodic_K, ties_case


def _trace(q_group, K, T, k, span):
    """The oracle's rounds: returns (final spans, [(candidate scores, k) per round with a cut])."""
    spans = [(i * T // k, (i + 1) * T // k) for i in range(k)]
    cuts = []
    while any(e - s > span for s, e in spans):
        cand = []
        for s, e in spans:
            if e - s > span:
                m = s + (e - s + 1) // 2
                cand += [(s, m), (m, e)]
            else:
                cand.append((s, e))
        keys = np.asarray(O.group_token_scores(q_group, K, [s for s, _ in cand]), dtype=np.float64)
        order = np.argsort(-keys, kind="stable")
        cuts.append(keys)
        spans = [cand[i] for i in np.sort(order[:k])]
    return spans, cuts


def _cut_is_stable(keys, k):
    """Every candidate equals theta exactly or lies outside the tie window around it."""
    if len(keys) <= k:
        return True, 0.0
    theta = float(np.sort(keys)[::-1][k - 1])
    tol = TIE_REL * (abs(theta) if theta != 0 else float(np.max(np.abs(keys))))
    near = (np.abs(keys - theta) <= tol) & (keys != theta)
    off = np.abs(keys - theta)[keys != theta]
    return not near.any(), float(off.min() / max(abs(theta), 1e-300)) if len(off) else np.inf


def _as_float32_ranking(monkeypatch):
    exact = O.group_token_scores

    def rounded(q_group, K, tokens):
        return np.asarray(exact(q_group, K, tokens), dtype=np.float32).astype(np.float64)

    monkeypatch.setattr(O, "group_token_scores", rounded)


def _check_workload(w, monkeypatch, K_override=None):
    q, K, V = dsgen.gen_cache(w)
    del V
    if K_override is not None:
        K = K_override(K)
    worst = np.inf
    results = []
    for b in range(w.B):
        for g in range(w.Hkv):
            qg = dsgen.to_f64(q[b, g * w.G:(g + 1) * w.G], w.dtype)
            Kf = dsgen.to_f64(K[b, g, :w.T], w.dtype)
            spans = O.hip_search(qg, Kf, w.T, w.k_units, w.block)
            traced, cuts = _trace(qg, Kf, w.T, w.k_units, w.block)
            assert traced == spans, f"{w.name} ({b},{g}): tracer left the oracle's search"
            for r, keys in enumerate(cuts):
                ok, gap = _cut_is_stable(keys, w.k_units)
                assert ok, f"{w.name} ({b},{g}) round {r}: a candidate lies inside the tie window"
                worst = min(worst, gap)
            results.append(((b, g), qg, Kf, spans))
    with monkeypatch.context() as m:
        _as_float32_ranking(m)
        for (b, g), qg, Kf, spans in results:
            assert O.hip_search(qg, Kf, w.T, w.k_units, w.block) == spans, \
                f"{w.name} ({b},{g}): float32 ranking chose other spans"
    return worst


@pytest.mark.parametrize("w", HIP_CASES, ids=[w.name for w in HIP_CASES])
def test_span_search_ranking_is_stable_on_gpu_test_inputs(w, monkeypatch):
    gap = _check_workload(w, monkeypatch)
    print(f"{w.name}: smallest relative gap to a round's theta {gap:.3g}")


@pytest.mark.parametrize("k", TIE_KS)
def test_span_search_ranking_is_stable_with_exact_ties(k, monkeypatch):
    w = ties_case(k)
    _check_workload(w, monkeypatch, K_override=lambda K: tie_periodic_K(K, w.T))


@pytest.mark.slow
@pytest.mark.parametrize("name", dsgen.HIP_ORDER)
def test_span_search_ranking_is_stable_at_full_size(name, monkeypatch):
    """The one-million-token workload of the benchmark, every row."""
    gap = _check_workload(dsgen.get(name), monkeypatch)
    print(f"{name}: smallest relative gap to a round's theta {gap:.3g}")


def test_float32_ranking_differs_from_float64_on_a_near_tie():
    """The pin above is not vacuous: two first tokens scoring 2^24 and 2^24 + 1 are one apart in
    float64 and equal in float32, so float64 ranking keeps the higher score and float32 ranking the
    lower start."""
    K = np.zeros((4, 4))
    K[0, 0], K[2, 0] = 2.0 ** 24, 2.0 ** 24 + 1
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    assert O.hip_search(q, K, 4, 1, 2) == [(2, 4)]
    keys = np.asarray(O.group_token_scores(q, K, [0, 2]), dtype=np.float32)
    assert keys[0] == keys[1]
