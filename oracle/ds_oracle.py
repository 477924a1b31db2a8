"""CPU oracle for the Double Sparsity decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Plain numpy in float64.  It follows the method step by step, in the order the
Double Sparsity page describes it (method details: offline calibration of a
static channel-sparsity pattern, then online selection of the important
tokens, then self-attention over those tokens only), not a fused or blocked
reformulation.  Inputs are the already-rounded stored values, widened exactly
to float64 by the caller.

Where the pages leave a step open, the reading taken is:
  * calibration score of channel c for KV head g: mean over the calibration
    queries of the group's query heads of |q_c|, times the mean over the
    calibration keys of |k_c| (the mean of |q_c|*|k_c| over all query/key
    pairs, which factorises into this product); keep the r largest, lower
    channel id first on ties, return ids ascending;
  * label score: sum over the r label channels and over the group's query
    heads of q_c * K_c, with no scale (a positive scale cannot change a
    ranking);
  * block score: the maximum label score over the tokens of the block that
    exist;
  * selection: the k largest scores, lower index first on ties, returned in
    ascending index order;
  * attention: softmax of q.K / sqrt(d) over the selected tokens only, no
    forced sink or recent tokens, no causal mask (a decode query sees all T).

The threshold rule (Jenga page, core method item 1) is read as follows:
  * a token's informativeness is the sum over the group's query heads of the
    head's label score, counting only the heads whose score is positive; with
    one decode query, the sum over the other queries of the page's definition
    is that query's score, and the query's own (just appended) key is scored
    like every other;
  * a block's informativeness is the maximum over its tokens, as above;
  * a unit is kept when its informativeness is at least the threshold; when
    more than k_max units pass, the k_max largest of them are kept (lower
    index first on ties);
  * with no unit kept, the attention output is zero.
"""
from __future__ import annotations

import math

import numpy as np


# -- offline stage ----------------------------------------------------------

def calibrate_channels(q_cal: np.ndarray, k_cal: np.ndarray, Hkv: int, r: int) -> np.ndarray:
    """Static label channels per KV head, [Hkv, r] int32, ascending.

    Double Sparsity page, method details and abstract: the channel-sparsity
    pattern is nearly static, so it is fixed offline from a small calibration
    set and reused at run time.  The page does not give the calibration rule;
    the rule used is the importance mean|q_c| * mean|k_c|, pooled over the
    query heads that share KV head g.

    q_cal: [n_q, Hq, d]; k_cal: [Hkv, n_k, d].
    """
    q = np.asarray(q_cal, dtype=np.float64)
    k = np.asarray(k_cal, dtype=np.float64)
    n_q, Hq, d = q.shape
    if Hq % Hkv or not (1 <= r <= d):
        raise ValueError("bad calibration shape")
    G = Hq // Hkv
    out = np.empty((Hkv, r), dtype=np.int32)
    for g in range(Hkv):
        a = np.abs(q[:, g * G:(g + 1) * G, :]).mean(axis=(0, 1))   # [d]
        b = np.abs(k[g]).mean(axis=0)                                # [d]
        importance = a * b
        order = np.argsort(-importance, kind="stable")                # ties: lower c first
        out[g] = np.sort(order[:r])
    return out


# -- online stage: identification through label channels --------------------

def label_rows(K: np.ndarray, ch: np.ndarray) -> np.ndarray:
    """Label cache of one KV head: L[t, j] = K[t, ch[j]]  ([T, r]).

    Double Sparsity page, key points and abstract: only the important feature
    channels of K are consulted to find the important tokens.
    """
    return np.asarray(K)[:, np.asarray(ch)]


def label_scores(q_group: np.ndarray, L: np.ndarray, ch: np.ndarray) -> np.ndarray:
    """Approximate score of every token, u[t] = sum_h sum_j q[h, ch[j]] * L[t, j].

    Double Sparsity page, abstract: channel sparsity identifies the important
    tokens.  Query heads that share one KV head are summed so the group keeps
    one token set.  q_group: [G, d]; L: [T, r].  Returns float64 [T].
    """
    qs = np.asarray(q_group, dtype=np.float64)[:, np.asarray(ch)]    # [G, r]
    per_head = np.asarray(L, dtype=np.float64) @ qs.T                 # [T, G]
    return per_head.sum(axis=1)


def block_scores(u: np.ndarray, block: int) -> np.ndarray:
    """Block informativeness = max of the token scores in the block.

    Jenga page, core method item 1: token scores are aggregated block-wise by
    taking the maximum (default block of 64 tokens).  A partial last block
    takes the max over the tokens it has.
    """
    u = np.asarray(u, dtype=np.float64)
    nb = -(-len(u) // block)
    return np.array([u[i * block:min((i + 1) * block, len(u))].max() for i in range(nb)])


def select_topk(u: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, ascending.

    Double Sparsity page, method details: the tokens with the higher
    (approximate) activations are the ones kept.  HiP page, abstract: the top-k
    keys for the query.
    """
    u = np.asarray(u, dtype=np.float64)
    if not (1 <= k <= len(u)):
        raise ValueError("k out of range")
    order = np.argsort(-u, kind="stable")
    return np.sort(order[:k]).astype(np.int64)


def blocks_to_tokens(blocks: np.ndarray, block: int, T: int) -> np.ndarray:
    """Token ids covered by the kept blocks, ascending, clipped to the T valid tokens."""
    blocks = np.sort(np.asarray(blocks, dtype=np.int64))
    toks = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return toks[toks < T]


# -- online stage: exact attention over the kept tokens ---------------------

def attention_weights(q_group: np.ndarray, K: np.ndarray, S: np.ndarray, scale: float) -> np.ndarray:
    """Softmax weights [G, |S|] of each query head over the kept tokens S."""
    z = np.asarray(q_group, dtype=np.float64) @ np.asarray(K, dtype=np.float64)[S].T * scale
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return w / w.sum(axis=1, keepdims=True)


def attend(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray, scale: float) -> np.ndarray:
    """Self-attention restricted to the kept tokens: out[h] = softmax(q_h.K_S * scale) V_S.

    Double Sparsity page, key points and abstract: token sparsity computes
    self-attention with the important tokens only.  Jenga page, core method
    item 3: kept rows are read in place from the original cache (no reordered
    copy), which does not change the result.  Returns float64 [G, d].
    """
    w = attention_weights(q_group, K, S, scale)
    return w @ np.asarray(V, dtype=np.float64)[S]


def attend_partial(q_group, K, V, S, scale):
    """Unnormalised softmax state over a slice S of the kept tokens: (m [G], l [G], acc [G, d])."""
    z = np.asarray(q_group, dtype=np.float64) @ np.asarray(K, dtype=np.float64)[S].T * scale
    m = z.max(axis=1)
    p = np.exp(z - m[:, None])
    return m, p.sum(axis=1), p @ np.asarray(V, dtype=np.float64)[S]


def merge_partials(parts):
    """Combine per-slice softmax states by log-sum-exp: m = max m_s, l = sum l_s e^(m_s - m),
    out = sum acc_s e^(m_s - m) / l.  Exact algebra of softmax over a partitioned set."""
    m = np.max(np.stack([p[0] for p in parts]), axis=0)
    l = sum(p[1] * np.exp(p[0] - m) for p in parts)
    acc = sum(p[2] * np.exp(p[0] - m)[:, None] for p in parts)
    return acc / l[:, None]


# -- one decode step of one (sequence, KV head) unit ------------------------

def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def decode_unit(q_group, K, V, ch, k_units, block=1, scale=None, T=None):
    """Double Sparsity decode for one unit, steps in the page's order.

    q_group [G, d], K and V [>= T, d] (float64 values), ch [r] label channels.
    Returns (out [G, d], kept unit ids ascending, scores of the units).
    """
    K = np.asarray(K, dtype=np.float64)
    if T is None:
        T = K.shape[0]
    K = K[:T]
    V = np.asarray(V, dtype=np.float64)[:T]
    if scale is None:
        scale = default_scale(K.shape[1])
    L = label_rows(K, ch)
    u = label_scores(q_group, L, ch)
    if block == 1:
        scores = u
        kept = select_topk(u, k_units)
        S = kept
    else:
        scores = block_scores(u, block)
        kept = select_topk(scores, k_units)
        S = blocks_to_tokens(kept, block, T)
    return attend(q_group, K, V, S, scale), kept, scores


def tokens_of(kept, block, T):
    """Token ids attended for a kept-unit list (identity for block == 1)."""
    kept = np.asarray(kept, dtype=np.int64)
    return kept if block == 1 else blocks_to_tokens(kept, block, T)


# -- threshold selection with positive-only head aggregation ----------------

def label_scores_positive(q_group: np.ndarray, L: np.ndarray, ch: np.ndarray) -> np.ndarray:
    """Informativeness of every token: u[t] = sum_h max(0, sum_j q[h, ch[j]] * L[t, j]).

    Jenga page, core method item 1: per-token informativeness aggregates the
    attention scores over heads counting only positive ones.  The score of
    head h is its label-channel approximation (Double Sparsity page,
    abstract).  q_group: [G, d]; L: [T, r].  Returns float64 [T].
    """
    qs = np.asarray(q_group, dtype=np.float64)[:, np.asarray(ch)]    # [G, r]
    per_head = np.asarray(L, dtype=np.float64) @ qs.T                 # [T, G]
    return np.maximum(per_head, 0.0).sum(axis=1)


def select_threshold(u: np.ndarray, tau: float, k_max: int) -> np.ndarray:
    """Units whose score is at least tau, ascending; when more than k_max pass,
    the k_max largest of them, ties to the lower index.

    Jenga page, core method item 1: block informativeness is compared with a
    layer-specific threshold and the blocks below it are eliminated.  k_max is
    the capacity of the caller's index buffer.
    """
    u = np.asarray(u, dtype=np.float64)
    if k_max < 1:
        raise ValueError("k_max out of range")
    passing = np.flatnonzero(u >= tau)
    if len(passing) <= k_max:
        return passing.astype(np.int64)
    order = passing[np.argsort(-u[passing], kind="stable")]   # passing is ascending: ties keep the lower index
    return np.sort(order[:k_max]).astype(np.int64)


def decode_unit_threshold(q_group, K, V, ch, k_max, tau, block=1, scale=None, T=None):
    """Decode for one unit with the threshold rule: positive-only head
    aggregation, block max, keep the units at or above tau (at most k_max),
    attention over their tokens (zero when none is kept).

    Returns (out [G, d], kept unit ids ascending, scores of the units).
    """
    K = np.asarray(K, dtype=np.float64)
    if T is None:
        T = K.shape[0]
    K = K[:T]
    V = np.asarray(V, dtype=np.float64)[:T]
    if scale is None:
        scale = default_scale(K.shape[1])
    u = label_scores_positive(q_group, label_rows(K, ch), ch)
    scores = u if block == 1 else block_scores(u, block)
    kept = select_threshold(scores, tau, k_max)
    S = tokens_of(kept, block, T)
    if len(S) == 0:
        return np.zeros((np.asarray(q_group).shape[0], K.shape[1])), kept, scores
    return attend(q_group, K, V, S, scale), kept, scores


# -- hierarchical span search (HiP page, abstract) ---------------------------

def group_token_scores(q_group, K, tokens):
    """Score of each listed key token for the query group: the float64 sum over
    the group's query heads of q_h . K_t (no scale; a positive scale cannot
    change a ranking).  The search ranks these float64 values."""
    qs = np.asarray(q_group, dtype=np.float64).sum(axis=0)        # [d]
    return np.asarray(K, dtype=np.float64)[np.asarray(tokens, dtype=np.int64)] @ qs


def hip_search(q_group, K, T, k, span):
    """Top-k key spans by hierarchical pruning, as (start, end) pairs ascending.

    HiP page, abstract: nearby key tokens tend to have similar attention scores
    ("attention locality"), so a tree-search-like procedure estimates the top-k
    keys of a query on the fly in O(log T) rounds.  The page gives no further
    detail; the procedure taken is a beam search over the binary halving tree:
      * start from k spans splitting [0, T) evenly (span i is
        [floor(i T / k), floor((i + 1) T / k)));
      * each round, split every span longer than `span` tokens into a left half
        of ceil(len / 2) tokens and a right half of the rest (shorter spans go
        on whole), score every candidate by its first token, and keep the k
        highest-scoring candidates (ties to the lower start);
      * stop when no span is longer than `span` tokens.
    Requires 1 <= k <= T and span >= 1.
    """
    if not (1 <= k <= T) or span < 1:
        raise ValueError("need 1 <= k <= T and span >= 1")
    spans = [(i * T // k, (i + 1) * T // k) for i in range(k)]
    score = dict(zip([s for s, _ in spans], group_token_scores(q_group, K, [s for s, _ in spans])))
    while any(e - s > span for s, e in spans):
        cand = []
        for s, e in spans:
            if e - s > span:
                m = s + (e - s + 1) // 2
                cand += [(s, m), (m, e)]
            else:
                cand.append((s, e))
        new = [c[0] for c in cand if c[0] not in score]
        if new:
            score.update(zip(new, group_token_scores(q_group, K, new)))
        keys = np.array([score[s] for s, _ in cand], dtype=np.float64)
        order = np.argsort(-keys, kind="stable")   # candidates are in start order: ties keep the lower start
        keep = np.sort(order[:k])
        spans = [cand[i] for i in keep]
    return spans


def spans_to_tokens(spans):
    """Token ids covered by the spans, ascending."""
    return np.concatenate([np.arange(s, e, dtype=np.int64) for s, e in spans]) if spans else \
        np.zeros(0, dtype=np.int64)


def decode_unit_hip(q_group, K, V, k, span, scale=None, T=None):
    """Decode for one unit with the hierarchical span search: attention over the
    tokens of the k kept spans.  Returns (out [G, d], kept spans)."""
    K = np.asarray(K, dtype=np.float64)
    if T is None:
        T = K.shape[0]
    K = K[:T]
    V = np.asarray(V, dtype=np.float64)[:T]
    if scale is None:
        scale = default_scale(K.shape[1])
    spans = hip_search(q_group, K, T, k, span)
    return attend(q_group, K, V, spans_to_tokens(spans), scale), spans
