// Hierarchical span search: the top-k key spans of a decode query found in
// O(log T) rounds, without scoring every token.
//
// HiP page (A Training-free Sub-quadratic Cost Transformer Model Serving
// Framework With Hierarchically Pruned Attention), abstract: nearby key tokens
// tend to have similar attention scores, so a tree-search-like procedure can
// estimate the top-k keys of a query on the fly.  The page gives no algorithm;
// the one built here is a beam search over the binary halving tree of [0, T):
//   * k spans split [0, T) evenly: span i = [floor(i T / k), floor((i+1) T / k));
//   * each round every span longer than `span` tokens is cut into a left part
//     of ceil(len / 2) tokens and the rest (shorter spans go on whole); every
//     candidate is scored by its first token, and the k best candidates are
//     kept, the lower start winning a tie;
//   * the rounds stop when no span is longer than `span` tokens.
// The score of token t for KV head g is the sum over the group's query heads
// of q_h . K_t: the exact dot product of the summed q with K_t, accumulated in
// double and ranked as float32.
//
// One 1024-thread workgroup per (sequence, KV head) row; thread i owns span i
// (k <= 1024), so its two children are candidates 2i and 2i + 1 and the
// candidate list is in ascending start order.  A round: the threads of split
// spans post their right child's first token; lane groups of 16 (bf16) or 32
// (fp32) lanes score the posted tokens, 256-byte K rows read once each; the
// exact top-k of the candidate keys (the left child keeps its parent's score)
// comes from the radix threshold and ordered emission of select_dev.h, which
// writes the kept candidates in ascending order as the next spans.
//
// Output: the spans (start, end) and the covered token ids, ascending, padded
// with -1 to the row's capacity, ready for the attention-from-indices kernels.
#include "select_dev.h"

namespace ds {
namespace {

constexpr int kST = 1024;
constexpr int kMaxSpans = 1024;

template <typename TE>
struct SearchLanes {
  static constexpr int EPL = 16 / int(sizeof(TE));   // elements per lane: 8 (bf16), 4 (fp32)
  static constexpr int LPT = kHeadDim / EPL;          // lanes per token row: 16, 32
  static constexpr int NG = kST / LPT;                // lane groups per workgroup
};

struct SearchSmem {
  SelSmem<kST> sel;
  int32_t req[kMaxSpans];      // token whose score thread i asked for, -1: none
  float score[kMaxSpans];
  int32_t ns[kMaxSpans], ne[kMaxSpans];   // kept candidates: the next spans
  uint32_t nkey[kMaxSpans];
  uint32_t wsum[kST / 64];
};

__device__ __forceinline__ double lane_sum(double v, int lanes) {
  for (int off = lanes >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// The group's summed q for this lane's channels (bf16 and fp32 sums are exact
// in double), heads added in order; each head's 16 bytes are one load, eight
// heads' loads issued before any is used.
template <typename TE>
__device__ __forceinline__ void group_qbar(const TE* __restrict__ q, int64_t h_first, int G, int sub,
                                           double (&qbar)[SearchLanes<TE>::EPL]) {
  using SL = SearchLanes<TE>;
#pragma unroll
  for (int e = 0; e < SL::EPL; ++e) qbar[e] = 0.0;
  for (int h0 = 0; h0 < G; h0 += 8) {
    uint4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = min(h0 + j, G - 1);
      w[j] = *reinterpret_cast<const uint4*>(q + (h_first + h) * kHeadDim + sub * SL::EPL);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (h0 + j >= G) break;
      const uint32_t u[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
      if constexpr (sizeof(TE) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qbar[2 * i] += double(bf16_lo(u[i]));
          qbar[2 * i + 1] += double(bf16_hi(u[i]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qbar[i] += double(__uint_as_float(u[i]));
      }
    }
  }
}

// A token's score from this lane's 16 bytes of its K row: the lane's products
// accumulated in double, then summed over the lane group (the same order in
// every kernel here, so every path ranks the same floats).
template <typename TE>
__device__ __forceinline__ float row_dot(const uint4& w, const double (&qbar)[SearchLanes<TE>::EPL]) {
  double acc = 0.0;
  if constexpr (sizeof(TE) == 2) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fma(qbar[2 * j], double(bf16_lo(u[j])), acc);
      acc = fma(qbar[2 * j + 1], double(bf16_hi(u[j])), acc);
    }
  } else {
    acc = fma(qbar[0], double(__uint_as_float(w.x)), acc);
    acc = fma(qbar[1], double(__uint_as_float(w.y)), acc);
    acc = fma(qbar[2], double(__uint_as_float(w.z)), acc);
    acc = fma(qbar[3], double(__uint_as_float(w.w)), acc);
  }
  return float(lane_sum(acc, SearchLanes<TE>::LPT));
}

// Scores of the posted tokens req[0, k): one lane group per token and step.
template <typename TE>
__device__ __forceinline__ void score_posted(SearchSmem& sm, int k, const TE* __restrict__ Kr,
                                             const double (&qbar)[SearchLanes<TE>::EPL]) {
  using SL = SearchLanes<TE>;
  const int lane = threadIdx.x & 63;
  const int grp = int(threadIdx.x) / SL::LPT, sub = lane % SL::LPT;
  for (int i = grp; i < k; i += SL::NG) {
    const int t = sm.req[i];
    if (t < 0) continue;   // uniform over the lane group
    const uint4 w = *reinterpret_cast<const uint4*>(Kr + int64_t(t) * kHeadDim + sub * SL::EPL);
    const float sc = row_dot<TE>(w, qbar);
    if (sub == 0) sm.score[i] = sc;
  }
}

template <typename TE>
__global__ __launch_bounds__(kST) void hip_search_kernel(const TE* __restrict__ q, const TE* __restrict__ K,
                                                         int Hq, int Hkv, int64_t T_cap, int T, int k, int span,
                                                         int rounds, int32_t* __restrict__ spans_out,
                                                         int32_t* __restrict__ tokens, int cap) {
  using SL = SearchLanes<TE>;
  __shared__ SearchSmem sm;
  const uint32_t row = blockIdx.x;
  const uint32_t b = row / uint32_t(Hkv), g = row - b * uint32_t(Hkv);
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int sub = (tid & 63) % SL::LPT;
  const TE* Kr = K + int64_t(row) * T_cap * kHeadDim;

  // The group's summed q for this lane's channels (bf16 and fp32 sums are exact in double).
  double qbar[SL::EPL];
  group_qbar<TE>(q, int64_t(b) * Hq + int64_t(g) * G, G, sub, qbar);

  // The first spans and their first tokens' scores.
  int s = 0, e = 0;
  uint32_t key = 0u;
  const bool mine = tid < k;
  if (mine) {
    s = int(int64_t(tid) * T / k);
    e = int(int64_t(tid + 1) * T / k);
  }
  if (tid < kMaxSpans) sm.req[tid] = mine ? s : -1;
  __syncthreads();
  score_posted<TE>(sm, k, Kr, qbar);
  __syncthreads();
  if (mine) key = float_key(sm.score[tid]);

  for (int r = 0; r < rounds; ++r) {
    const int len = e - s;
    const bool split = mine && len > span;
    const int m = s + (len + 1) / 2;
    if (tid < kMaxSpans) sm.req[tid] = split ? m : -1;
    __syncthreads();
    score_posted<TE>(sm, k, Kr, qbar);
    __syncthreads();
    uint32_t keys[2] = {key, split ? float_key(sm.score[tid]) : 0u};
    bool valid[2] = {mine, split};
    uint32_t kk, mask;
    const uint32_t tau = select_threshold<kST, 2>(keys, valid, uint32_t(k), sm.sel, kk, mask, false, 0u, 0u);
    const int ls = s, le = split ? m : e, rs = m, re = e;
    for_each_kept<kST, 2>(keys, valid, int64_t(2 * tid), tau, mask, kk, sm.sel, [&](int64_t c, int64_t pos) {
      const bool right = (c & 1) != 0;
      sm.ns[pos] = right ? rs : ls;
      sm.ne[pos] = right ? re : le;
      sm.nkey[pos] = right ? keys[1] : keys[0];
    });
    __syncthreads();
    if (mine) {
      s = sm.ns[tid];
      e = sm.ne[tid];
      key = sm.nkey[tid];
    }
  }

  // Spans, then the covered tokens in ascending order, -1 after them.
  if (mine) {
    int32_t* so = spans_out + (int64_t(row) * k + tid) * 2;
    so[0] = s;
    so[1] = e;
  }
  uint32_t total;
  const uint32_t off = block_exclusive_scan1<kST>(mine ? uint32_t(e - s) : 0u, sm.wsum, total);
  int32_t* tr = tokens + int64_t(row) * cap;
  if (mine)
    for (int t = s; t < e; ++t) tr[off + uint32_t(t - s)] = t;
  for (int i = int(total) + tid; i < cap; i += kST) tr[i] = -1;
}


// ---------------------------------------------------------------------------
// k <= 64 spans: the same search with one wavefront selecting and the other
// fifteen scoring ahead.
//
// A round's candidates (at most 128) fit one wavefront, two per lane: wave 0
// sorts their keys in registers (a bitonic network whose lane exchanges are
// DPP permutations and the permlane swaps, no LDS and no barrier), reads the
// k-th largest key, and keeps the keys above it plus, lowest candidate first,
// as many keys equal to it as are still needed; ballots give every kept
// candidate its ascending position.  Meanwhile waves 1-15 score the first
// token of the right part of every candidate that will be split if it is
// kept, so the next round's scores are ready when the selection ends and a
// round costs one K-row read or one sort, whichever is longer, instead of
// both.  A round's candidates are never stored: lane i of wave 0 derives the
// two children of kept span i from the previous round's kept list, and the
// scoring waves derive the same; the kept lists and the scores ahead are
// double-buffered by round parity, so a round needs one barrier.  (Scoring two
// levels ahead every other round, three K rows per candidate, measured slower:
// the reads of one workgroup are not pure latency.)  The scores and the tie
// rule are those of the kernel above.

constexpr int kWaveSpans = 64;
constexpr int kWaveCand = 2 * kWaveSpans;

// Round r reads buffers (r - 1) & 1 and writes buffers r & 1.
struct WaveSearchSmem {
  int32_t ks[2][kWaveSpans], ke[2][kWaveSpans];   // kept spans (start, end), ascending
  uint32_t kkey[2][kWaveSpans];                    // their keys (their first tokens' scores)
  int32_t kc[2][kWaveSpans];                       // the candidate each was, in the round that kept it
  float spec[2][kWaveCand];                        // score of candidate c's right part's first token
  int32_t tok[kWaveCand];                          // first round: tokens to score
  float tsc[kWaveCand];
  uint32_t wsum[kST / 64];
};

// Child j (0: left, 1: right) of a kept span [s, e) in the next round: its
// bounds, and whether it exists (a span no longer than `span` goes on whole
// as its left child).
__device__ __forceinline__ bool child_of(int s, int e, int j, int span, int& cs, int& ce) {
  const bool split = e - s > span;
  const int m = s + (e - s + 1) / 2;
  cs = j == 0 ? s : m;
  ce = j == 0 ? (split ? m : e) : e;
  return j == 0 || split;
}

constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i of each 8-lane half takes lane 7 - i
constexpr int kDppQuadRev = 0x1B;       // quad_perm [3,2,1,0]

// The value held by lane (lane ^ D) of the wavefront, D a power of two < 64.
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane) {
  if constexpr (D == 1) {
    return dpp_u32<kDppXor1>(v);
  } else if constexpr (D == 2) {
    return dpp_u32<kDppXor2>(v);
  } else if constexpr (D == 4) {
    // Mirror within each half row (lane i takes i ^ 7), then reverse each
    // quad (i takes i ^ 3): i takes i ^ 4.
    return dpp_u32<kDppQuadRev>(dpp_u32<kDppHalfMirror>(v));
  } else if constexpr (D == 8) {
    return dpp_u32<kDppRor8>(v);   // rotating a 16-lane row by 8 pairs i with i ^ 8
  } else if constexpr (D == 16) {
    // Rows 2p and 2p + 1 swap: the first result holds the even row's values
    // in both rows, the second the odd row's.
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(D == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// Bitonic sort, descending, of the wavefront's 128 keys: element t * 64 + lane
// is x[t] of that lane.
template <int SIZE, int DIST>
__device__ __forceinline__ void bitonic_merge(uint32_t (&x)[2], int lane) {
  if constexpr (DIST == 64) {
    const uint32_t hi = max(x[0], x[1]), lo = min(x[0], x[1]);
    x[0] = hi;
    x[1] = lo;
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = t * 64 + lane;
      const uint32_t p = lane_xor<DIST>(x[t], lane);
      // The lower element of a pair takes the larger key in a descending run,
      // the smaller in an ascending one.
      const bool take_max = ((j & SIZE) == 0) == ((j & DIST) == 0);
      x[t] = take_max ? max(x[t], p) : min(x[t], p);
    }
  }
  if constexpr (DIST > 1) bitonic_merge<SIZE, DIST / 2>(x, lane);
}

template <int SIZE>
__device__ __forceinline__ void bitonic_sort(uint32_t (&x)[2], int lane) {
  if constexpr (SIZE > 2) bitonic_sort<SIZE / 2>(x, lane);
  bitonic_merge<SIZE, SIZE / 2>(x, lane);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// Wave 0, round r: the k best children of the previous round's kept spans
// (buffer rb), in ascending order, to buffer wb.  Lane i holds both children
// of kept span i (candidates 2 i and 2 i + 1); lanes >= k hold none (key 0).
__device__ __forceinline__ void wave_select(WaveSearchSmem& sm, int k, int span, int rb, int wb, int lane) {
  int cs[2] = {0, 0}, ce[2] = {0, 0};
  uint32_t o[2] = {0u, 0u};
  if (lane < k) {
    const int s = sm.ks[rb][lane], e = sm.ke[rb][lane];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (child_of(s, e, j, span, cs[j], ce[j]))
        o[j] = j == 0 ? sm.kkey[rb][lane] : float_key(sm.spec[rb][sm.kc[rb][lane]]);
  }
  uint32_t x[2] = {o[0], o[1]};
  bitonic_sort<kWaveCand>(x, lane);
  // Every span leaves at least one valid candidate, so k valid keys (all
  // nonzero) exist and the k-th largest is one of them.
  const uint32_t thr = __builtin_amdgcn_readlane(x[0], k - 1);
  const uint32_t n_gt = uint32_t(__popcll(__ballot(o[0] > thr))) + uint32_t(__popcll(__ballot(o[1] > thr)));
  const uint32_t eq_take = uint32_t(k) - n_gt;
  const bool e0 = o[0] == thr, e1 = o[1] == thr;
  const uint32_t eb0 = lanes_below(__ballot(e0)) + lanes_below(__ballot(e1));
  const uint32_t eb1 = eb0 + uint32_t(e0);
  const bool k0 = o[0] > thr || (e0 && eb0 < eq_take);
  const bool k1 = o[1] > thr || (e1 && eb1 < eq_take);
  const uint32_t p0 = lanes_below(__ballot(k0)) + lanes_below(__ballot(k1));
  const uint32_t p1 = p0 + uint32_t(k0);
  if (k0) {
    sm.ks[wb][p0] = cs[0];
    sm.ke[wb][p0] = ce[0];
    sm.kkey[wb][p0] = o[0];
    sm.kc[wb][p0] = 2 * lane;
  }
  if (k1) {
    sm.ks[wb][p1] = cs[1];
    sm.ke[wb][p1] = ce[1];
    sm.kkey[wb][p1] = o[1];
    sm.kc[wb][p1] = 2 * lane + 1;
  }
}

// Scores of the tokens t[u] (t < 0: none; token 0 is read in its place) of
// this lane group, every K row requested before any is used.
template <typename TE, int PER>
__device__ __forceinline__ void score_tokens(const int32_t (&t)[PER], const TE* __restrict__ Kr, int sub,
                                             const double (&qbar)[SearchLanes<TE>::EPL], float (&out)[PER]) {
  using SL = SearchLanes<TE>;
  uint4 w[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u)
    w[u] = *reinterpret_cast<const uint4*>(Kr + int64_t(t[u] < 0 ? 0 : t[u]) * kHeadDim + sub * SL::EPL);
#pragma unroll
  for (int u = 0; u < PER; ++u) out[u] = row_dot<TE>(w[u], qbar);
}

template <typename TE>
__global__ __launch_bounds__(kST) void hip_search_wave_kernel(const TE* __restrict__ q, const TE* __restrict__ K,
                                                              int Hq, int Hkv, int64_t T_cap, int T, int k, int span,
                                                              int rounds, int32_t* __restrict__ spans_out,
                                                              int32_t* __restrict__ tokens, int cap) {
  using SL = SearchLanes<TE>;
  constexpr int NG = SL::NG;                        // lane groups of the workgroup
  constexpr int NGS = SL::NG - 64 / SL::LPT;        // lane groups of waves 1-15
  constexpr int PER0 = (kWaveCand + NG - 1) / NG;   // first round: tokens per lane group
  constexpr int PERS = (kWaveCand + NGS - 1) / NGS; // later rounds
  __shared__ WaveSearchSmem sm;
  const uint32_t row = blockIdx.x;
  const uint32_t b = row / uint32_t(Hkv), g = row - b * uint32_t(Hkv);
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % SL::LPT, gid = tid / SL::LPT;
  const TE* Kr = K + int64_t(row) * T_cap * kHeadDim;

  double qbar[SL::EPL];
  group_qbar<TE>(q, int64_t(b) * Hq + int64_t(g) * G, G, sub, qbar);

  const bool mine = tid < k;
  const int s0 = mine ? int(int64_t(tid) * T / k) : 0;
  const int e0 = mine ? int(int64_t(tid + 1) * T / k) : 0;
  // The first spans are the kept list of round 0 (buffer 0), each its own
  // candidate tid; their first tokens' scores and their right parts' first
  // tokens' scores are taken together.
  if (mine) {
    sm.ks[0][tid] = s0;
    sm.ke[0][tid] = e0;
    sm.kc[0][tid] = tid;
  }
  int fin = 0;   // buffer holding the final spans
  if (rounds > 0) {
    const bool split0 = mine && e0 - s0 > span;
    if (tid < kWaveSpans) {
      sm.tok[2 * tid] = mine ? s0 : -1;
      sm.tok[2 * tid + 1] = split0 ? s0 + (e0 - s0 + 1) / 2 : -1;
    }
    __syncthreads();
    {
      int32_t t[PER0];
      float sc[PER0];
#pragma unroll
      for (int u = 0; u < PER0; ++u) {
        const int c = gid + NG * u;
        t[u] = c < kWaveCand ? sm.tok[c] : -1;
      }
      score_tokens<TE, PER0>(t, Kr, sub, qbar, sc);
#pragma unroll
      for (int u = 0; u < PER0; ++u)
        if (sub == 0 && t[u] >= 0) sm.tsc[gid + NG * u] = sc[u];
    }
    __syncthreads();
    if (mine) {
      sm.kkey[0][tid] = float_key(sm.tsc[2 * tid]);
      if (split0) sm.spec[0][tid] = sm.tsc[2 * tid + 1];
    }
    __syncthreads();

    for (int r = 1; r <= rounds; ++r) {
      const int rb = (r - 1) & 1, wb = r & 1;
      if (wave == 0) {
        wave_select(sm, k, span, rb, wb, lane);
      } else if (r < rounds) {
        // Scores ahead: the right part's first token of every candidate that
        // would be split next round.
        const int gs = gid - 64 / SL::LPT;
        int32_t t[PERS];
        float sc[PERS];
#pragma unroll
        for (int u = 0; u < PERS; ++u) {
          const int c = gs + NGS * u;
          t[u] = -1;
          if (c < 2 * k) {
            int cs, ce;
            if (child_of(sm.ks[rb][c >> 1], sm.ke[rb][c >> 1], c & 1, span, cs, ce) && ce - cs > span)
              t[u] = cs + (ce - cs + 1) / 2;
          }
        }
        score_tokens<TE, PERS>(t, Kr, sub, qbar, sc);
#pragma unroll
        for (int u = 0; u < PERS; ++u)
          if (sub == 0 && t[u] >= 0) sm.spec[wb][gs + NGS * u] = sc[u];
      }
      __syncthreads();
    }
    fin = rounds & 1;
  } else {
    __syncthreads();
  }

  // Spans, then the covered tokens in ascending order, -1 after them.
  const int s = mine ? sm.ks[fin][tid] : 0, e = mine ? sm.ke[fin][tid] : 0;
  if (mine) {
    int32_t* so = spans_out + (int64_t(row) * k + tid) * 2;
    so[0] = s;
    so[1] = e;
  }
  uint32_t total;
  const uint32_t off = block_exclusive_scan1<kST>(mine ? uint32_t(e - s) : 0u, sm.wsum, total);
  int32_t* tr = tokens + int64_t(row) * cap;
  if (mine)
    for (int t = s; t < e; ++t) tr[off + uint32_t(t - s)] = t;
  for (int i = int(total) + tid; i < cap; i += kST) tr[i] = -1;
}

}  // namespace

hipError_t launch_hip_search(const void* q, const void* K, int is_bf16, int B, int Hq, int Hkv, int64_t T_cap,
                             int64_t T, int k, int span, int rounds, int32_t* spans, int32_t* tokens, int64_t cap,
                             hipStream_t s) {
  const dim3 grid(unsigned(int64_t(B) * Hkv));
  if (k <= kWaveSpans) {
    if (is_bf16)
      hipLaunchKernelGGL(hip_search_wave_kernel<uint16_t>, grid, dim3(kST), 0, s, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(K), Hq, Hkv, T_cap, int(T), k, span, rounds, spans, tokens,
                         int(cap));
    else
      hipLaunchKernelGGL(hip_search_wave_kernel<float>, grid, dim3(kST), 0, s, static_cast<const float*>(q),
                         static_cast<const float*>(K), Hq, Hkv, T_cap, int(T), k, span, rounds, spans, tokens,
                         int(cap));
    return hipGetLastError();
  }
  if (is_bf16)
    hipLaunchKernelGGL(hip_search_kernel<uint16_t>, grid, dim3(kST), 0, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(K), Hq, Hkv, T_cap, int(T), k, span, rounds, spans, tokens,
                       int(cap));
  else
    hipLaunchKernelGGL(hip_search_kernel<float>, grid, dim3(kST), 0, s, static_cast<const float*>(q),
                       static_cast<const float*>(K), Hq, Hkv, T_cap, int(T), k, span, rounds, spans, tokens,
                       int(cap));
  return hipGetLastError();
}

}  // namespace ds
