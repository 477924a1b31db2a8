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
    acc = lane_sum(acc, SL::LPT);
    if (sub == 0) sm.score[i] = float(acc);
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
#pragma unroll
  for (int e = 0; e < SL::EPL; ++e) qbar[e] = 0.0;
  for (int h = 0; h < G; ++h) {
    const TE* qh = q + (int64_t(b) * Hq + int64_t(g) * G + h) * kHeadDim + sub * SL::EPL;
#pragma unroll
    for (int e = 0; e < SL::EPL; ++e) qbar[e] += double(elem_to_f32(qh[e]));
  }

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

}  // namespace

hipError_t launch_hip_search(const void* q, const void* K, int is_bf16, int B, int Hq, int Hkv, int64_t T_cap,
                             int64_t T, int k, int span, int rounds, int32_t* spans, int32_t* tokens, int64_t cap,
                             hipStream_t s) {
  const dim3 grid(unsigned(int64_t(B) * Hkv));
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
