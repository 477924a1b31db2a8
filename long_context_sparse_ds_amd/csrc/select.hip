// Per-row exact top-k selection.
//
// Double Sparsity page, method details: the tokens whose approximate scores
// are highest are the ones kept; HiP page, abstract: the top-k keys of the
// query.  Ties go to the lower index, and the kept indices are written in
// ascending order.
//
// One workgroup of 1024 threads per row.  Scores are mapped to order-
// preserving 32-bit keys; three most-significant-digit radix passes (11, 11
// and 10 bits) with LDS histograms find the exact k-th largest key tau and how
// many keys equal to tau must be taken (the lowest-indexed ones).  A final pass
// compacts the kept indices in order with a workgroup prefix sum.
#include "ds_common.h"

namespace ds {
namespace {

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;
constexpr int kItems = 4;   // consecutive keys per thread in the compaction pass

// Exclusive prefix sum over the workgroup, in thread order.  `total` receives
// the sum of all values.  Uses wsum[kNW] of LDS; ends with a barrier so wsum can
// be reused at once.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < kNW ? wsum[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kNW; o <<= 1) {
      const uint32_t y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kNW) wsum[lane] = w;
  }
  __syncthreads();
  const uint32_t before = wid ? wsum[wid - 1] : 0u;
  total = wsum[kNW - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kNT) void select_kernel(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                     int64_t k, int32_t* __restrict__ idx_out) {
  const int64_t row = blockIdx.x;
  const float* s = scores + row * ld;
  int32_t* out = idx_out + row * k;
  const int tid = threadIdx.x;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[kNW];
  __shared__ uint32_t sh_digit, sh_above;

  uint32_t prefix = 0u, mask = 0u;
  uint32_t kk = uint32_t(k);   // keys still to take among those matching `prefix`
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass < 2 ? 2048 : 1024;
    for (int i = tid; i < 2048; i += kNT) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kNT) {
      const uint32_t key = float_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & uint32_t(nb - 1)], 1u);
    }
    __syncthreads();
    // Thread t owns bins in descending digit order: nb-1-(t*per) ... ; an
    // exclusive scan gives the count of keys in higher bins.
    const int per = nb / kNT;
    uint32_t mine = 0u;
    for (int j = 0; j < per; ++j) mine += hist[nb - 1 - (tid * per + j)];
    uint32_t tot;
    uint32_t above = block_exclusive_scan(mine, wsum, tot);
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (tid * per + j);
      const uint32_t c = hist[bin];
      if (above < kk && above + c >= kk) {
        sh_digit = uint32_t(bin);
        sh_above = above;
      }
      above += c;
    }
    __syncthreads();
    kk -= sh_above;
    prefix |= sh_digit << shift;
    mask |= uint32_t(nb - 1) << shift;
    __syncthreads();
  }

  // prefix is now the k-th largest key tau; kk (>= 1) of the keys equal to tau
  // are kept, lowest index first.
  const uint32_t tau = prefix;
  uint32_t eq_rem = kk;
  int64_t out_pos = 0;
  for (int64_t base = 0; base < n; base += int64_t(kNT) * kItems) {
    uint32_t keys[kItems];
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t i = base + int64_t(tid) * kItems + j;
      keys[j] = i < n ? float_key(s[i]) : 0u;   // 0 is below every real key
      gt += keys[j] > tau;
      eq += (i < n) && keys[j] == tau;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((gt << 16) | eq, wsum, tot);
    const uint32_t gt_before = ex >> 16, eq_before = ex & 0xFFFFu;
    const uint32_t tot_gt = tot >> 16, tot_eq = tot & 0xFFFFu;
    int64_t pos = out_pos + gt_before + min(eq_before, eq_rem);
    uint32_t eq_seen = eq_before;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t i = base + int64_t(tid) * kItems + j;
      if (i >= n) continue;
      // pos < k always holds when the counts above are right; the bound keeps
      // every store inside this row's output even if they were not.
      if (keys[j] > tau) {
        if (pos < k) out[pos] = int32_t(i);
        ++pos;
      } else if (keys[j] == tau) {
        if (eq_seen < eq_rem) {
          if (pos < k) out[pos] = int32_t(i);
          ++pos;
        }
        ++eq_seen;
      }
    }
    const uint32_t took = min(tot_eq, eq_rem);
    out_pos += tot_gt + took;
    eq_rem -= took;
  }
}

}  // namespace

hipError_t launch_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx,
                         hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(rows)), dim3(kNT), 0, s, scores, n, ld, k, idx);
  return hipGetLastError();
}

}  // namespace ds
