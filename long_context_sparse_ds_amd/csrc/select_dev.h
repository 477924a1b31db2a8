// Device building blocks of the exact per-row top-k selection.
//
// Double Sparsity page, method details: the tokens with the highest
// approximate scores are kept; HiP page, abstract: the top-k keys for the
// query.  The k largest scores are kept, the lower index winning a tie, and the
// kept indices are listed in ascending order.
//
// Scores are compared through order-preserving 32-bit keys (float_key).  Three
// most-significant-digit radix passes (11, 11, 10 bits) over LDS histograms
// find the exact k-th largest key tau and how many keys equal to tau are kept
// (the lowest-indexed ones).  Keys stay in registers, each thread holding a
// contiguous segment of the row, so one prefix sum gives every kept unit its
// position in the ascending output list.
#pragma once

#include "ds_common.h"

namespace ds {

// Candidates (keys sharing the k-th largest key's top 11 bits) gathered into
// LDS for the remaining radix passes; more than this (a kernel may choose a
// larger capacity) falls back to passes over all the register-resident keys.
constexpr int kCandCap = 2048;

template <int NT, int CAP = kCandCap>
struct SelSmem {
  static constexpr int kCap = CAP;
  uint32_t hist[2048];
  uint32_t cand[CAP];
  uint32_t wsum[3][NT / 64];   // one per scan use, so no scan needs a trailing barrier
  uint32_t digit, above, ncand, tau, kk;
};

// Inclusive prefix sum across the 64 lanes of a wavefront with DPP: shifts of
// 1, 2, 4, 8 lanes inside each 16-lane row, then row 0's total is added into
// row 1 and row 2's into row 3 (row_bcast:15, rows 1 and 3 enabled), then
// lane 31's running total into rows 2 and 3 (row_bcast:31).  Lanes whose
// source falls outside the row read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xF, true));
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32<0x111>(x);        // row_shr:1
  x += dpp_u32<0x112>(x);        // row_shr:2
  x += dpp_u32<0x114>(x);        // row_shr:4
  x += dpp_u32<0x118>(x);        // row_shr:8
  x += dpp_u32<0x142, 0xA>(x);   // row_bcast:15
  x += dpp_u32<0x143, 0xC>(x);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over the workgroup in thread order; `total` receives the
// sum.  Ends with a barrier, so wsum can be reused at once.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const uint32_t w = wave_inclusive_scan(lane < NW ? wsum[lane] : 0u);
    if (lane < NW) wsum[lane] = w;
  }
  __syncthreads();
  const uint32_t before = wid ? wsum[wid - 1] : 0u;
  total = wsum[NW - 1];
  __syncthreads();
  return before + x - v;
}

// Lane of the wavefront where an inclusive scan `incl` first reaches kk
// (incl is non-decreasing over the lanes; the caller guarantees some lane does).
__device__ __forceinline__ int first_lane_reaching(uint32_t incl, uint32_t kk) {
  const unsigned long long m = __ballot(incl >= kk);
  return __ffsll(m) - 1;
}

// With the histogram of the current digit complete in sm.hist (nb bins), find
// the digit that holds the kk-th largest candidate, and narrow prefix, mask and
// kk to it.  Wavefront 0 does the search in two parallel steps: lane l sums
// the nb/64 bins just below nb - l * nb/64 (highest digits first; the reads are
// lane-rotated so one step's reads fall in distinct LDS banks), a lane scan
// finds the lane whose bins hold the kk-th key, then that lane's bins are
// spread over the lanes and scanned again.
template <int NT, int CAP>
__device__ __forceinline__ void pick_digit(SelSmem<NT, CAP>& sm, int nb, int shift, uint32_t& prefix, uint32_t& mask,
                                           uint32_t& kk) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = nb >> 6;   // 32 or 16
    const int top = nb - 1 - lane * per;
    uint32_t sum = 0u;
    for (int j = 0; j < per; ++j) sum += sm.hist[top - ((j + lane) & (per - 1))];
    const uint32_t incl = wave_inclusive_scan(sum);
    const int L = first_lane_reaching(incl, kk);
    const uint32_t above_L = __shfl(incl - sum, L);
    const int topL = nb - 1 - L * per;
    const uint32_t c = lane < per ? sm.hist[topL - lane] : 0u;
    const uint32_t incl2 = wave_inclusive_scan(c) + above_L;
    const int j = first_lane_reaching(incl2, kk);
    if (lane == j) {
      sm.digit = uint32_t(topL - j);
      sm.above = incl2 - c;
    }
  }
  __syncthreads();
  kk -= sm.above;
  prefix |= sm.digit << shift;
  mask |= uint32_t(nb - 1) << shift;
}

// Exclusive prefix sum over the workgroup in thread order with a single
// barrier; `wsum` (NT/64 words) must not be written again until every thread
// has returned.  After the barrier every wavefront reads the NT/64 wave totals
// (one per lane, at most 16), scans them inside its first 16-lane row with DPP,
// and takes its own offset and the total with two lane reads.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan1(uint32_t v, uint32_t* wsum, uint32_t& total) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 16, "wave totals scanned inside one 16-lane row");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  uint32_t w = lane < NW ? wsum[lane] : 0u;
  w += dpp_u32<0x111>(w);   // row_shr:1
  w += dpp_u32<0x112>(w);   // row_shr:2
  w += dpp_u32<0x114>(w);   // row_shr:4
  w += dpp_u32<0x118>(w);   // row_shr:8: lane i < 16 holds the total of waves 0..i
  total = uint32_t(__builtin_amdgcn_readlane(int(w), NW - 1));
  const uint32_t before = wid > 0 ? uint32_t(__builtin_amdgcn_readlane(int(w), wid - 1)) : 0u;
  return before + x - v;
}

// One radix pass over the candidate keys in sm.cand (all sharing the bits of
// `mask`, equal to `prefix`): histogram of the next digit, then the digit that
// holds the kk-th largest.  Returns the number of candidates in that digit.
// The histogram must be zeroed (and a barrier passed) on entry.
template <int NT, int CAP>
__device__ __forceinline__ uint32_t candidate_pass(SelSmem<NT, CAP>& sm, int n, int shift, int nb, uint32_t& prefix,
                                                   uint32_t& mask, uint32_t& kk) {
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t c = sm.cand[i];
    if ((c & mask) == prefix) atomicAdd(&sm.hist[(c >> shift) & uint32_t(nb - 1)], 1u);
  }
  __syncthreads();
  pick_digit(sm, nb, shift, prefix, mask, kk);
  const uint32_t count = sm.hist[sm.digit];
  __syncthreads();   // every thread holds the count before anyone clears the histogram
  return count;
}

// Threshold of the k largest valid register-resident keys of the workgroup
// (1 <= k <= number of valid keys), as (tau, mask, kk): the kept keys are those
// with (key & mask) > tau, plus the kk lowest-indexed ones with
// (key & mask) == tau.  mask is all ones unless the selection settles at a
// coarser digit (then every key equal to tau under the mask is kept and kk is
// their count).  hist_hi / hist_lo: when have_hist, the number of valid keys
// whose top 11 bits are 2047 - 2t and 2046 - 2t for thread t (NT = 1024);
// otherwise the histogram is built here.
template <int NT, int ITEMS, int CAP>
__device__ __forceinline__ uint32_t select_threshold(const uint32_t (&key)[ITEMS], const bool (&valid)[ITEMS],
                                                     uint32_t k, SelSmem<NT, CAP>& sm, uint32_t& kk_out,
                                                     uint32_t& mask_out, bool have_hist, uint32_t hist_hi,
                                                     uint32_t hist_lo) {
  static_assert(NT * 2 == 2048, "two top-digit bins per thread");
  const int tid = threadIdx.x, lane = tid & 63;
  if (!have_hist) {
    for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (valid[j]) atomicAdd(&sm.hist[key[j] >> 21], 1u);
    __syncthreads();
    hist_hi = sm.hist[2047 - 2 * tid];
    hist_lo = sm.hist[2046 - 2 * tid];
  }
  if (tid == 0) sm.ncand = 0u;
  // Pass 0: threads in descending-digit order; one scan finds the digit.
  uint32_t tot;
  const uint32_t above = block_exclusive_scan1<NT>(hist_hi + hist_lo, sm.wsum[0], tot);
  if (above < k && above + hist_hi >= k) {
    sm.digit = 2047u - 2u * tid;
    sm.above = above;
  } else if (above + hist_hi < k && above + hist_hi + hist_lo >= k) {
    sm.digit = 2046u - 2u * tid;
    sm.above = above + hist_hi;
  }
  __syncthreads();
  const uint32_t digit = sm.digit;
  uint32_t kk = k - sm.above;
  // Gather the candidates sharing that top digit.
  uint32_t mine = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) mine += valid[j] && (key[j] >> 21) == digit;
  const uint32_t incl = wave_inclusive_scan(mine);
  uint32_t base = 0u;
  if (lane == 63 && incl > 0u) base = atomicAdd(&sm.ncand, incl);
  base = __shfl(base, 63);
  uint32_t at = base + incl - mine;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (valid[j] && (key[j] >> 21) == digit) {
      if (at < uint32_t(CAP)) sm.cand[at] = key[j];
      ++at;
    }
  // Zero the histogram for the next pass while the candidates land.
  for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0u;
  __syncthreads();
  const uint32_t ncand = sm.ncand;
  if (ncand <= uint32_t(CAP)) {
    // Bits 20..10 of the candidates; when the chosen digit holds exactly the kk
    // keys still needed, all of them are kept and the selection is settled at
    // that precision (no tie can straddle it): return the 22-bit prefix as tau
    // with the mask, so the caller compares masked keys.
    uint32_t prefix = digit << 21, mask = 0xFFE00000u;
    const uint32_t c1 = candidate_pass(sm, int(ncand), 10, 2048, prefix, mask, kk);
    if (c1 == kk) {
      kk_out = kk;
      mask_out = mask;
      return prefix;
    }
    for (int i = tid; i < 1024; i += NT) sm.hist[i] = 0u;
    __syncthreads();
    candidate_pass(sm, int(ncand), 0, 1024, prefix, mask, kk);
    kk_out = kk;
    mask_out = 0xFFFFFFFFu;
    return prefix;
  }
  // Too many keys share the top digit: workgroup-wide passes over the registers.
  uint32_t prefix = digit << 21, mask = 0xFFE00000u;
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0, nb = pass == 1 ? 2048 : 1024;
    if (pass == 2) for (int i = tid; i < nb; i += NT) sm.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (valid[j] && (key[j] & mask) == prefix) atomicAdd(&sm.hist[(key[j] >> shift) & uint32_t(nb - 1)], 1u);
    __syncthreads();
    pick_digit(sm, nb, shift, prefix, mask, kk);
  }
  kk_out = kk;
  mask_out = 0xFFFFFFFFu;
  return prefix;
}

__device__ __forceinline__ int radix_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int radix_bins(int pass) { return pass < 2 ? 2048 : 1024; }

// Calls fn(unit, position) for every kept unit of this thread's segment
// [first, first + ITEMS), positions ascending with the unit index across the
// whole row, for the threshold (tau, mask, kk) of select_threshold.  NT * ITEMS
// must stay below 65536.
template <int NT, int ITEMS, int CAP, class F>
__device__ __forceinline__ void for_each_kept(const uint32_t (&key)[ITEMS], const bool (&valid)[ITEMS], int64_t first,
                                              uint32_t tau, uint32_t mask, uint32_t kk, SelSmem<NT, CAP>& sm, F&& fn) {
  static_assert(int64_t(NT) * ITEMS < 65536, "per-row counts must fit in 16 bits");
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    gt += valid[j] && (key[j] & mask) > tau;
    eq += valid[j] && (key[j] & mask) == tau;
  }
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan1<NT>((gt << 16) | eq, sm.wsum[1], tot);
  const uint32_t eq_before = ex & 0xFFFFu;
  int64_t pos = int64_t(ex >> 16) + min(eq_before, kk);
  uint32_t eq_seen = eq_before;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    bool take = false;
    if (valid[j]) {
      const uint32_t km = key[j] & mask;
      if (km > tau) {
        take = true;
      } else if (km == tau) {
        take = eq_seen < kk;
        ++eq_seen;
      }
    }
    if (take) fn(first + j, pos++);
  }
}

// The float of a key (inverse of float_key for non-NaN floats; -0.0 comes back as +0.0).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Load units [tid * ITEMS, tid * ITEMS + ITEMS) of a score row as keys.
template <int ITEMS>
__device__ __forceinline__ void load_keys(const float* s, int64_t n, uint32_t (&key)[ITEMS], bool (&valid)[ITEMS]) {
  const int64_t first = int64_t(threadIdx.x) * ITEMS;
  if ((reinterpret_cast<uintptr_t>(s) & 15) == 0 && first + ITEMS <= n) {
#pragma unroll
    for (int v = 0; v < ITEMS / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(s + first + 4 * v);
      key[4 * v + 0] = float_key(f.x);
      key[4 * v + 1] = float_key(f.y);
      key[4 * v + 2] = float_key(f.z);
      key[4 * v + 3] = float_key(f.w);
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) valid[j] = true;
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      valid[j] = first + j < n;
      key[j] = valid[j] ? float_key(s[first + j]) : 0u;
    }
  }
}

}  // namespace ds
