// Per-row exact top-k selection as a kernel of its own.
//
// Used by the selection-only entry point and by decode rows longer than the
// fused select+attention kernel holds (more than 32768 units): either as the
// first, per-partition stage of a two-stage selection (when the partitions'
// candidates fit the fused kernel) or as a whole-row selection.  One workgroup
// of 1024 threads per row.  Rows of up to 32768 keys are read once into
// registers and selected with the shared radix routine; longer rows are
// streamed from memory (L2-resident after the score kernel) once per radix
// pass, eight independent loads in flight per thread, and compacted in
// ordered tiles.
#include "select_dev.h"

namespace ds {
namespace {

constexpr int kNT = 1024;

template <int ITEMS>
__global__ __launch_bounds__(kNT) void select_regs_kernel(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                          int64_t k, int32_t* __restrict__ idx_out) {
  __shared__ SelSmem<kNT> sm;
  const int64_t row = blockIdx.x;
  int32_t* out = idx_out + row * k;
  uint32_t key[ITEMS];
  bool valid[ITEMS];
  load_keys<ITEMS>(scores + row * ld, n, key, valid);
  uint32_t kk, mask;
  const uint32_t tau = select_threshold<kNT, ITEMS>(key, valid, uint32_t(k), sm, kk, mask, false, 0u, 0u);
  for_each_kept<kNT, ITEMS>(key, valid, int64_t(threadIdx.x) * ITEMS, tau, mask, kk, sm, [&](int64_t unit, int64_t pos) {
    if (pos < k) out[pos] = int32_t(unit);   // always true when the counts are right
  });
}

constexpr int kBatch = 8;

__global__ __launch_bounds__(kNT) void select_stream_kernel(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                            int64_t k, int32_t* __restrict__ idx_out) {
  __shared__ SelSmem<kNT> sm;
  const int64_t row = blockIdx.x;
  const float* s = scores + row * ld;
  int32_t* out = idx_out + row * k;
  const int tid = threadIdx.x;

  uint32_t prefix = 0u, mask = 0u, kk = uint32_t(k);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = radix_shift(pass), nb = radix_bins(pass);
    for (int i = tid; i < nb; i += kNT) sm.hist[i] = 0u;
    __syncthreads();
    for (int64_t base = 0; base < n; base += int64_t(kNT) * kBatch) {
      uint32_t key[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = base + int64_t(j) * kNT + tid;
        key[j] = i < n ? float_key(s[i]) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = base + int64_t(j) * kNT + tid;
        if (i < n && (key[j] & mask) == prefix) atomicAdd(&sm.hist[(key[j] >> shift) & uint32_t(nb - 1)], 1u);
      }
    }
    __syncthreads();
    pick_digit<kNT>(sm, nb, shift, prefix, mask, kk);
  }

  // Ordered compaction over tiles of kNT * 4 consecutive keys.
  const uint32_t tau = prefix;
  uint32_t eq_rem = kk;
  int64_t out_pos = 0;
  constexpr int IT = 4;
  for (int64_t base = 0; base < n; base += int64_t(kNT) * IT) {
    uint32_t key[IT];
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const int64_t i = base + int64_t(tid) * IT + j;
      key[j] = i < n ? float_key(s[i]) : 0u;
      gt += i < n && key[j] > tau;
      eq += i < n && key[j] == tau;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kNT>((gt << 16) | eq, sm.wsum[2], tot);
    const uint32_t eq_before = ex & 0xFFFFu;
    int64_t pos = out_pos + int64_t(ex >> 16) + min(eq_before, eq_rem);
    uint32_t eq_seen = eq_before;
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const int64_t i = base + int64_t(tid) * IT + j;
      bool take = false;
      if (i < n) {
        if (key[j] > tau) {
          take = true;
        } else if (key[j] == tau) {
          take = eq_seen < eq_rem;
          ++eq_seen;
        }
      }
      if (take) {
        if (pos < k) out[pos] = int32_t(i);
        ++pos;
      }
    }
    const uint32_t took = min(tot & 0xFFFFu, eq_rem);
    out_pos += (tot >> 16) + took;
    eq_rem -= took;
  }
}

// First stage of the exact top-k of a long row: the top k of each partition of
// kPartUnits consecutive units (all of it when it holds fewer).  Every unit of
// the row's top k is in its partition's top k under the same tie rule, so the
// second stage, the top k of the candidates, is exact.  Candidates go out in
// ascending unit order (partition by partition, each ascending), so a tie among
// them still goes to the lower unit id: cand_score[row][p * k + i] and
// cand_id[row][p * k + i]; the slots of a partition past its kept count hold
// -inf and -1.
// tile_hist (may be null): the score kernel's top-digit histograms of the
// row's tiles of kHistTileUnits units, tiles per row; a partition sums its
// tiles' counts instead of building its histogram with LDS atomics (which
// contend badly on the few digits that high scores share).  cand_hist (may be
// null; needs tile_hist): the top-digit histogram of each partition's
// candidates, [rows][parts][2048] uint16, for the fused kernel that selects
// among them.
__global__ __launch_bounds__(kNT) void partition_topk_kernel(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                             int64_t k, float* __restrict__ cand_score,
                                                             int64_t cand_ld, int32_t* __restrict__ cand_id,
                                                             int64_t n_cand, const uint16_t* __restrict__ tile_hist,
                                                             int64_t tiles, uint16_t* __restrict__ cand_hist) {
  constexpr int ITEMS = int(kPartUnits / kNT);
  // k is often a quarter of the partition here, so the digit holding the k-th
  // key can hold thousands of keys: room for 8192 candidates.
  __shared__ SelSmem<kNT, 8192> sm;
  const int64_t p = blockIdx.x, row = blockIdx.y;
  const int64_t base = p * kPartUnits;
  const int64_t n_p = min(kPartUnits, n - base);
  const int64_t k_p = min(k, n_p);
  float* cs = cand_score + row * cand_ld + p * k;
  int32_t* ci = cand_id + row * n_cand + p * k;
  uint32_t key[ITEMS];
  bool valid[ITEMS];
  load_keys<ITEMS>(scores + row * ld + base, n_p, key, valid);
  // This thread's two top-digit bins, 2047 - 2t (high half of word 1023 - t)
  // and 2046 - 2t (low half), summed over the partition's tiles.
  uint32_t hist_hi = 0u, hist_lo = 0u;
  const bool have_hist = tile_hist != nullptr;
  if (have_hist) {
    constexpr int kPartTiles = int(kPartUnits / kHistTileUnits);
    const uint32_t* th = reinterpret_cast<const uint32_t*>(tile_hist + row * tiles * kHistBins) +
                         (kHistBins / 2 - 1 - int(threadIdx.x));
    const int64_t t0 = p * kPartTiles;
    uint32_t w[kPartTiles];
#pragma unroll
    for (int t = 0; t < kPartTiles; ++t) w[t] = th[(t0 + t < tiles ? t0 + t : t0) * (kHistBins / 2)];
#pragma unroll
    for (int t = 0; t < kPartTiles; ++t) {
      if (t0 + t < tiles) {
        hist_hi += w[t] >> 16;
        hist_lo += w[t] & 0xFFFFu;
      }
    }
  }
  uint32_t kk, mask;
  const uint32_t tau = select_threshold<kNT, ITEMS>(key, valid, uint32_t(k_p), sm, kk, mask, have_hist, hist_hi,
                                                    hist_lo);
  if (cand_hist != nullptr) {
    // The candidates' histogram: every key in a digit above d0 is kept, k_p
    // minus those in d0, none below.
    const uint32_t d0 = tau >> 21;
    const uint32_t bin_hi = 2047u - 2u * threadIdx.x, bin_lo = bin_hi - 1u;
    uint32_t tot;
    block_exclusive_scan1<kNT>((bin_hi > d0 ? hist_hi : 0u) + (bin_lo > d0 ? hist_lo : 0u), sm.wsum[2], tot);
    const uint32_t in_d0 = uint32_t(k_p) - tot;
    const uint32_t c_hi = bin_hi > d0 ? hist_hi : (bin_hi == d0 ? in_d0 : 0u);
    const uint32_t c_lo = bin_lo > d0 ? hist_lo : (bin_lo == d0 ? in_d0 : 0u);
    const int64_t parts = n_cand / k;
    reinterpret_cast<uint32_t*>(cand_hist + (row * parts + p) * kHistBins)[kHistBins / 2 - 1 - threadIdx.x] =
        (c_hi << 16) | c_lo;
  }
  // The kept units go out in windows of the candidate buffer's size: the
  // emission places each window's keys in that buffer (free once the
  // threshold is known) and their partition-local ids beside them, at their
  // final positions, and the window is then written with coalesced stores.
  // Scattered 4-byte stores straight from the emission cost more than the
  // selection itself.
  constexpr int kWin = decltype(sm)::kCap;
  __shared__ uint16_t kept_id[kWin];
  static_assert(kPartUnits <= 65536, "partition-local ids fit 16 bits");
  const int64_t first = int64_t(threadIdx.x) * ITEMS;
  for (int64_t w0 = 0; w0 < k_p; w0 += kWin) {
    const int64_t w1 = min(w0 + int64_t(kWin), k_p);
    __syncthreads();   // the previous window (or the threshold search) is done with the buffers
    for_each_kept<kNT, ITEMS>(key, valid, first, tau, mask, kk, sm, [&](int64_t unit, int64_t pos) {
      if (pos >= w0 && pos < w1) {
        sm.cand[pos - w0] = key[unit - first];
        kept_id[pos - w0] = uint16_t(unit);
      }
    });
    __syncthreads();
    for (int64_t i = threadIdx.x; i < w1 - w0; i += kNT) {
      cs[w0 + i] = key_to_float(sm.cand[i]);
      ci[w0 + i] = int32_t(base + kept_id[i]);
    }
  }
  for (int64_t i = k_p + threadIdx.x; i < k; i += kNT) {
    cs[i] = -INFINITY;
    ci[i] = -1;
  }
}

}  // namespace

hipError_t launch_partition_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k,
                                 float* cand_score, int64_t cand_ld, int32_t* cand_id, const uint16_t* tile_hist,
                                 int64_t tiles, uint16_t* cand_hist, hipStream_t s) {
  const int64_t parts = (n + kPartUnits - 1) / kPartUnits;
  hipLaunchKernelGGL(partition_topk_kernel, dim3(unsigned(parts), unsigned(rows)), dim3(kNT), 0, s, scores, n, ld, k,
                     cand_score, cand_ld, cand_id, parts * k, tile_hist, tiles, cand_hist);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx,
                         hipStream_t s) {
  const dim3 grid{unsigned(rows)}, block{unsigned(kNT)};
  if (n <= int64_t(kNT) * 4)
    hipLaunchKernelGGL(select_regs_kernel<4>, grid, block, 0, s, scores, n, ld, k, idx);
  else if (n <= int64_t(kNT) * 8)
    hipLaunchKernelGGL(select_regs_kernel<8>, grid, block, 0, s, scores, n, ld, k, idx);
  else if (n <= int64_t(kNT) * 16)
    hipLaunchKernelGGL(select_regs_kernel<16>, grid, block, 0, s, scores, n, ld, k, idx);
  else if (n <= int64_t(kNT) * 32)
    hipLaunchKernelGGL(select_regs_kernel<32>, grid, block, 0, s, scores, n, ld, k, idx);
  else
    hipLaunchKernelGGL(select_stream_kernel, grid, block, 0, s, scores, n, ld, k, idx);
  return hipGetLastError();
}

}  // namespace ds
