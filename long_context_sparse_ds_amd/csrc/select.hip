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
#include "label_dot.h"
#include "select_dev.h"

DS_STAMP_BUFFER(select)

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
// cand_hist (may be null; needs the partition's top-digit histogram): the
// top-digit histogram of each partition's candidates, [rows][parts][2048]
// uint16, for the fused kernel that selects among them.
//
// The end common to both forms below, once thread t holds the keys of units
// [t ITEMS, (t + 1) ITEMS) of the partition (and, when have_hist, the
// partition's counts of its two top-digit bins 2047 - 2t and 2046 - 2t).
template <int ITEMS, int CAP>
__device__ __forceinline__ void partition_finish(const uint32_t (&key)[ITEMS], const bool (&valid)[ITEMS],
                                                 SelSmem<kNT, CAP>& sm, uint16_t* kept_id, bool have_hist,
                                                 uint32_t hist_hi, uint32_t hist_lo, int64_t row, int64_t p,
                                                 int64_t base, int64_t k_p, int64_t k, float* __restrict__ cand_score,
                                                 int64_t cand_ld, int32_t* __restrict__ cand_id, int64_t n_cand,
                                                 uint16_t* __restrict__ cand_hist) {
  float* cs = cand_score + row * cand_ld + p * k;
  int32_t* ci = cand_id + row * n_cand + p * k;
  uint32_t kk, mask;
  const uint32_t tau = select_threshold<kNT, ITEMS>(key, valid, uint32_t(k_p), sm, kk, mask, have_hist, hist_hi,
                                                    hist_lo);
  DS_STAMP(select, 3);   // the partition's threshold
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
  DS_STAMP(select, 4);   // candidates' histogram stored
  constexpr int kWin = CAP;
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
    // Non-temporal: the second stage reads a row's candidates from other XCDs'
    // writes anyway, and lines left dirty in the L2 are written back at the
    // kernel's end, before the next kernel may start.
    for (int64_t i = threadIdx.x; i < w1 - w0; i += kNT) {
      __builtin_nontemporal_store(key_to_float(sm.cand[i]), cs + w0 + i);
      __builtin_nontemporal_store(int32_t(base + kept_id[i]), ci + w0 + i);
    }
  }
  for (int64_t i = k_p + threadIdx.x; i < k; i += kNT) {
    __builtin_nontemporal_store(-INFINITY, cs + i);
    __builtin_nontemporal_store(int32_t(-1), ci + i);
  }
  DS_STAMP(select, 5);   // candidates emitted (stores issued)
  DS_STAMP_END(select);
}

constexpr int kPartItems = int(kPartUnits / kNT);
// k is often a quarter of the partition here, so the digit holding the k-th
// key can hold thousands of keys: room for 8192 candidates.
constexpr int kPartCap = 8192;

// The first stage from a score buffer.  tile_hist (may be null): the score
// kernel's top-digit histograms of the row's tiles of kHistTileUnits units,
// tiles per row; a partition sums its tiles' counts instead of building its
// histogram with LDS atomics (which contend badly on the few digits that high
// scores share).
__global__ __launch_bounds__(kNT) void partition_topk_kernel(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                             int64_t k, float* __restrict__ cand_score,
                                                             int64_t cand_ld, int32_t* __restrict__ cand_id,
                                                             int64_t n_cand, const uint16_t* __restrict__ tile_hist,
                                                             int64_t tiles, uint16_t* __restrict__ cand_hist) {
  constexpr int ITEMS = kPartItems;
  __shared__ SelSmem<kNT, kPartCap> sm;
  __shared__ uint16_t kept_id[kPartCap];
  const int64_t p = blockIdx.x, row = blockIdx.y;
  const int64_t base = p * kPartUnits;
  const int64_t n_p = min(kPartUnits, n - base);
  const int64_t k_p = min(k, n_p);
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
  partition_finish<ITEMS>(key, valid, sm, kept_id, have_hist, hist_hi, hist_lo, row, p, base, k_p, k, cand_score,
                          cand_ld, cand_id, n_cand, cand_hist);
}

// The first stage in one pass over the label cache, for token-level rows: the
// partition's scores are computed here (Double Sparsity page, method details:
// the label channels' dot product with the group's q, as in the score kernel,
// with the same float64 arithmetic, so the scores equal the score kernel's bit
// for bit), with rows [t_append, n) rebuilt from K first (the label-row
// append).  No score buffer goes to memory.  Pass c covers tokens c NT + tid
// of the partition, so a wavefront reads 64 consecutive label rows per load;
// each score goes to the LDS slot of the thread that owns its token in the
// selection, and into the partition's top-digit histogram.  R: label channels
// (LNV 16-byte words per row), or R = 0 for any width (element loads, r at
// run time).  Partition 0 of a row also zeroes the row's merge tickets for the
// fused kernel that follows.
template <typename TE, int R, int LNV>
__global__ __launch_bounds__(kNT) void partition_onepass_kernel(
    const TE* __restrict__ q, TE* __restrict__ label, const TE* __restrict__ Kc, const int32_t* __restrict__ ch,
    int32_t r_rt, int32_t G, int32_t Hkv, int64_t T_cap, int64_t n, int64_t t_append, int64_t k,
    float* __restrict__ cand_score, int64_t cand_ld, int32_t* __restrict__ cand_id, int64_t n_cand,
    uint16_t* __restrict__ cand_hist, unsigned* __restrict__ tickets, int32_t tickets_per_row) {
  constexpr int ITEMS = kPartItems;
  constexpr int RMAX = R > 0 ? R : kHeadDim;
  // Label rows requested together per thread: 64 bytes of 16-byte rows, one
  // row otherwise (two 32-byte rows with their sixteen double channel weights
  // need more than the 128 VGPRs of a 1024-thread workgroup).
  constexpr int CB = R == 0 ? 4 : (LNV == 1 ? 4 : 1);
  static_assert(ITEMS % CB == 0, "whole batches of passes");
  DS_STAMP_START(select);
  __shared__ union {
    float sc[kPartUnits];   // the partition's scores, in the owners' layout
    struct {
      SelSmem<kNT, kPartCap> sel;
      uint16_t kept_id[kPartCap];
    } b;
  } u;
  __shared__ uint32_t hist1[kHistBins];
  __shared__ double qall[kHeadDim];   // the group's q summed over its heads, every channel
  __shared__ double qs_l[RMAX];
  __shared__ int ch_l[RMAX];
  const int r = R > 0 ? R : r_rt;
  const int64_t p = blockIdx.x, row = blockIdx.y;
  const int tid = int(threadIdx.x);
  const int64_t base = p * kPartUnits;
  const int64_t n_p = min(kPartUnits, n - base);
  const int64_t k_p = min(k, n_p);
  const int g = int(row % Hkv);
  // Requests that do not wait on each other, ahead of any use: the group's q
  // for all 128 channels (so that no sum waits for the channel table), the
  // channel table and the first pass's label rows; the label channels' sums
  // are picked after the barrier.  The loads are unconditional and only the
  // stores are not: a load in a branch is waited for where the branch ends.
  const TE* qg = q + row * G * kHeadDim;
  float qv8[8];
  q_load8(qg, G, tid & (kHeadDim - 1), qv8);
  const int cj = ch[g * r + (tid < r ? tid : 0)];
  TE* lab = label + row * T_cap * r;
  uint4 raw[CB][LNV > 0 ? LNV : 1];
  const auto load_pass = [&](int c0) {
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int64_t t = base + (c0 + i) * kNT + tid;
        const uint4* pr = reinterpret_cast<const uint4*>(lab + (t < n ? t : 0) * R);   // row 0 exists
#pragma unroll
        for (int v = 0; v < LNV; ++v) raw[i][v] = pr[v];
      }
    }
  };
  load_pass(0);
  const double qsum = q_score_sum(qv8, qg, G, tid & (kHeadDim - 1));
  if (tid < kHeadDim) qall[tid] = qsum;
  if (tid < r) ch_l[tid] = cj;
  for (int i = tid; i < kHistBins; i += kNT) hist1[i] = 0u;
  if (tickets != nullptr && p == 0)
    for (int i = tid; i < tickets_per_row; i += kNT) tickets[row * tickets_per_row + i] = 0u;
  __syncthreads();
  if (tid < r) qs_l[tid] = qall[ch_l[tid]];
  __syncthreads();
  double qr[RMAX];
  if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < R; ++j) qr[j] = qs_l[j];
  }
  for (int c0 = 0; c0 < ITEMS; c0 += CB) {
    if (c0 > 0) load_pass(c0);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int uloc = (c0 + i) * kNT + tid;
      const int64_t t = base + uloc;
      float sv;
      if (t >= n) {
        sv = -INFINITY;
      } else if (t >= t_append) {
        if constexpr (R > 0) sv = append_row_n<R>(Kc + (row * T_cap + t) * kHeadDim, lab + t * R, ch_l, qs_l);
        else sv = append_row(Kc + (row * T_cap + t) * kHeadDim, lab + t * r, ch_l, qs_l, r);
      } else if constexpr (R > 0) {
        sv = float(dot_label<LNV>(raw[i], qr, TE()));
      } else {
        double a = 0.0;
        for (int j = 0; j < r; ++j) a = fma(qs_l[j], double(elem_to_f32(lab[t * r + j])), a);
        sv = float(a);
      }
      if (t < n) atomicAdd(&hist1[float_key(sv) >> 21], 1u);
      const int ut = uloc / ITEMS, uj = uloc % ITEMS;
      u.sc[((uj >> 2) * kNT + ut) * 4 + (uj & 3)] = sv;
    }
  }
  __syncthreads();
  DS_STAMP(select, 2);   // the partition scored
  // Units past the partition get key 0, below every finite score's key (at
  // least 0x00800000, so their top digit is below any digit the selection can
  // reach): they are never counted, gathered or kept, as k_p never exceeds the
  // partition's units.  So no per-unit validity is carried (a bool array of
  // ITEMS flags lives in scalar lane masks, which spill at this register count).
  uint32_t key[ITEMS];
  bool valid[ITEMS];
  const int first = tid * ITEMS;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    valid[j] = true;
    key[j] = first + j < int(n_p) ? float_key(u.sc[((j >> 2) * kNT + tid) * 4 + (j & 3)]) : 0u;
  }
  const uint32_t hist_hi = hist1[2047 - 2 * tid], hist_lo = hist1[2046 - 2 * tid];
  __syncthreads();   // the scores are in registers: the selection's buffers overlay them
  partition_finish<ITEMS>(key, valid, u.b.sel, u.b.kept_id, true, hist_hi, hist_lo, row, p, base, k_p, k,
                          cand_score, cand_ld, cand_id, n_cand, cand_hist);
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

namespace {
template <typename TE, int R, int LNV>
hipError_t launch_onepass_t(const void* q, void* label, const void* K, const int32_t* ch, int r, int G, int Hkv,
                            int64_t rows, int64_t T_cap, int64_t T, int64_t t_append, int64_t k, float* cand_score,
                            int64_t cand_ld, int32_t* cand_id, uint16_t* cand_hist, unsigned* tickets,
                            int tickets_per_row, hipStream_t s) {
  const int64_t parts = (T + kPartUnits - 1) / kPartUnits;
  hipLaunchKernelGGL((partition_onepass_kernel<TE, R, LNV>), dim3(unsigned(parts), unsigned(rows)), dim3(kNT), 0, s,
                     static_cast<const TE*>(q), static_cast<TE*>(label), static_cast<const TE*>(K), ch, r, G, Hkv,
                     T_cap, T, t_append, k, cand_score, cand_ld, cand_id, parts * k, cand_hist, tickets,
                     tickets_per_row);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_partition_onepass(const void* q, void* label, const void* K, const int32_t* ch, int r, int is_bf16,
                                    int B, int Hq, int Hkv, int64_t T_cap, int64_t T, int64_t t_append, int64_t k,
                                    float* cand_score, int64_t cand_ld, int32_t* cand_id, uint16_t* cand_hist,
                                    unsigned* tickets, int tickets_per_row, hipStream_t s) {
  const int G = Hq / Hkv;
  const int64_t rows = int64_t(B) * Hkv;
#define DS_ONEPASS(TE, R, LNV)                                                                                     \
  return launch_onepass_t<TE, R, LNV>(q, label, K, ch, r, G, Hkv, rows, T_cap, T, t_append, k, cand_score, cand_ld, \
                                      cand_id, cand_hist, tickets, tickets_per_row, s)
  if (is_bf16) {
    if (r == 8) DS_ONEPASS(uint16_t, 8, 1);
    if (r == 16) DS_ONEPASS(uint16_t, 16, 2);
    DS_ONEPASS(uint16_t, 0, 0);
  }
  if (r == 4) DS_ONEPASS(float, 4, 1);
  if (r == 8) DS_ONEPASS(float, 8, 2);
  if (r == 16) DS_ONEPASS(float, 16, 4);
  DS_ONEPASS(float, 0, 0);
#undef DS_ONEPASS
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
