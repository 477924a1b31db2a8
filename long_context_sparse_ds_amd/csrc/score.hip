// Approximate token scores from the label cache, and the block-max variant.
//
// Double Sparsity page, abstract and method details: the offline-calibrated
// label channels identify the important tokens; the score of token t for KV
// head g is sum_h sum_j q[h, ch[g, j]] * label[t, j] over the group's query
// heads h (summing q over the group first is the same sum).  Jenga page, core
// method item 1: a block's score is the max of its tokens' scores.
//
// This is the only O(T) stream of the decode step: each token contributes
// r * element_size bytes.  Four tokens per thread, all requested before any
// arithmetic, so a wavefront reads 64 consecutive label rows per
// load instruction.  Products are exact in double precision for bf16 and fp32
// inputs and the sum of at most d of them is accumulated in double, so the
// float32 result is the exact score rounded once.
//
// POS (Jenga page, core method item 1): a token's informativeness counts only
// the query heads whose score is positive, u[t] = sum_h max(0, s_h[t]) with
// s_h[t] = sum_j q[h, ch[g, j]] * label[t, j]; each head's sum and the sum over
// heads are accumulated in double, so here too the float32 result is the
// exact value rounded once (up to double rounding of the sums).
//
// SORT (token-level rows split over several workgroups of the fused kernel):
// instead of the scores in unit order and a histogram, each tile writes its
// units in descending order of the top 11 bits of their score keys (a counting
// sort: the histogram's LDS atomics return each unit's rank within its bin),
// one 32-bit word per unit: the key's low 21 bits above the 11-bit tile-local
// id (the top 11 bits are the digit, known from the unit's place in the list);
// plus the tile's exclusive descending prefix P[b] = number of units whose top
// digit exceeds b.  The selection kernel then finds any digit's units of a
// tile at a known offset without reading the rest of the row.
//
// Tokens in [t_append, T) first get their label rows rebuilt from K (the
// per-step label-row append of the newest tokens, fused here so a decode step
// is a single pass over the label cache); they are scored from the values just
// gathered, summed in the same channel order.
#include <type_traits>

#include "label_dot.h"
#include "select_dev.h"

DS_STAMP_BUFFER(score)

namespace ds {
namespace {

constexpr int kThreads = 512;
constexpr int kTPT = 4;                     // tokens per thread
constexpr int kTile = kThreads * kTPT;      // tokens per workgroup
static_assert(kTile == kScoreTile, "tile size shared with the fused kernel's histogram reader");

// Unpack NV 16-byte words of label values into doubles.
template <int NV>
__device__ __forceinline__ void label_values(const uint4 (&raw)[NV], double* lv, uint16_t) {
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lv[v * 8 + 2 * k] = double(bf16_lo(w[k]));
      lv[v * 8 + 2 * k + 1] = double(bf16_hi(w[k]));
    }
  }
}
template <int NV>
__device__ __forceinline__ void label_values(const uint4 (&raw)[NV], double* lv, float) {
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    lv[v * 4 + 0] = double(__uint_as_float(raw[v].x));
    lv[v * 4 + 1] = double(__uint_as_float(raw[v].y));
    lv[v * 4 + 2] = double(__uint_as_float(raw[v].z));
    lv[v * 4 + 3] = double(__uint_as_float(raw[v].w));
  }
}

// R > 0: label width known at compile time and R * sizeof(TE) a multiple of 16 bytes.
// R == 0: any width, element loads.
// append_row (label_dot.h) with positive-only head aggregation; qh holds q[h, ch[j]] at h * r + j.
template <typename TE>
__device__ __forceinline__ float append_row_pos(const TE* __restrict__ Krow, TE* __restrict__ Lrow, const int* sch,
                                                const double* qh, int r, int G) {
  for (int j = 0; j < r; ++j) Lrow[j] = Krow[sch[j]];
  double a = 0.0;
  for (int h = 0; h < G; ++h) {
    double s = 0.0;
    for (int j = 0; j < r; ++j) s = fma(qh[h * r + j], double(elem_to_f32(Krow[sch[j]])), s);
    a += fmax(s, 0.0);
  }
  return float(a);
}

// The arguments the first loads need come first: the first 14 dwords are
// preloaded into SGPRs at wave launch where the firmware supports it, so the
// label stream starts without a kernel-argument round trip.
// RAGGED: sequence b holds seq_lens[b] tokens (clamped to [1, T]); its last
// n_append rows are rebuilt, and its scores past its length are written as
// -inf up to T, so a row's score buffer is always T entries long.
// POS: positive-only head aggregation (G <= 8, checked on the host).
// Grid: (8, tiles, rows / 8) when xcd_rows (row = 8 z + x, tile = y: every
// tile of a row runs on the XCD of the fused kernel's splits of that row, whose
// L2 then holds what this kernel wrote), else (tiles, Hkv, B).
// SORT: sorted-list output (block == 1, tile_hist given), in the score buffer.
// The unsorted bf16 instance for 16 label channels is held to 80 VGPRs (six
// wavefronts per SIMD: three workgroups per CU instead of two, for more label
// rows in flight on long streams); it fits without spilling, where the other
// instances would spill.
template <typename TE, int R, bool RAGGED, bool POS, bool SORT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(TE) == 2 && R == 16 && !RAGGED && !POS && !SORT ? 6 : 1))) void score_kernel(const TE* __restrict__ q, TE* __restrict__ label,
                                                         const int32_t* __restrict__ ch, int64_t T_cap, int T,
                                                         int t_append, int G, int Hkv, int r, int block,
                                                         const TE* __restrict__ Kc, float* __restrict__ scores,
                                                         int64_t ld, uint16_t* __restrict__ tile_hist,
                                                         unsigned* __restrict__ tickets, int tickets_per_row,
                                                         const int32_t* __restrict__ seq_lens, int n_append,
                                                         int xcd_rows, int n_tiles) {
  // 32-bit index math throughout (T < 2^31 is checked on the host); 64-bit
  // only for element offsets.
  uint32_t row, tile, g, b;
  if (xcd_rows) {
    row = blockIdx.z * uint32_t(kXcds) + blockIdx.x;
    tile = blockIdx.y;
    b = row / uint32_t(Hkv);
    g = row - b * uint32_t(Hkv);
  } else {
    tile = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
    row = b * uint32_t(Hkv) + g;
  }
  TE* L = label + int64_t(row) * T_cap * r;
  DS_STAMP_START(score);
  const int t0 = int(tile) * kTile + int(threadIdx.x);
  int Ti = T, ta = t_append;
  if constexpr (RAGGED) {
    Ti = min(max(seq_lens[b], 1), T);
    ta = max(Ti - n_append, 0);
  }
  constexpr int NV = R > 0 ? R * int(sizeof(TE)) / 16 : 1;
  // Requests in the order they are needed: the group's q values for every
  // channel (up to 8 heads at a time) and the channel table first, since they
  // gate the arithmetic; then the label rows, whose latency the q-sum and the
  // histogram clearing overlap.
  constexpr int kQB = 8;
  __shared__ double qall[POS ? kQB : 1][kHeadDim];
  __shared__ double qs[POS ? kQB * kHeadDim : kHeadDim];   // POS: q[h, ch[j]] at h * r + j
  __shared__ int sch[kHeadDim];
  __shared__ uint32_t h[kHistBins];
  static_assert(kThreads >= kHeadDim, "one thread per channel");
  // All loads below are unconditional, with clamped indices and masked values:
  // conditional loads leave the compiler unable to count the loads in flight,
  // and it then waits for all of them at the first use of any.
  const int ql = threadIdx.x < kHeadDim ? int(threadIdx.x) : 0;
  const TE* qg = q + int64_t(row) * G * kHeadDim + ql;
  float qv[kQB];
#pragma unroll
  for (int h8 = 0; h8 < kQB; ++h8) qv[h8] = elem_to_f32(qg[int64_t(h8 < G ? h8 : 0) * kHeadDim]);
  double qrest = 0.0;   // heads past the first 8 (rare), fetched before the label rows
  for (int h = kQB; h < G; ++h) qrest += double(elem_to_f32(qg[int64_t(h) * kHeadDim]));
  // POS: thread i < G * r needs channel i % r (and thread j < r channel j).
  const int tx = int(threadIdx.x);
  const int jj = POS ? (tx < kQB * r ? tx % r : 0) : (tx < r ? tx : 0);
  const int cj = ch[g * r + jj];
  // Label-row append: the K rows of this tile's first appended tokens, one
  // whole row per wavefront, requested ahead of the label rows (their
  // rebuild would otherwise wait on a second round trip after the scan).
  // POS rebuilds its rows inside the scoring loop, from global memory: moving
  // it out of the loop made the double-precision head loop measurably slower.
  using RowWord = std::conditional_t<sizeof(TE) == 2, uint32_t, uint2>;   // a row is 64 of these
  static_assert(kHeadDim * sizeof(TE) == 64 * sizeof(RowWord), "one row per wavefront, one word per lane");
  constexpr int kPreRows = kThreads / 64;
  __shared__ RowWord krow[kPreRows][64];
  const int tile0 = int(tile) * kTile;
  const int a_lo = max(ta, tile0), a_hi = min(Ti, tile0 + kTile);   // appended tokens in this tile
  const int wv = int(threadIdx.x) >> 6;
  const bool pre = !POS && a_lo + wv < a_hi;   // uniform over the wavefront
  RowWord kw{};
  if (pre)
    kw = reinterpret_cast<const RowWord*>(Kc + (int64_t(row) * T_cap + a_lo + wv) * kHeadDim)[threadIdx.x & 63];
  uint4 raw[kTPT][NV];
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      const uint4* p = reinterpret_cast<const uint4*>(L + int64_t(t < Ti ? t : 0) * R);   // token 0 exists
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (SORT) {
          // Sorted form: the label rows are read once and the next kernel
          // reads this kernel's lists, so the stream is kept out of the caches.
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + v));
          raw[i][v] = make_uint4(x.x, x.y, x.z, x.w);
        } else {
          raw[i][v] = p[v];
        }
      }
    }
  }
  if (tile_hist != nullptr)
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
  if (pre) krow[wv][threadIdx.x & 63] = kw;
  if (threadIdx.x < kHeadDim) {
    if constexpr (POS) {
#pragma unroll
      for (int h8 = 0; h8 < kQB; ++h8) qall[h8][threadIdx.x] = double(qv[h8]);
    } else {
      double s = qrest;
#pragma unroll
      for (int h8 = 0; h8 < kQB; ++h8) s += h8 < G ? double(qv[h8]) : 0.0;
      qall[0][threadIdx.x] = s;
    }
  }
  __syncthreads();
  if constexpr (POS) {
    if (int(threadIdx.x) < G * r) qs[threadIdx.x] = qall[int(threadIdx.x) / r][cj];
  } else {
    if (threadIdx.x < r) qs[threadIdx.x] = qall[0][cj];
  }
  if (threadIdx.x < r) sch[threadIdx.x] = cj;
  __syncthreads();
  DS_STAMP(score, 2);   // q and the channel table in

  // An appended token's label row and score, from the staged K row when
  // there is one (separate calls keep the LDS reads LDS reads).
  // A staged row's label row is stored at the end of the kernel: a barrier
  // waits for the workgroup's outstanding global stores.
  const auto append = [&](int t, TE* Lrow) -> float {
    if (t - a_lo < kPreRows) return append_score(reinterpret_cast<const TE*>(krow[t - a_lo]), sch, qs, r);
    return append_row(Kc + (int64_t(row) * T_cap + t) * kHeadDim, Lrow, sch, qs, r);
  };
  float u[kTPT];
  if constexpr (POS && R > 0) {
    // Head-outer: one head's q values (LDS broadcast reads) against one token's
    // label values held in double (one token at a time keeps the kernel at
    // 126 VGPRs for r = 16, two workgroups per CU).
    constexpr int TCH = 1;
#pragma unroll
    for (int c0 = 0; c0 < kTPT; c0 += TCH) {
      double lv[TCH][R];
#pragma unroll
      for (int i = 0; i < TCH; ++i) label_values<NV>(raw[c0 + i], lv[i], TE());
      double acc[TCH];
#pragma unroll
      for (int i = 0; i < TCH; ++i) acc[i] = 0.0;
      for (int h = 0; h < G; ++h) {
        double qh[R];
#pragma unroll
        for (int j = 0; j < R; ++j) qh[j] = qs[h * R + j];
#pragma unroll
        for (int i = 0; i < TCH; ++i) {
          double sdot = 0.0;
#pragma unroll
          for (int j = 0; j < R; ++j) sdot = fma(qh[j], lv[i][j], sdot);
          acc[i] += fmax(sdot, 0.0);
        }
      }
#pragma unroll
      for (int i = 0; i < TCH; ++i) {
        const int t = t0 + (c0 + i) * kThreads;
        if (t >= Ti) u[c0 + i] = -INFINITY;
        else if (t >= ta)
          u[c0 + i] = append_row_pos(Kc + (int64_t(row) * T_cap + t) * kHeadDim, L + int64_t(t) * R, sch, qs, R, G);
        else u[c0 + i] = float(acc[i]);
      }
    }
  } else if constexpr (POS) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      double a = 0.0;
      if (t < Ti && t < ta)
        for (int h = 0; h < G; ++h) {
          double sdot = 0.0;
          for (int j = 0; j < r; ++j) sdot = fma(qs[h * r + j], double(elem_to_f32(L[int64_t(t) * r + j])), sdot);
          a += fmax(sdot, 0.0);
        }
      if (t >= Ti) u[i] = -INFINITY;
      else if (t >= ta)
        u[i] = append_row_pos(Kc + (int64_t(row) * T_cap + t) * kHeadDim, L + int64_t(t) * r, sch, qs, r, G);
      else u[i] = float(a);
    }
  } else if constexpr (R > 0) {
    double qr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qr[j] = qs[j];
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      u[i] = t >= Ti ? -INFINITY : float(dot_label<NV>(raw[i], qr, TE()));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      double a = 0.0;
      if (t < Ti && t < ta)
        for (int j = 0; j < r; ++j) a = fma(qs[j], double(elem_to_f32(L[int64_t(t) * r + j])), a);
      u[i] = t >= Ti ? -INFINITY : float(a);
    }
  }
  // The appended tokens (the newest rows, in at most two tiles): their label
  // rows are rebuilt and their scores replaced, apart from the loop above so
  // that the common path carries none of this code.
  if (!POS && a_lo < a_hi) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      if (t >= a_lo && t < a_hi) u[i] = append(t, L + int64_t(t) * r);
    }
  }

  DS_STAMP(score, 3);   // wavefront 0's label rows in and scored
  float* out = scores + int64_t(row) * ld;
  // Each unit score this thread writes: value and whether it exists.
  float uv[kTPT];
  bool has[kTPT];
  if (block == 1) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      uv[i] = u[i];
      has[i] = t < Ti;
    }
  } else {
    // 64 consecutive tokens per wavefront, 64-aligned: blocks of `block` lanes.
    const int lb = __builtin_ctz(unsigned(block));
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      float v = u[i];
      for (int off = block >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      const int t = t0 + i * kThreads;
      uv[i] = v;
      has[i] = t < Ti && (t & (block - 1)) == 0;
    }
  }
  // The unit scores (-inf past this sequence's length), stored after the
  // histogram's barrier: a barrier waits for the workgroup's outstanding
  // global stores.
  const auto store_scores = [&]() {
    const int lb = __builtin_ctz(unsigned(block));
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      if (t < T && (t & (block - 1)) == 0) out[t >> lb] = uv[i];
    }
  };
  constexpr int per = kHistBins / kThreads;   // 4 bins per thread: one 8-byte store
  static_assert(per == 4, "one uint2 of packed 16-bit counts per thread");
  if constexpr (SORT) {
    // Counting sort of the tile's units by top digit, highest digit first.
    // The histogram's atomics return each unit's rank within its bin (any
    // order: the selection kernel orders equal keys by unit id itself).
    uint32_t bin[kTPT], rk[kTPT];
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      bin[i] = float_key(uv[i]) >> 21;
      rk[i] = has[i] ? atomicAdd(&h[bin[i]], 1u) : 0u;
    }
    __syncthreads();
    DS_STAMP(score, 4);   // the tile's top-digit histogram
    // Thread t owns bins 2047 - 4t down to 2044 - 4t, so thread order is
    // descending digit order and one prefix sum gives every bin's start.
    const int hb = kHistBins - 1 - per * int(threadIdx.x);
    uint32_t c[per], sum = 0u;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      c[j] = h[hb - j];
      sum += c[j];
    }
    __shared__ uint32_t wsum[kThreads / 64];
    uint32_t tot;
    uint32_t p = block_exclusive_scan1<kThreads>(sum, wsum, tot);   // one barrier; wsum is not used again
    DS_STAMP(score, 5);   // bin starts
    uint32_t P[per];
#pragma unroll
    for (int j = 0; j < per; ++j) {
      P[j] = p;   // units of this tile whose top digit exceeds bin hb - j
      h[hb - j] = p;
      p += c[j];
    }
    __syncthreads();
    DS_STAMP(score, 6);   // bin starts in LDS
    __shared__ __align__(16) uint32_t sent[SORT ? kTile : 1];
#pragma unroll
    for (int i = 0; i < kTPT; ++i)
      if (has[i])
        sent[h[bin[i]] + rk[i]] = ((float_key(uv[i]) & 0x1FFFFFu) << 11) | uint32_t(threadIdx.x + i * kThreads);
    __syncthreads();
    DS_STAMP(score, 7);   // the tile sorted in LDS
    const int n_tile = min(kTile, Ti - tile0);
    uint32_t* sl = reinterpret_cast<uint32_t*>(out) + tile0;
    // Non-temporal stores: the selection kernel reads these from other XCDs
    // anyway, and lines left dirty in the L2 are written back at the kernel's
    // end, before the next kernel starts.
    // The head of the list (the selection kernel's first round of loads reads
    // the first 2048 / tiles-padded-to-8-or-16 entries) and the prefix go out
    // as ordinary stores; the rest of the list, rarely read, non-temporally.
    const int head = 2 * 1024 / (n_tiles <= 8 ? 8 : 16);
    if (n_tile == kTile) {
      const int e = int(threadIdx.x) * kTPT;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      if (e < head)
        *reinterpret_cast<uint4*>(sl + e) = *reinterpret_cast<const uint4*>(&sent[e]);
      else
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&sent[e]), reinterpret_cast<u32x4*>(sl + e));
    } else {
      for (int e = threadIdx.x; e < n_tile; e += kThreads) {
        if (e < head) sl[e] = sent[e];
        else __builtin_nontemporal_store(sent[e], sl + e);
      }
    }
    // The tile's descending prefix, after the last barrier.
    uint16_t* dst = tile_hist + (int64_t(row) * n_tiles + tile) * kHistBins + (hb - (per - 1));
    *reinterpret_cast<uint2*>(dst) = make_uint2(P[3] | (P[2] << 16), P[1] | (P[0] << 16));
  } else if (tile_hist != nullptr) {
    // Dense histogram of the top 11 key bits of this tile's units (cleared
    // above, before the barriers), every bin written, so the buffer needs no
    // clearing between calls.
#pragma unroll
    for (int i = 0; i < kTPT; ++i)
      if (has[i]) atomicAdd(&h[float_key(uv[i]) >> 21], 1u);
    __syncthreads();
    const int b0 = threadIdx.x * per;
    uint16_t* dst = tile_hist + (int64_t(row) * n_tiles + tile) * kHistBins + b0;
    *reinterpret_cast<uint2*>(dst) = make_uint2(h[b0] | (h[b0 + 1] << 16), h[b0 + 2] | (h[b0 + 3] << 16));
    store_scores();
  } else {
    store_scores();
  }
  // The label rows of the staged appended tokens (their scores are above).
  if (!POS && a_lo < a_hi) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int t = t0 + i * kThreads;
      if (t >= a_lo && t < a_hi && t - a_lo < kPreRows) {
        const TE* kr = reinterpret_cast<const TE*>(krow[t - a_lo]);
        TE* Lrow = L + int64_t(t) * r;
        for (int j = 0; j < r; ++j) Lrow[j] = kr[sch[j]];
      }
    }
  }
  // The row's merge tickets for the fused kernel that follows start at zero.
  if (tickets != nullptr && tile == 0)
    for (int i = threadIdx.x; i < tickets_per_row; i += kThreads) tickets[int64_t(row) * tickets_per_row + i] = 0u;
  DS_STAMP(score, 8);   // stores issued
  DS_STAMP_END(score);
}

template <typename TE, bool RAGGED, bool POS, bool SORT>
hipError_t dispatch_r(const TE* q, TE* label, const TE* Kc, const int32_t* ch, int r, int B, int Hq, int Hkv,
                      int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores, int64_t ld,
                      uint16_t* tile_hist, unsigned* tickets, int tickets_per_row, const int32_t* seq_lens,
                      int n_append, hipStream_t s) {
  const unsigned tiles = unsigned((T + kTile - 1) / kTile);
  const unsigned rows = unsigned(B) * unsigned(Hkv);
  // A row's tiles spread over the XCDs (tile = blockIdx.x): measured faster for
  // the label stream than keeping a row's tiles on one XCD.
  const int xcd = 0;
  const dim3 grid = xcd ? dim3(unsigned(kXcds), tiles, rows / kXcds) : dim3(tiles, unsigned(Hkv), unsigned(B));
  const bool vec = (int64_t(r) * sizeof(TE)) % 16 == 0;
#define DS_SCORE(RR)                                                                                               \
  hipLaunchKernelGGL((score_kernel<TE, RR, RAGGED, POS, SORT>), grid, dim3(kThreads), 0, s, q, label, ch, T_cap,     \
                     int(T), int(t_append), Hq / Hkv, Hkv, r, block, Kc, scores, ld, tile_hist, tickets,           \
                     tickets_per_row, seq_lens, n_append, xcd, int(tiles))
  if (vec && r == 8) DS_SCORE(8);
  else if (vec && r == 16) DS_SCORE(16);
  else if (vec && r == 32) DS_SCORE(32);
  else DS_SCORE(0);
#undef DS_SCORE
  return hipGetLastError();
}

template <typename TE>
hipError_t dispatch(const TE* q, TE* label, const TE* Kc, const int32_t* ch, int r, int B, int Hq, int Hkv,
                    int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores, int64_t ld,
                    uint16_t* tile_hist, unsigned* tickets, int tickets_per_row, const int32_t* seq_lens,
                    int n_append, bool positive, bool sorted, hipStream_t s) {
  if (positive)
    return dispatch_r<TE, false, true, false>(q, label, Kc, ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores,
                                              ld, tile_hist, tickets, tickets_per_row, nullptr, 0, s);
  if (seq_lens != nullptr)
    return dispatch_r<TE, true, false, false>(q, label, Kc, ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores,
                                              ld, tile_hist, tickets, tickets_per_row, seq_lens, n_append, s);
  if (sorted)
    return dispatch_r<TE, false, false, true>(q, label, Kc, ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores,
                                              ld, tile_hist, tickets, tickets_per_row, nullptr, 0, s);
  return dispatch_r<TE, false, false, false>(q, label, Kc, ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores,
                                             ld, tile_hist, tickets, tickets_per_row, nullptr, 0, s);
}

}  // namespace

hipError_t launch_scores(const void* q, void* label, const void* K, const int32_t* ch, int r, int is_bf16, int B,
                         int Hq, int Hkv, int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores,
                         int64_t ld, uint16_t* tile_hist, unsigned* tickets, int tickets_per_row,
                         const int32_t* seq_lens, int n_append, bool positive, hipStream_t s, bool sorted) {
  if (is_bf16)
    return dispatch(static_cast<const uint16_t*>(q), static_cast<uint16_t*>(label), static_cast<const uint16_t*>(K),
                    ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores, ld, tile_hist, tickets, tickets_per_row,
                    seq_lens, n_append, positive, sorted, s);
  return dispatch(static_cast<const float*>(q), static_cast<float*>(label), static_cast<const float*>(K), ch, r, B,
                  Hq, Hkv, T_cap, T, t_append, block, scores, ld, tile_hist, tickets, tickets_per_row, seq_lens,
                  n_append, positive, sorted, s);
}

}  // namespace ds
