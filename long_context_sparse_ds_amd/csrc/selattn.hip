// Fused top-k selection and sparse attention, one launch per decode step.
//
// Double Sparsity page, method details and abstract: keep the tokens with the
// highest approximate scores, then compute self-attention over those tokens
// only.  Jenga page, core method item 3: kept K/V rows are read in place from
// the cache by index.
//
// One workgroup per (row = b * Hkv + g, head chunk, split), 1024 threads.  Every workgroup
// of a row reads the row's scores (from L2 / Infinity Cache: the row was just
// written by the score kernel) into registers and finds the row's exact
// threshold itself, so no workgroup waits for another and the kept indices
// never make a round trip through memory before the gather.  Split s then owns
// kept positions [s * chunk, (s + 1) * chunk) of the ascending kept list: it
// writes those indices, and gathers and attends over those rows only.  When a
// row has one split the workgroup writes the normalised output.  Otherwise it
// publishes its softmax state (m, l, unnormalised acc) and takes a ticket; the
// row's last workgroup merges the states by log-sum-exp and writes the output.
// Workgroups of a row run on different XCDs, whose L2 caches are not kept
// coherent with each other, so the states go through agent-scope accesses
// (written through past the L2, read around it), and a workgroup's stores have
// completed (s_waitcnt) before its ticket is taken.  No cache-wide writeback
// or invalidate is needed.
#include "select_dev.h"

namespace ds {
namespace {

constexpr int kNT = 1024;
constexpr int kNWave = kNT / 64;
constexpr int kMaxChunk = int(kFusedMaxChunk);
constexpr int kU = 2;             // kept rows per lane group per step
constexpr int kXcds = 8;          // MI355X: 8 XCDs, each with its own L2

template <typename TE>
struct Lanes {
  static constexpr int EPL = 16 / int(sizeof(TE));   // elements per lane: 8 (bf16), 4 (fp32)
  static constexpr int LPT = kHeadDim / EPL;          // lanes per 128-wide row: 16, 32
  static constexpr int GPW = 64 / LPT;                // lane groups per wavefront
  static constexpr int NG = kNWave * GPW;             // lane groups per workgroup
};

__device__ __forceinline__ void unpack(const uint4& w, float (&f)[8], uint16_t) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[4], float) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

template <typename TE>
__device__ __forceinline__ float group_sum(float v) {
  v = row16_sum(v);
  if constexpr (Lanes<TE>::LPT == 32) v += __shfl_xor(v, 16);
  return v;
}

// Merge the softmax state of lane groups `off` apart within a wavefront.
template <int HC, int EPL>
__device__ __forceinline__ void merge_lanes(float (&m)[HC], float (&l)[HC], float (&acc)[HC][EPL], int off) {
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const float mo = __shfl_xor(m[h], off);
    const float lo = __shfl_xor(l[h], off);
    const float M = fmaxf(m[h], mo);
    const float fa = m[h] == -INFINITY ? 0.f : __expf(m[h] - M);
    const float fb = mo == -INFINITY ? 0.f : __expf(mo - M);
    l[h] = l[h] * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * fa + __shfl_xor(acc[h][e], off) * fb;
    m[h] = M;
  }
}

template <typename TE, int HC, int ITEMS>
__global__ __launch_bounds__(kNT) void selattn_kernel(const TE* __restrict__ q, const TE* __restrict__ K,
                                                      const TE* __restrict__ V, const float* __restrict__ scores,
                                                      int64_t ld, const uint16_t* __restrict__ tile_hist,
                                                      int tiles, int64_t n_units, int64_t k_units, int Hq, int Hkv,
                                                      int64_t T_cap, int64_t T, int block, int64_t kv_virtual,
                                                      int64_t chunk, int n_split, float scale,
                                                      int32_t* __restrict__ indices, float* __restrict__ part_acc,
                                                      float* __restrict__ part_ml, float* __restrict__ out,
                                                      unsigned* __restrict__ tickets) {
  using LN = Lanes<TE>;
  constexpr int EPL = LN::EPL, LPT = LN::LPT, GPW = LN::GPW, NG = LN::NG;
  __shared__ SelSmem<kNT> sm;
  __shared__ int32_t sel[kMaxChunk];
  __shared__ float wm[kNWave][HC], wl[kNWave][HC], wf[kNWave][HC];
  __shared__ float wacc[kNWave][HC][kHeadDim];
  __shared__ float sM[HC], sL[HC];

  // 1-D grid over (row, head chunk, split).  Workgroups are dealt to the 8 XCDs
  // round-robin by id, so when the (row, chunk) count is a multiple of 8 the ids
  // are arranged to keep every split of a row on one XCD: the row's scores
  // and histograms are then fetched into that XCD's L2 once and shared.
  const int64_t wg = blockIdx.x;
  const int64_t n_rc = int64_t(gridDim.x) / n_split;   // rows * head chunks
  const int head_chunks = (Hq / Hkv) / HC;
  int64_t rc;
  int split;
  if (n_rc % kXcds == 0) {
    const int64_t j = wg / kXcds;
    split = int(j % n_split);
    rc = (j / n_split) * kXcds + wg % kXcds;
  } else {
    split = int(wg % n_split);
    rc = wg / n_split;
  }
  const int64_t row = rc / head_chunks;
  const int hchunk = int(rc % head_chunks);
  const int b = int(row / Hkv), g = int(row % Hkv);
  const int G = Hq / Hkv;
  const int h0 = g * G + hchunk * HC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPT, sub = lane % LPT;
  const int gid = wave * GPW + grp;

  // q slices for the chunk's heads, issued first (independent of the selection).
  float qv[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + (int64_t(b) * Hq + h0 + h) * kHeadDim + sub * EPL);
    unpack(w, qv[h], TE());
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[h][e] *= scale;
  }

  // 1. The row's exact threshold.
  const int64_t p_begin = int64_t(split) * chunk;                 // virtual positions of this split
  const int64_t p_end = min(p_begin + chunk, kv_virtual);
  const int64_t u_lo = p_begin / block, u_hi = (p_end + block - 1) / block;   // kept-list positions
  {
    uint32_t key[ITEMS];
    bool valid[ITEMS];
    load_keys<ITEMS>(scores + row * ld, n_units, key, valid);
    // Top-digit histogram of the row, when the score kernel left one per tile:
    // thread t sums bins 2047 - 2t (high half of the word) and 2046 - 2t.
    uint32_t hi = 0u, lo = 0u;
    if (tile_hist != nullptr) {
      static_assert(kHistBins == 2 * kNT, "two bins per thread");
      const uint32_t* th = reinterpret_cast<const uint32_t*>(tile_hist + row * tiles * kHistBins) +
                           (kHistBins / 2 - 1 - threadIdx.x);
      // All tiles' words requested at once (at most kMaxHistTiles of them).
      uint32_t w[kMaxHistTiles];
#pragma unroll
      for (int t = 0; t < int(kMaxHistTiles); ++t) w[t] = t < tiles ? th[int64_t(t) * (kHistBins / 2)] : 0u;
#pragma unroll
      for (int t = 0; t < int(kMaxHistTiles); ++t) {
        hi += w[t] >> 16;
        lo += w[t] & 0xFFFFu;
      }
    }
    uint32_t kk, mask;
    const uint32_t tau = select_threshold<kNT, ITEMS>(key, valid, uint32_t(k_units), sm, kk, mask,
                                                      tile_hist != nullptr, hi, lo);
    int32_t* ridx = indices + row * k_units;
    const bool write_idx = hchunk == 0;
    for_each_kept<kNT, ITEMS>(key, valid, int64_t(threadIdx.x) * ITEMS, tau, mask, kk, sm,
                              [&](int64_t unit, int64_t pos) {
      if (pos >= u_lo && pos < u_hi) {
        sel[pos - u_lo] = int32_t(unit);
        if (write_idx) ridx[pos] = int32_t(unit);
      }
    });
  }
  __syncthreads();

  // 2. Attention over the split's kept rows.
  float m[HC], l[HC], acc[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const TE* Kr = K + row * T_cap * kHeadDim + sub * EPL;
  const TE* Vr = V + row * T_cap * kHeadDim + sub * EPL;
  for (int64_t base = p_begin; base < p_end; base += int64_t(NG) * kU) {
    int64_t tok[kU];
    bool ok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t p = base + int64_t(gid) * kU + u;
      ok[u] = p < p_end;
      tok[u] = 0;
      if (ok[u]) {
        const int64_t rel = p - p_begin;
        const int64_t unit = sel[rel / block];
        tok[u] = unit * block + rel % block;
        ok[u] = tok[u] < T;
      }
    }
    uint4 kr[kU], vr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ok[u]) {
        kr[u] = *reinterpret_cast<const uint4*>(Kr + tok[u] * kHeadDim);
        vr[u] = *reinterpret_cast<const uint4*>(Vr + tok[u] * kHeadDim);
      } else {
        kr[u] = make_uint4(0u, 0u, 0u, 0u);
        vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    float kf[kU][EPL], vf[kU][EPL];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      unpack(kr[u], kf[u], TE());
      unpack(vr[u], vf[u], TE());
    }
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float z[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qv[h][e], kf[u][e], d);
        d = group_sum<TE>(d);
        z[u] = ok[u] ? d : -INFINITY;
      }
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < kU; ++u) mx = fmaxf(mx, z[u]);
      if (mx == -INFINITY) continue;   // uniform across the lane group
      const float alpha = __expf(m[h] - mx);
      float p[kU], psum = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        p[u] = __expf(z[u] - mx);
        psum += p[u];
      }
      l[h] = l[h] * alpha + psum;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[h][e] * alpha;
#pragma unroll
        for (int u = 0; u < kU; ++u) a = fmaf(p[u], vf[u][e], a);
        acc[h][e] = a;
      }
      m[h] = mx;
    }
  }

  // 3. Merge the lane groups of each wavefront, then the wavefronts.
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) merge_lanes<HC, EPL>(m, l, acc, off);
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      if (sub == 0) {
        wm[wave][h] = m[h];
        wl[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) wacc[wave][h][sub * EPL + e] = acc[h][e];
    }
  }
  __syncthreads();
  if (threadIdx.x < HC) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < kNWave; ++w) M = fmaxf(M, wm[w][h]);
    float Ls = 0.f;
    for (int w = 0; w < kNWave; ++w) {
      const float f = M == -INFINITY ? 0.f : __expf(wm[w][h] - M);
      wf[w][h] = f;
      Ls += wl[w][h] * f;
    }
    sM[h] = M;
    sL[h] = Ls;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HC * kHeadDim; i += kNT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    float A = 0.f;
    for (int w = 0; w < kNWave; ++w) A = fmaf(wacc[w][h][c], wf[w][h], A);
    const int64_t bh = int64_t(b) * Hq + h0 + h;
    if (n_split == 1) {
      out[bh * kHeadDim + c] = A / sL[h];
    } else {
      __hip_atomic_store(&part_acc[(bh * n_split + split) * kHeadDim + c], A, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) {
        __hip_atomic_store(&part_ml[(bh * n_split + split) * 2 + 0], sM[h], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&part_ml[(bh * n_split + split) * 2 + 1], sL[h], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (n_split == 1) return;

  // 4. The row's last workgroup merges the splits.
  __shared__ unsigned sh_ticket;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's state stores have completed
  __syncthreads();
  unsigned* ticket = tickets + rc;
  if (threadIdx.x == 0) sh_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sh_ticket != unsigned(n_split - 1)) return;
  for (int i = threadIdx.x; i < HC * kHeadDim; i += kNT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    const int64_t bh = int64_t(b) * Hq + h0 + h;
    const float* ml = part_ml + bh * n_split * 2;
    const float* pa = part_acc + bh * n_split * kHeadDim + c;
    float M = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp)
      M = fmaxf(M, __hip_atomic_load(&ml[2 * sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    float L = 0.f, A = 0.f;
    for (int sp = 0; sp < n_split; ++sp) {
      const float m = __hip_atomic_load(&ml[2 * sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float l = __hip_atomic_load(&ml[2 * sp + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float a = __hip_atomic_load(&pa[int64_t(sp) * kHeadDim], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float f = __expf(m - M);   // an empty split has m = -inf: f = 0
      L = fmaf(l, f, L);
      A = fmaf(a, f, A);
    }
    out[bh * kHeadDim + c] = A / L;
  }
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename TE, int HC>
hipError_t dispatch_items(const TE* q, const TE* K, const TE* V, const float* scores, int64_t ld,
                          const uint16_t* tile_hist, int64_t n_units,
                          int64_t k_units, int Hq, int Hkv, int64_t T_cap, int64_t T, int block,
                          const DecodePlan& pl, float scale, int32_t* indices, float* part_acc, float* part_ml,
                          float* out, unsigned* tickets, hipStream_t s) {
  const dim3 grid(unsigned(int64_t(pl.sp.n_split) * pl.rows * pl.sp.head_chunks));
#define DS_SA(IT)                                                                                                  \
  hipLaunchKernelGGL((selattn_kernel<TE, HC, IT>), grid, dim3(kNT), 0, s, q, K, V, scores, ld, tile_hist,        \
                     int(pl.tiles), n_units, k_units, Hq,                                                          \
                     Hkv, T_cap, T, block, pl.kv_virtual, pl.sp.chunk, pl.sp.n_split, scale, indices, part_acc, part_ml,    \
                     out, tickets)
  if (n_units <= kNT * 4) DS_SA(4);
  else if (n_units <= kNT * 8) DS_SA(8);
  else if (n_units <= kNT * 16) DS_SA(16);
  else DS_SA(32);
#undef DS_SA
  return hipGetLastError();
}

template <typename TE>
hipError_t dispatch(const TE* q, const TE* K, const TE* V, const float* scores, int64_t ld,
                    const uint16_t* tile_hist, int64_t n_units,
                    int64_t k_units, int Hq, int Hkv, int64_t T_cap, int64_t T, int block, const DecodePlan& pl,
                    float scale, int32_t* indices, float* part_acc, float* part_ml, float* out, unsigned* tickets,
                    hipStream_t s) {
  switch (pl.sp.head_chunk) {
    case 4:
      return dispatch_items<TE, 4>(q, K, V, scores, ld, tile_hist, n_units, k_units, Hq, Hkv, T_cap, T, block, pl, scale,
                                   indices, part_acc, part_ml, out, tickets, s);
    case 2:
      return dispatch_items<TE, 2>(q, K, V, scores, ld, tile_hist, n_units, k_units, Hq, Hkv, T_cap, T, block, pl, scale,
                                   indices, part_acc, part_ml, out, tickets, s);
    default:
      return dispatch_items<TE, 1>(q, K, V, scores, ld, tile_hist, n_units, k_units, Hq, Hkv, T_cap, T, block, pl, scale,
                                   indices, part_acc, part_ml, out, tickets, s);
  }
}

}  // namespace

hipError_t launch_select_attention(const void* q, const void* K, const void* V, int is_bf16, const float* scores,
                                   int64_t ld, const uint16_t* tile_hist, int Hq, int Hkv, int64_t T_cap, int64_t T,
                                   int block, int64_t k_units, float scale, const DecodePlan& pl, int32_t* indices,
                                   float* part_acc, float* part_ml, float* out, unsigned* tickets, hipStream_t s) {
  if (is_bf16)
    return dispatch(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                    scores, ld, tile_hist, pl.n_units, k_units, Hq, Hkv, T_cap, T, block, pl, scale, indices,
                    part_acc, part_ml, out, tickets, s);
  return dispatch(static_cast<const float*>(q), static_cast<const float*>(K), static_cast<const float*>(V), scores, ld,
                  tile_hist, pl.n_units, k_units, Hq, Hkv, T_cap, T, block, pl, scale, indices, part_acc, part_ml,
                  out, tickets, s);
}

}  // namespace ds
