// Approximate token scores from the label cache, and the block-max variant.
//
// Double Sparsity page, abstract and method details: the offline-calibrated
// label channels identify the important tokens; the score of token t for KV
// head g is sum_h sum_j q[h, ch[g, j]] * label[t, j] over the group's query
// heads h (summing q over the group first is the same sum).  Jenga page, core
// method item 1: a block's score is the max of its tokens' scores.
//
// This is the only O(T) stream of the decode step: each token contributes
// r * element_size bytes.  One thread per token, four tokens per thread issued
// before any arithmetic, so a wavefront reads 64 consecutive label rows per
// load instruction.  Products are exact in double precision for bf16 and fp32
// inputs and the sum of at most d of them is accumulated in double, so the
// float32 result is the exact score rounded once.
//
// Tokens in [t_append, T) first get their label rows rebuilt from K (the
// per-step label-row append of the newest tokens, fused here so a decode step
// is a single pass over the label cache); they are scored from the values just
// gathered, summed in the same channel order.
#include "ds_common.h"

namespace ds {
namespace {

constexpr int kThreads = 256;
constexpr int kTPT = 4;                     // tokens per thread
constexpr int kTile = kThreads * kTPT;      // tokens per workgroup
static_assert(kTile == kScoreTile, "tile size shared with the fused kernel's histogram reader");

template <int NV>
__device__ __forceinline__ double dot_label(const uint4 (&raw)[NV], const double* qr, uint16_t) {
  double a = 0.0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a = fma(qr[v * 8 + 2 * k], double(bf16_lo(w[k])), a);
      a = fma(qr[v * 8 + 2 * k + 1], double(bf16_hi(w[k])), a);
    }
  }
  return a;
}

template <int NV>
__device__ __forceinline__ double dot_label(const uint4 (&raw)[NV], const double* qr, float) {
  double a = 0.0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) a = fma(qr[v * 4 + k], double(__uint_as_float(w[k])), a);
  }
  return a;
}

// R > 0: label width known at compile time and R * sizeof(TE) a multiple of 16 bytes.
// R == 0: any width, element loads.
// Label-row append of token t: gather its r channels from K into the label
// cache and return its score.
template <typename TE>
__device__ __forceinline__ float append_row(const TE* __restrict__ Krow, TE* __restrict__ Lrow, const int* sch,
                                            const double* qs, int r) {
  double a = 0.0;
  for (int j = 0; j < r; ++j) {
    const TE v = Krow[sch[j]];
    Lrow[j] = v;
    a = fma(qs[j], double(elem_to_f32(v)), a);
  }
  return float(a);
}

template <typename TE, int R>
__global__ __launch_bounds__(kThreads) void score_kernel(const TE* __restrict__ q, TE* __restrict__ label,
                                                         const TE* __restrict__ Kc, const int32_t* __restrict__ ch,
                                                         int r, int Hq, int Hkv, int64_t T_cap, int64_t T,
                                                         int64_t t_append, int block, float* __restrict__ scores,
                                                         int64_t ld, uint16_t* __restrict__ tile_hist,
                                                         unsigned* __restrict__ tickets, int tickets_per_row) {
  const int64_t row = blockIdx.y;
  if (tickets != nullptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < tickets_per_row; i += kThreads) tickets[row * tickets_per_row + i] = 0u;
  const int b = int(row / Hkv), g = int(row % Hkv);
  const int G = Hq / Hkv;
  TE* L = label + row * T_cap * r;
  const int64_t t0 = int64_t(blockIdx.x) * kTile + threadIdx.x;
  constexpr int NV = R > 0 ? R * int(sizeof(TE)) / 16 : 1;
  // The label rows are requested first: they do not depend on q or the
  // channel table, so their latency overlaps the q-sum below.
  uint4 raw[kTPT][NV];
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      if (t < T && t < t_append) {
        const uint4* p = reinterpret_cast<const uint4*>(L + t * R);
#pragma unroll
        for (int v = 0; v < NV; ++v) raw[i][v] = p[v];
      }
    }
  }
  // The group's q summed over its heads for all 128 channels, and the channel
  // table, are fetched side by side (neither waits for the other); the label
  // channels' sums are then picked out of LDS.
  __shared__ double qall[kHeadDim];
  __shared__ double qs[kHeadDim];
  __shared__ int sch[kHeadDim];
  static_assert(kThreads >= kHeadDim, "one thread per channel");
  if (threadIdx.x < kHeadDim) {
    const TE* qg = q + (int64_t(b) * Hq + int64_t(g) * G) * kHeadDim + threadIdx.x;
    double s = 0.0;
    for (int h = 0; h < G; ++h) s += double(elem_to_f32(qg[int64_t(h) * kHeadDim]));
    qall[threadIdx.x] = s;
  }
  int cj = 0;
  if (threadIdx.x < r) cj = ch[g * r + threadIdx.x];
  __syncthreads();
  if (threadIdx.x < r) {
    qs[threadIdx.x] = qall[cj];
    sch[threadIdx.x] = cj;
  }
  __syncthreads();

  float u[kTPT];
  if constexpr (R > 0) {
    double qr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qr[j] = qs[j];
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      if (t >= T) u[i] = -INFINITY;
      else if (t >= t_append) u[i] = append_row(Kc + (row * T_cap + t) * kHeadDim, L + t * R, sch, qs, R);
      else u[i] = float(dot_label<NV>(raw[i], qr, TE()));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      double a = 0.0;
      if (t < T && t < t_append)
        for (int j = 0; j < r; ++j) a = fma(qs[j], double(elem_to_f32(L[t * r + j])), a);
      if (t >= T) u[i] = -INFINITY;
      else if (t >= t_append) u[i] = append_row(Kc + (row * T_cap + t) * kHeadDim, L + t * r, sch, qs, r);
      else u[i] = float(a);
    }
  }

  float* out = scores + row * ld;
  // Each unit score this thread writes: value and whether it exists.
  float uv[kTPT];
  bool has[kTPT];
  if (block == 1) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      uv[i] = u[i];
      has[i] = t < T;
      if (has[i]) out[t] = u[i];
    }
  } else {
    // 64 consecutive tokens per wavefront, 64-aligned: blocks of `block` lanes.
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      float v = u[i];
      for (int off = block >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      const int64_t t = t0 + i * kThreads;
      uv[i] = v;
      has[i] = t < T && (t % block) == 0;
      if (has[i]) out[t / block] = v;
    }
  }
  if (tile_hist != nullptr) {
    // Dense histogram of the top 11 key bits of this tile's units, every bin
    // written, so the buffer needs no clearing between calls.
    __shared__ uint32_t h[kHistBins];
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTPT; ++i)
      if (has[i]) atomicAdd(&h[float_key(uv[i]) >> 21], 1u);
    __syncthreads();
    constexpr int per = kHistBins / kThreads;   // 8 bins per thread: one 16-byte store
    const int b0 = threadIdx.x * per;
    uint32_t w[per / 2];
#pragma unroll
    for (int j = 0; j < per / 2; ++j) w[j] = h[b0 + 2 * j] | (h[b0 + 2 * j + 1] << 16);
    uint16_t* dst = tile_hist + (row * gridDim.x + blockIdx.x) * kHistBins + b0;
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename TE>
hipError_t dispatch(const TE* q, TE* label, const TE* Kc, const int32_t* ch, int r, int B, int Hq, int Hkv,
                    int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores, int64_t ld,
                    uint16_t* tile_hist, unsigned* tickets, int tickets_per_row, hipStream_t s) {
  const dim3 grid(unsigned((T + kTile - 1) / kTile), unsigned(int64_t(B) * Hkv));
  const bool vec = (int64_t(r) * sizeof(TE)) % 16 == 0;
#define DS_SCORE(RR) \
  hipLaunchKernelGGL((score_kernel<TE, RR>), grid, dim3(kThreads), 0, s, q, label, Kc, ch, r, Hq, Hkv, T_cap, T,     \
                     t_append, block, scores, ld, tile_hist, tickets, tickets_per_row)
  if (vec && r == 8) DS_SCORE(8);
  else if (vec && r == 16) DS_SCORE(16);
  else if (vec && r == 32) DS_SCORE(32);
  else DS_SCORE(0);
#undef DS_SCORE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores(const void* q, void* label, const void* K, const int32_t* ch, int r, int is_bf16, int B,
                         int Hq, int Hkv, int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores,
                         int64_t ld, uint16_t* tile_hist, unsigned* tickets, int tickets_per_row, hipStream_t s) {
  if (is_bf16)
    return dispatch(static_cast<const uint16_t*>(q), static_cast<uint16_t*>(label), static_cast<const uint16_t*>(K),
                    ch, r, B, Hq, Hkv, T_cap, T, t_append, block, scores, ld, tile_hist, tickets, tickets_per_row, s);
  return dispatch(static_cast<const float*>(q), static_cast<float*>(label), static_cast<const float*>(K), ch, r, B,
                  Hq, Hkv, T_cap, T, t_append, block, scores, ld, tile_hist, tickets, tickets_per_row, s);
}

}  // namespace ds
