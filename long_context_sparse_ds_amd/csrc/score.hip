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
#include "ds_common.h"

namespace ds {
namespace {

constexpr int kThreads = 256;
constexpr int kTPT = 4;                     // tokens per thread
constexpr int kTile = kThreads * kTPT;      // tokens per workgroup

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
template <typename TE, int R>
__global__ __launch_bounds__(kThreads) void score_kernel(const TE* __restrict__ q, const TE* __restrict__ label,
                                                         const int32_t* __restrict__ ch, int r, int Hq, int Hkv,
                                                         int64_t T_cap, int64_t T, int block,
                                                         float* __restrict__ scores, int64_t ld) {
  const int64_t row = blockIdx.y;
  const int b = int(row / Hkv), g = int(row % Hkv);
  const int G = Hq / Hkv;
  __shared__ double qs[kHeadDim];
  for (int j = threadIdx.x; j < r; j += kThreads) {
    const int c = ch[g * r + j];
    double s = 0.0;
    for (int h = 0; h < G; ++h) s += double(elem_to_f32(q[(int64_t(b) * Hq + int64_t(g) * G + h) * kHeadDim + c]));
    qs[j] = s;
  }
  __syncthreads();

  const TE* L = label + row * T_cap * r;
  const int64_t t0 = int64_t(blockIdx.x) * kTile + threadIdx.x;
  float u[kTPT];
  if constexpr (R > 0) {
    constexpr int NV = R * int(sizeof(TE)) / 16;
    double qr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qr[j] = qs[j];
    uint4 raw[kTPT][NV];
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      if (t < T) {
        const uint4* p = reinterpret_cast<const uint4*>(L + t * R);
#pragma unroll
        for (int v = 0; v < NV; ++v) raw[i][v] = p[v];
      }
    }
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      u[i] = t < T ? float(dot_label<NV>(raw[i], qr, TE())) : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      double a = 0.0;
      if (t < T)
        for (int j = 0; j < r; ++j) a = fma(qs[j], double(elem_to_f32(L[t * r + j])), a);
      u[i] = t < T ? float(a) : -INFINITY;
    }
  }

  float* out = scores + row * ld;
  if (block == 1) {
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      const int64_t t = t0 + i * kThreads;
      if (t < T) out[t] = u[i];
    }
  } else {
    // 64 consecutive tokens per wavefront, 64-aligned: blocks of `block` lanes.
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
      float v = u[i];
      for (int off = block >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      const int64_t t = t0 + i * kThreads;
      if (t < T && (t % block) == 0) out[t / block] = v;
    }
  }
}

template <typename TE>
hipError_t dispatch(const TE* q, const TE* label, const int32_t* ch, int r, int B, int Hq, int Hkv,
                    int64_t T_cap, int64_t T, int block, float* scores, int64_t ld, hipStream_t s) {
  const dim3 grid(unsigned((T + kTile - 1) / kTile), unsigned(int64_t(B) * Hkv));
  const bool vec = (int64_t(r) * sizeof(TE)) % 16 == 0;
#define DS_SCORE(RR) \
  hipLaunchKernelGGL((score_kernel<TE, RR>), grid, dim3(kThreads), 0, s, q, label, ch, r, Hq, Hkv, T_cap, T, block, \
                     scores, ld)
  if (vec && r == 8) DS_SCORE(8);
  else if (vec && r == 16) DS_SCORE(16);
  else if (vec && r == 32) DS_SCORE(32);
  else DS_SCORE(0);
#undef DS_SCORE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores(const void* q, const void* label, const int32_t* ch, int r, int is_bf16, int B, int Hq,
                         int Hkv, int64_t T_cap, int64_t T, int block, float* scores, int64_t ld, hipStream_t s) {
  if (is_bf16)
    return dispatch(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(label), ch, r, B, Hq, Hkv, T_cap,
                    T, block, scores, ld, s);
  return dispatch(static_cast<const float*>(q), static_cast<const float*>(label), ch, r, B, Hq, Hkv, T_cap, T,
                  block, scores, ld, s);
}

}  // namespace ds
