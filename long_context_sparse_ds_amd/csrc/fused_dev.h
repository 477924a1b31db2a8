// Device pieces shared by the fused select + attention kernels: the lane
// layout of a K/V row gather, the radix digit pick over an LDS histogram, and
// the softmax-state merges across lane groups.
#pragma once

#include "select_dev.h"

namespace ds {
namespace {

// Operand and accumulator types of the matrix-core instructions.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short bf16x4_t;   // four bf16 bit patterns
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// A float rounded to the nearest bf16, ties to even, as its 16-bit pattern in
// the low half (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <typename TE, int NT>
struct Lanes {
  static constexpr int NW = NT / 64;                  // wavefronts
  static constexpr int EPL = 16 / int(sizeof(TE));   // elements per lane: 8 (bf16), 4 (fp32)
  static constexpr int LPT = kHeadDim / EPL;          // lanes per 128-wide row: 16, 32
  static constexpr int GPW = 64 / LPT;                // lane groups per wavefront
  static constexpr int NG = NW * GPW;                 // lane groups per workgroup
  static constexpr int KU = NT >= 1024 ? 2 : 4;       // kept rows per lane group per step
};

// Inverse of float_key for keys of non-NaN floats.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Thread t of NT owns bins [NB - BPT * (t + 1), NB - BPT * t) of an NB-bin
// histogram, highest first, so thread order is descending digit order.  c[i]
// is the count of bin NB - 1 - BPT * t - i.  With the workgroup prefix sum of
// the per-thread totals, the thread whose bins hold the kk-th largest key
// stores (digit, count above it, count in it) to out.  The caller passes a
// barrier before reading out.  `extra` (a per-thread count) is summed over the
// workgroup in the same prefix sum, in the high 16 bits (every total here is at
// most 32768), and its workgroup total is returned.
template <int NT, int NB>
__device__ __forceinline__ uint32_t pick_bin(const uint32_t (&c)[NB / NT], uint32_t kk, uint32_t* wsum, uint32_t* out,
                                             uint32_t extra = 0u) {
  constexpr int BPT = NB / NT;
  uint32_t sum = 0u;
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += c[i];
  uint32_t tot;
  uint32_t above = block_exclusive_scan1<NT>(sum | (extra << 16), wsum, tot) & 0xFFFFu;
  if (above < kk && above + sum >= kk) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (above < kk && above + c[i] >= kk) {
        out[0] = uint32_t(NB - 1 - BPT * int(threadIdx.x) - i);
        out[1] = above;
        out[2] = c[i];
      }
      above += c[i];
    }
  }
  return tot >> 16;
}

// Counts of this thread's bins of an LDS histogram, highest first.
template <int NT, int NB>
__device__ __forceinline__ void read_bins(const uint32_t* hist, uint32_t (&c)[NB / NT]) {
  constexpr int BPT = NB / NT;
  const int lo = NB - BPT * (int(threadIdx.x) + 1);
#pragma unroll
  for (int i = 0; i < BPT; ++i) c[i] = hist[lo + BPT - 1 - i];
}

template <typename TE>
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[8], TE) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[4], float) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

template <typename TE, int NT>
__device__ __forceinline__ float group_sum(float v) {
  v = row16_sum(v);
  if constexpr (Lanes<TE, NT>::LPT == 32) v += __shfl_xor(v, 16);
  return v;
}

// The values of a pair of lane groups: with OFF = 16, rows 0-1 and rows 2-3 of
// the wavefront (v_permlane16_swap); with OFF = 32, its two halves
// (v_permlane32_swap).  Both lanes of a pair receive the same two values, so a
// symmetric combination of them leaves the pair holding one identical result.
template <int OFF>
__device__ __forceinline__ void pair_values(float v, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// Merge the softmax states (m, l, acc) of the lane-group pairs OFF lanes apart.
template <int OFF, int HC, int EPL>
__device__ __forceinline__ void merge_pairs(float (&m)[HC], float (&l)[HC], float (&acc)[HC][EPL]) {
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    float ma, mb, la, lb;
    pair_values<OFF>(m[h], ma, mb);
    pair_values<OFF>(l[h], la, lb);
    const float M = fmaxf(ma, mb);
    const float fa = ma == -INFINITY ? 0.f : __expf(ma - M);
    const float fb = mb == -INFINITY ? 0.f : __expf(mb - M);
    l[h] = la * fa + lb * fb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float xa, xb;
      pair_values<OFF>(acc[h][e], xa, xb);
      acc[h][e] = xa * fa + xb * fb;
    }
    m[h] = M;
  }
}

}  // namespace
}  // namespace ds
