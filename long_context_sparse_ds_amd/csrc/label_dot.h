// The approximate score of one token from its label row, shared by the score
// kernel and the fused kernel's one-pass form so that both give the same
// float32 value bit for bit.
//
// Double Sparsity page, method details: the score of token t for KV head g is
// sum_j qs[j] * label[t, j], with qs[j] the group's q summed over its heads at
// channel ch[g, j].  A bf16 x bf16 or fp32 x fp32 product is exact in double,
// and the r products are accumulated in double in channel order, so the score
// is the exact value rounded once to float32 (up to the double rounding of the
// running sum).
#pragma once

#include "ds_common.h"

namespace ds {

// qs at channel c: the group's q summed in head order from +0.0, which is the
// score kernel's sum for groups of up to eight heads (it adds any heads past
// the eighth first).
template <typename TE>
__device__ __forceinline__ double group_q_sum(const TE* __restrict__ qg, int G, int c) {
  double s = 0.0;
  for (int h = 0; h < G; ++h) s += double(elem_to_f32(qg[int64_t(h) * kHeadDim + c]));
  return s;
}

// qs at channel c in the score kernel's own order for any group size (the
// heads past the eighth first, then heads 0 .. 7: group_q_sum's result for
// groups of up to eight heads), in two steps so that other requests can go
// out between the loads and the additions: q_load8 requests the first eight
// heads' values together (a loop over a run-time head count would wait for
// each), q_score_sum adds them, reading any further heads itself.
template <typename TE>
__device__ __forceinline__ void q_load8(const TE* __restrict__ qg, int G, int c, float (&v)[8]) {
#pragma unroll
  for (int h = 0; h < 8; ++h) v[h] = elem_to_f32(qg[int64_t(h < G ? h : 0) * kHeadDim + c]);
}

template <typename TE>
__device__ __forceinline__ double q_score_sum(const float (&v)[8], const TE* __restrict__ qg, int G, int c) {
  double s = 0.0;
  for (int h = 8; h < G; ++h) s += double(elem_to_f32(qg[int64_t(h) * kHeadDim + c]));
#pragma unroll
  for (int h = 0; h < 8; ++h)
    if (h < G) s += double(v[h]);
  return s;
}

// NV 16-byte words of one label row against qr[0 .. 8 NV) (bf16) or
// qr[0 .. 4 NV) (fp32), in channel order.
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

// Label-row append of token t: gather its r channels from its K row (a staged
// copy in LDS, or global memory) into the label cache and return its score,
// accumulated in the same channel order as dot_label.
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

// append_row's score alone (same arithmetic), for a caller that stores the
// label row later.
template <typename TE>
__device__ __forceinline__ float append_score(const TE* __restrict__ Krow, const int* sch, const double* qs, int r) {
  double a = 0.0;
  for (int j = 0; j < r; ++j) a = fma(qs[j], double(elem_to_f32(Krow[sch[j]])), a);
  return float(a);
}

// append_row for a label width R known at compile time: every channel is
// requested before any is used (one round trip), with the same arithmetic.
template <int R, typename TE>
__device__ __forceinline__ float append_row_n(const TE* __restrict__ Krow, TE* __restrict__ Lrow, const int* sch,
                                              const double* qs) {
  TE v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = Krow[sch[j]];
  double a = 0.0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    Lrow[j] = v[j];
    a = fma(qs[j], double(elem_to_f32(v[j])), a);
  }
  return float(a);
}

}  // namespace ds
