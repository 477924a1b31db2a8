// Exact softmax attention over given kept units, split along the kept list,
// and the log-sum-exp merge of the splits.
//
// Double Sparsity page, key points and abstract: token sparsity computes
// self-attention with the important tokens only.  Jenga page, core method
// item 3: kept rows are read in place from the original cache by index; no
// reordered copy is ever materialised.
//
// Decode attention is a GEMV per query head, so this runs on the vector ALUs,
// not the matrix cores.  Grid = (split, row = b * Hkv + g, head chunk).  A
// workgroup streams its slice of the kept list: each 16-lane group (bf16; 32
// lanes for fp32) owns one 256-byte K row and one V row per step, four rows per
// group in flight, scores them for every query head of the chunk (the K and V
// rows are read once for the whole GQA group), and keeps a running softmax
// state (max m, sum l, unnormalised acc) that is rescaled once per four rows.
// Lane groups and wavefronts are merged through LDS.  A row with one split
// writes its output directly; otherwise each split writes its state and the
// merge kernel combines them (a kernel boundary orders the two without any
// device-wide cache maintenance inside a kernel).
#include "ds_common.h"

namespace ds {
namespace {

constexpr int kAT = 256;
constexpr int kAW = kAT / 64;
constexpr int kU = 4;   // kept rows per lane group per step

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

template <typename TE>
struct Lanes {
  static constexpr int EPL = 16 / int(sizeof(TE));   // elements per lane: 8 (bf16), 4 (fp32)
  static constexpr int LPT = kHeadDim / EPL;          // lanes per token row: 16, 32
  static constexpr int GPW = 64 / LPT;                // lane groups per wavefront
  static constexpr int NG = kAW * GPW;                // lane groups per workgroup
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

template <typename TE, int HC>
__global__ __launch_bounds__(kAT) void attn_kernel(const TE* __restrict__ q, const TE* __restrict__ K,
                                                   const TE* __restrict__ V, const int32_t* __restrict__ idx,
                                                   int Hq, int Hkv, int64_t T_cap, int64_t T, int block,
                                                   int64_t k_units, int64_t kv_virtual, int64_t chunk, int n_split,
                                                   float scale, float* __restrict__ part_acc,
                                                   float* __restrict__ part_ml, float* __restrict__ out) {
  using LN = Lanes<TE>;
  constexpr int EPL = LN::EPL, LPT = LN::LPT, GPW = LN::GPW, NG = LN::NG;
  const int split = blockIdx.x;
  const uint32_t row = blockIdx.y;
  const uint32_t b = row / uint32_t(Hkv), g = row - b * uint32_t(Hkv);
  const int G = int(uint32_t(Hq) / uint32_t(Hkv));
  const int lb = __builtin_ctz(unsigned(block));
  const int h0 = g * G + int(blockIdx.z) * HC;   // first query head of this chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPT, sub = lane % LPT;
  const int gid = wave * GPW + grp;

  // bf16: q stays packed and q.k runs on v_dot2_f32_bf16 (exact bf16 products,
  // float32 sums), scaled after the lane-group sum; nothing of K is unpacked,
  // which keeps the kernel at four workgroups per CU.  fp32: scaled floats.
  constexpr bool kDot2 = sizeof(TE) == 2;
  uint32_t qp[HC][4];
  float qv[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + (int64_t(b) * Hq + h0 + h) * kHeadDim + sub * EPL);
    qp[h][0] = w.x;
    qp[h][1] = w.y;
    qp[h][2] = w.z;
    qp[h][3] = w.w;
    if constexpr (!kDot2) {
      unpack(w, qv[h], TE());
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[h][e] *= scale;
    }
  }

  float m[HC], l[HC], acc[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int64_t p_begin = int64_t(split) * chunk;
  const int64_t p_end = min(p_begin + chunk, kv_virtual);
  const int32_t* ridx = idx + int64_t(row) * k_units;
  const TE* Kr = K + int64_t(row) * T_cap * kHeadDim + sub * EPL;
  const TE* Vr = V + int64_t(row) * T_cap * kHeadDim + sub * EPL;

  for (int64_t base = p_begin; base < p_end; base += int64_t(NG) * kU) {
    // Every load is issued unconditionally: positions past the slice read the
    // slice's first index, and invalid slots read token 0 (always a real row)
    // and are masked after the load.  A load inside a branch makes the
    // compiler wait for it before the next one is issued.
    int64_t tok[kU];
    bool ok[kU];
    int32_t unit[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t p = base + int64_t(gid) * kU + u;
      ok[u] = p < p_end;
      unit[u] = ridx[(ok[u] ? p : p_begin) >> lb];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t p = base + int64_t(gid) * kU + u;
      tok[u] = (int64_t(unit[u]) << lb) + (p & (block - 1));
      ok[u] = ok[u] && unit[u] >= 0 && tok[u] < T;
      if (!ok[u]) tok[u] = 0;
    }
    uint4 kr[kU], vr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      kr[u] = *reinterpret_cast<const uint4*>(Kr + tok[u] * kHeadDim);
      vr[u] = *reinterpret_cast<const uint4*>(Vr + tok[u] * kHeadDim);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {   // masked rows add nothing, whatever they hold (a bit mask, not a branch)
      const uint32_t keep = ok[u] ? 0xFFFFFFFFu : 0u;
      vr[u].x &= keep;
      vr[u].y &= keep;
      vr[u].z &= keep;
      vr[u].w &= keep;
    }
    float vf[kU][EPL];
#pragma unroll
    for (int u = 0; u < kU; ++u) unpack(vr[u], vf[u], TE());
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float z[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float dsum = 0.f;
        if constexpr (kDot2) {
          const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[h][j]),
                                                   __builtin_bit_cast(bf16x2_t, kw[j]), dsum, false);
          dsum = group_sum<TE>(dsum) * scale;
        } else {
          float kf[EPL];
          unpack(kr[u], kf, TE());
#pragma unroll
          for (int e = 0; e < EPL; ++e) dsum = fmaf(qv[h][e], kf[e], dsum);
          dsum = group_sum<TE>(dsum);
        }
        z[u] = ok[u] ? dsum : -INFINITY;
      }
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < kU; ++u) mx = fmaxf(mx, z[u]);
      if (mx == -INFINITY) continue;   // nothing valid seen yet (uniform across the lane group)
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

  // Merge the NG lane-group states of this workgroup.
  __shared__ float sm_m[NG][HC], sm_l[NG][HC], sm_f[NG][HC];
  __shared__ float sm_M[HC], sm_L[HC];
  __shared__ float sm_acc[NG][HC][kHeadDim];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    if (sub == 0) {
      sm_m[gid][h] = m[h];
      sm_l[gid][h] = l[h];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[gid][h][sub * EPL + e] = acc[h][e];
  }
  __syncthreads();
  if (threadIdx.x < HC) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, sm_m[gg][h]);
    float Ls = 0.f;
    for (int gg = 0; gg < NG; ++gg) {
      const float f = M == -INFINITY ? 0.f : __expf(sm_m[gg][h] - M);
      sm_f[gg][h] = f;
      Ls += sm_l[gg][h] * f;
    }
    sm_M[h] = M;
    sm_L[h] = Ls;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HC * kHeadDim; i += kAT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    float A = 0.f;
    for (int gg = 0; gg < NG; ++gg) A = fmaf(sm_acc[gg][h][c], sm_f[gg][h], A);
    const int64_t bh = int64_t(b) * Hq + h0 + h;
    if (n_split == 1) {
      out[bh * kHeadDim + c] = A / sm_L[h];
    } else {
      part_acc[(bh * n_split + split) * kHeadDim + c] = A;
      if (c == 0) {
        part_ml[(bh * n_split + split) * 2 + 0] = sm_M[h];
        part_ml[(bh * n_split + split) * 2 + 1] = sm_L[h];
      }
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, query head).  kMergeSG
// groups of one thread per channel each take every kMergeSG-th split, with all
// of a batch's values requested before any is used, and the groups' partial
// states are combined through LDS: 64 splits are one batch of loads.
constexpr int kMergeBatch = 16;
constexpr int kMergeSG = 4;

__global__ __launch_bounds__(kHeadDim * kMergeSG) void merge_kernel(const float* __restrict__ part_acc,
                                                                    const float* __restrict__ part_ml,
                                                                    int n_split, float* __restrict__ out) {
  __shared__ float sm_m[kMergeSG][kHeadDim], sm_l[kMergeSG][kHeadDim], sm_a[kMergeSG][kHeadDim];
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x % kHeadDim, sg = threadIdx.x / kHeadDim;
  const float* ml = part_ml + bh * n_split * 2;
  const float* pa = part_acc + bh * n_split * kHeadDim + c;
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int s0 = sg; s0 < n_split; s0 += kMergeSG * kMergeBatch) {
    float a[kMergeBatch], m[kMergeBatch], l[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int sp = s0 + j * kMergeSG;
      const bool ok = sp < n_split;
      const int sc = ok ? sp : sg;   // clamped: every load is issued, masked after
      a[j] = pa[int64_t(sc) * kHeadDim];
      m[j] = ml[2 * sc];
      l[j] = ml[2 * sc + 1];
      if (!ok) m[j] = -INFINITY;
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, m[j]);
    if (Mb == -INFINITY) continue;
    const float r = __expf(M - Mb);   // M = -inf: 0
    L *= r;
    A *= r;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float f = __expf(m[j] - Mb);   // empty or masked split (m = -inf): 0
      L = fmaf(l[j], f, L);
      A = fmaf(a[j], f, A);
    }
    M = Mb;
  }
  sm_m[sg][c] = M;
  sm_l[sg][c] = L;
  sm_a[sg][c] = A;
  __syncthreads();
  if (sg == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < kMergeSG; ++g) Mt = fmaxf(Mt, sm_m[g][c]);
    float Lt = 0.f, At = 0.f;
#pragma unroll
    for (int g = 0; g < kMergeSG; ++g) {
      const float f = sm_m[g][c] == -INFINITY ? 0.f : __expf(sm_m[g][c] - Mt);
      Lt = fmaf(sm_l[g][c], f, Lt);
      At = fmaf(sm_a[g][c], f, At);
    }
    out[bh * kHeadDim + c] = At / Lt;
  }
}

template <typename TE>
hipError_t dispatch(const TE* q, const TE* K, const TE* V, int Hq, int Hkv, int64_t T_cap, int64_t T, int block,
                    int64_t k_units, const int32_t* idx, float scale, int64_t rows, int64_t kv_virtual,
                    const SplitPlan& sp, float* part_acc, float* part_ml, float* out, hipStream_t s) {
  const dim3 grid(unsigned(sp.n_split), unsigned(rows), unsigned(sp.head_chunks));
#define DS_ATTN(HH)                                                                                              \
  hipLaunchKernelGGL((attn_kernel<TE, HH>), grid, dim3(kAT), 0, s, q, K, V, idx, Hq, Hkv, T_cap, T, block,       \
                     k_units, kv_virtual, sp.chunk, sp.n_split, scale, part_acc, part_ml, out)
  if (sp.head_chunk == 8) DS_ATTN(8);
  else if (sp.head_chunk == 4) DS_ATTN(4);
  else if (sp.head_chunk == 2) DS_ATTN(2);
  else DS_ATTN(1);
#undef DS_ATTN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const void* q, const void* K, const void* V, int is_bf16, int B, int Hq, int Hkv,
                            int64_t T_cap, int64_t T, int block, int64_t k_units, const int32_t* idx, float scale,
                            int64_t kv_virtual, const SplitPlan& sp, float* part_acc, float* part_ml, float* out,
                            hipStream_t s) {
  const int64_t rows = int64_t(B) * Hkv;
  if (is_bf16)
    return dispatch(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                    Hq, Hkv, T_cap, T, block, k_units, idx, scale, rows, kv_virtual, sp, part_acc, part_ml, out, s);
  return dispatch(static_cast<const float*>(q), static_cast<const float*>(K), static_cast<const float*>(V), Hq, Hkv,
                  T_cap, T, block, k_units, idx, scale, rows, kv_virtual, sp, part_acc, part_ml, out, s);
}

__global__ void zero_u32_kernel(unsigned* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(unsigned(want < 1024 ? want : 1024)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_acc, const float* part_ml, int64_t BH, int n_split, float* out,
                        hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(BH)), dim3(kHeadDim * kMergeSG), 0, s, part_acc, part_ml, n_split,
                     out);
  return hipGetLastError();
}

}  // namespace ds
