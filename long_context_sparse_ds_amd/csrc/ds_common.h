// Internal declarations shared by the host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ds {

constexpr int kHeadDim = 128;

// How one decode call is laid out on the device.  Computed identically by the
// workspace query and by the launch, from the shape alone.
struct DecodePlan {
  int64_t rows;        // B * Hkv selection rows
  int64_t n_units;     // ceil(T / block)
  int64_t score_ld;    // row stride of the score buffer, floats (multiple of 64)
  int64_t kv_virtual;  // k_units * block: attention positions per row (some may lie past T)
  int64_t chunk;       // positions per split
  int n_split;         // splits per row
  size_t off_scores, off_acc, off_ml, total_bytes;
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int64_t T, int block, int64_t k_units);

// Kernel launchers (enqueue only; return the launch status).
hipError_t launch_pack(const void* K, int is_bf16, int B, int Hkv, int64_t T_cap, const int32_t* ch, int r,
                       int64_t t_begin, int64_t t_end, void* label, hipStream_t s);

hipError_t launch_scores(const void* q, const void* label, const int32_t* ch, int r, int is_bf16, int B, int Hq,
                         int Hkv, int64_t T_cap, int64_t T, int block, float* scores, int64_t ld, hipStream_t s);

hipError_t launch_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx,
                         hipStream_t s);

hipError_t launch_attention(const void* q, const void* K, const void* V, int is_bf16, int B, int Hq, int Hkv,
                            int64_t T_cap, int64_t T, int block, int64_t k_units, const int32_t* idx, float scale,
                            const DecodePlan& plan, float* part_acc, float* part_ml, float* out, hipStream_t s);

}  // namespace ds

#ifdef __HIPCC__
namespace ds {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ float elem_to_f32(uint16_t h) { return bf16_to_f32(h); }
__device__ __forceinline__ float elem_to_f32(float f) { return f; }

// Order-preserving map float -> uint32: a > b as floats iff key(a) > key(b)
// as integers; -0.0 is folded onto +0.0.  Finite values map to >= 0x00800000,
// so 0 is a safe "below everything" sentinel.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP lane moves within a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppRor4>(v);
  v += dpp_f32<kDppRor8>(v);
  return v;
}

}  // namespace ds
#endif
