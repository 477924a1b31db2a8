// Clock stamps for per-phase timelines of the decode kernels.
//
// Compiled in only with -DDS_STAMPS (build.py --stamps builds that variant of
// the library beside the ordinary one); otherwise every macro below is empty
// and the kernels are unchanged.  Thread 0 of a workgroup stores the shader
// clock (s_memtime, core cycles) at a numbered point; slot 0 holds the 100 MHz
// constant clock (s_memrealtime) at the workgroup's start, slot 1 the shader
// clock there, slot 31 the constant clock at its end.  Each stamped source
// file keeps its own buffer (no relocatable device code across files), indexed
// by the workgroup's linear id; a launch overwrites the previous one's stamps.
// The host reads a buffer with ds_stamps_dump_<name>(host pointer,
// kStampWgs * kStampSlots 64-bit words); slots never written in a launch keep
// old contents, so the host clears the buffer (ds_stamps_clear_<name>) before
// the launch it reads.
#pragma once

#include <hip/hip_runtime.h>

namespace ds {
constexpr int kStampWgs = 4096;    // workgroups stamped per launch (linear ids below this)
constexpr int kStampSlots = 32;
}  // namespace ds

#ifdef DS_STAMPS

#define DS_STAMP_BUFFER(name)                                                                            \
  __device__ unsigned long long ds_stamps_##name[ds::kStampWgs * ds::kStampSlots];                       \
  extern "C" int ds_stamps_dump_##name(void* host) {                                                     \
    return int(hipMemcpyFromSymbol(host, HIP_SYMBOL(ds_stamps_##name), sizeof(ds_stamps_##name)));       \
  }                                                                                                      \
  extern "C" int ds_stamps_clear_##name() {                                                              \
    void* p = nullptr;                                                                                   \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(ds_stamps_##name));                                \
    if (e == hipSuccess) e = hipMemset(p, 0, sizeof(ds_stamps_##name));                                  \
    if (e == hipSuccess) e = hipDeviceSynchronize();                                                     \
    return int(e);                                                                                       \
  }

#define DS_STAMP_AT_(name, slot, clock)                                                                   \
  do {                                                                                                   \
    if (threadIdx.x == 0) {                                                                              \
      const unsigned ds_w_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);            \
      if (ds_w_ < unsigned(ds::kStampWgs)) ds_stamps_##name[ds_w_ * ds::kStampSlots + (slot)] = clock;   \
    }                                                                                                    \
  } while (0)

#define DS_STAMP(name, slot) DS_STAMP_AT_(name, slot, __builtin_amdgcn_s_memtime())
#define DS_STAMP_START(name)                                          \
  do {                                                                \
    DS_STAMP_AT_(name, 0, __builtin_amdgcn_s_memrealtime());          \
    DS_STAMP_AT_(name, 1, __builtin_amdgcn_s_memtime());              \
  } while (0)
#define DS_STAMP_END(name) DS_STAMP_AT_(name, 31, __builtin_amdgcn_s_memrealtime())

#else

#define DS_STAMP_BUFFER(name)
#define DS_STAMP(name, slot) \
  do {                       \
  } while (0)
#define DS_STAMP_START(name) \
  do {                       \
  } while (0)
#define DS_STAMP_END(name) \
  do {                     \
  } while (0)

#endif
