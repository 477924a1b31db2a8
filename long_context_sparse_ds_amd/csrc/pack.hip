// Label-cache pack: label[b, g, t, j] = K[b, g, t, ch[g, j]] for t in [t_begin, t_end).
//
// Double Sparsity page, abstract: only the important channels of K are needed
// to identify the important tokens, so they are gathered once into a compact
// [B, Hkv, T_cap, r] row per token that the per-step score scan streams.
//
// Grid = (64-token tiles, row = b * Hkv + g); four lanes per token, each
// gathering every fourth label channel from the token's 256-byte K row (one
// cache-line fetch serves the token's lanes).  32-bit index math: T < 2^31 is
// checked on the host.
#include "ds_common.h"

namespace ds {
namespace {

constexpr int kPackTokens = 64;   // tokens per 256-thread workgroup

template <typename TE>
__global__ __launch_bounds__(256) void pack_kernel(const TE* __restrict__ K, int Hkv, int64_t T_cap,
                                                   const int32_t* __restrict__ ch, int r, int t_begin, int t_end,
                                                   TE* __restrict__ label) {
  const uint32_t row = blockIdx.y;
  const uint32_t g = row % uint32_t(Hkv);
  const int t = t_begin + int(blockIdx.x) * kPackTokens + int(threadIdx.x >> 2);
  if (t >= t_end) return;
  const TE* Kr = K + (int64_t(row) * T_cap + t) * kHeadDim;
  TE* Lr = label + (int64_t(row) * T_cap + t) * r;
  const int32_t* cg = ch + int64_t(g) * r;
  for (int j = int(threadIdx.x & 3); j < r; j += 4) Lr[j] = Kr[cg[j]];
}

}  // namespace

hipError_t launch_pack(const void* K, int is_bf16, int B, int Hkv, int64_t T_cap, const int32_t* ch, int r,
                       int64_t t_begin, int64_t t_end, void* label, hipStream_t s) {
  const int64_t n_tok = t_end - t_begin;
  if (n_tok <= 0) return hipSuccess;
  const dim3 grid(unsigned((n_tok + kPackTokens - 1) / kPackTokens), unsigned(int64_t(B) * Hkv));
  if (is_bf16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(K), Hkv, T_cap, ch,
                       r, int(t_begin), int(t_end), static_cast<uint16_t*>(label));
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(K), Hkv, T_cap, ch, r,
                       int(t_begin), int(t_end), static_cast<float*>(label));
  return hipGetLastError();
}

}  // namespace ds
