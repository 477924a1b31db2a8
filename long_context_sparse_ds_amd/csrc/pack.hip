// Label-cache pack: label[b, g, t, j] = K[b, g, t, ch[g, j]] for t in [t_begin, t_end).
//
// Double Sparsity page, abstract: only the important channels of K are needed
// to identify the important tokens, so they are gathered once into a compact
// [B, Hkv, T_cap, r] row per token that the per-step score scan streams.
//
// One thread per label element: consecutive threads write consecutive label
// elements (coalesced stores); the reads of one wavefront touch a few 256-byte
// K rows, which the cache line fetch brings in whole.
#include "ds_common.h"

namespace ds {
namespace {

template <typename TE>
__global__ __launch_bounds__(256) void pack_kernel(const TE* __restrict__ K, int Hkv, int64_t T_cap,
                                                   const int32_t* __restrict__ ch, int r, int64_t t_begin,
                                                   int64_t n_tok, int64_t total, TE* __restrict__ label) {
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t j = e % r;
    const int64_t rt = e / r;            // row * n_tok + token offset
    const int64_t row = rt / n_tok;      // b * Hkv + g
    const int64_t t = t_begin + rt % n_tok;
    const int g = int(row % Hkv);
    const int c = ch[g * r + j];
    label[(row * T_cap + t) * r + j] = K[(row * T_cap + t) * kHeadDim + c];
  }
}

}  // namespace

hipError_t launch_pack(const void* K, int is_bf16, int B, int Hkv, int64_t T_cap, const int32_t* ch, int r,
                       int64_t t_begin, int64_t t_end, void* label, hipStream_t s) {
  const int64_t n_tok = t_end - t_begin;
  const int64_t total = int64_t(B) * Hkv * n_tok * r;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = unsigned(want < 65536 ? want : 65536);
  if (is_bf16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(K), Hkv,
                       T_cap, ch, r, t_begin, n_tok, total, static_cast<uint16_t*>(label));
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(K), Hkv, T_cap,
                       ch, r, t_begin, n_tok, total, static_cast<float*>(label));
  return hipGetLastError();
}

}  // namespace ds
