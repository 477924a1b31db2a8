// Internal declarations shared by the host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "stamps.h"

namespace ds {

constexpr int kHeadDim = 128;
// MI355X: 8 XCDs, each with its own L2.  Workgroups are dealt to the XCDs
// round-robin by linear id, so in a grid (8, Y, Z) blockIdx.x is the XCD.
constexpr int kXcds = 8;

// Rows of up to this many units take the fused select+attention kernel, whose
// workgroups (1024 threads) hold a whole score row in registers.
constexpr int64_t kFusedMaxUnits = 32768;
// Kept positions handled by one fused split (its LDS list of unit ids).
constexpr int64_t kFusedMaxChunk = 4096;
// Tokens per score-kernel workgroup (one "tile"); a row's tile histograms are
// summed by the fused kernel when a row has at most kMaxHistTiles tiles.
constexpr int64_t kScoreTile = 2048;
constexpr int64_t kMaxHistTiles = 16;
constexpr int kHistBins = 2048;   // top 11 bits of a score key
// Units per score tile of token-level rows (the tile histograms' granularity).
constexpr int64_t kHistTileUnits = kScoreTile;

// Units per partition of the two-stage selection of long rows (the top k of
// each partition, then the top k of those candidates in the fused kernel).
constexpr int64_t kPartUnits = 32768;

// Query heads processed together by one attention workgroup (divides G).
inline __host__ __device__ int head_chunk8(int G) { return G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }
inline __host__ __device__ int head_chunk4(int G) { return G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }

// How the kept positions of each row are split over attention workgroups.
struct SplitPlan {
  int64_t chunk;     // virtual kept positions per split (multiple of 64 and of the block size)
  int n_split;       // splits per row
  int head_chunk;    // query heads per workgroup
  int head_chunks;   // G / head_chunk
};

// How one decode call is laid out on the device.  Computed identically by the
// workspace query and by the launches, from the shape alone.
struct DecodePlan {
  int64_t rows;        // B * Hkv selection rows
  int64_t n_units;     // ceil(T / block)
  int64_t score_ld;    // row stride of the score buffer, floats (multiple of 64)
  int64_t kv_virtual;  // k_units * block: attention positions per row (some may lie past T)
  bool fused;          // select and attention in one kernel
  bool partitioned;    // longer rows: per-partition top k, then the fused kernel over the candidates
  int64_t n_cand;      // partitioned: candidates per row (partitions * k_units)
  int64_t cand_ld;     // partitioned: row stride of the candidate scores, floats (multiple of 64)
  bool cand_hist;      // partitioned: the first stage writes its candidates' top-digit histograms
  bool part_onepass;   // partitioned token-level rows: the first stage scores the label cache itself (the
                       // decode step's score phase), so no score buffer or tile histograms are written
  bool tile_hist;      // the score kernel writes per-tile key histograms for the fused kernel
  bool bucketed;       // token-level rows over several fused workgroups: sorted tile lists and the
                       // bucket kernel (for the plain top-k step; ragged and threshold calls keep the
                       // histogram form)
  int64_t tiles;       // score tiles per row
  SplitPlan sp;        // splits of the decode call
  SplitPlan sp_idx;    // splits of the attention-from-indices call
  size_t off_scores, off_tile_hist, off_acc, off_ml, off_tickets, off_cand_score, off_cand_id,
      off_cand_hist, total_bytes;
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int64_t T, int block, int64_t k_units);

// Kernel launchers (enqueue only; return the launch status).
hipError_t launch_pack(const void* K, int is_bf16, int B, int Hkv, int64_t T_cap, const int32_t* ch, int r,
                       int64_t t_begin, int64_t t_end, void* label, hipStream_t s);

// Scores of units [0, ceil(T/block)).  Rows [t_append, T) of the label cache
// are first rebuilt from K (label-row append); pass t_append = T to skip, and
// K may then be null.  tile_hist (may be null): uint16 [rows][tiles][2048]
// histogram of the top 11 key bits of each tile's units.  tickets (may be
// null): tickets_per_row merge tickets per row, zeroed here for the fused
// kernel that follows.
// seq_lens (may be null): device int32 [B]; sequence b then holds seq_lens[b]
// tokens (clamped to [1, T]), its last n_append rows are rebuilt (t_append is
// ignored), and its scores past its length are written as -inf up to T.
// sorted (token-level rows, not ragged or positive, tile_hist given): the
// sorted-list form.  Tile i of a row writes its units in descending order of
// top score digit, as 32-bit words (score key bits 20..0 above the 11-bit
// tile-local id) at ((uint32_t*)scores)[row * ld + 2048 i + e]; tile_hist then
// holds each tile's exclusive descending prefix P[b] (units whose top digit
// exceeds b) instead of counts.
hipError_t launch_scores(const void* q, void* label, const void* K, const int32_t* ch, int r, int is_bf16, int B,
                         int Hq, int Hkv, int64_t T_cap, int64_t T, int64_t t_append, int block, float* scores,
                         int64_t ld, uint16_t* tile_hist, unsigned* tickets, int tickets_per_row,
                         const int32_t* seq_lens, int n_append, bool positive, hipStream_t s,
                         bool sorted = false);

hipError_t launch_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx,
                         hipStream_t s);

// Per-partition top k of rows longer than kPartUnits: candidates [rows][parts * k]
// (scores with row stride cand_ld, unit ids with row stride parts * k), in
// ascending unit order; unused slots hold -inf and -1.
// tile_hist (may be null): the score kernel's tile histograms (token-level rows,
// tiles per row); cand_hist (may be null; needs tile_hist): the candidates'
// top-digit histograms [rows][parts][2048] for the fused kernel.
hipError_t launch_partition_topk(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k,
                                 float* cand_score, int64_t cand_ld, int32_t* cand_id, const uint16_t* tile_hist,
                                 int64_t tiles, uint16_t* cand_hist, hipStream_t s);

// The same first stage in one pass over the label cache, for token-level rows
// (block 1): each partition is scored from its label rows (rows [t_append, T)
// rebuilt from K first), with the score kernel's arithmetic, and its top k and
// the candidates' top-digit histogram (cand_hist, may be null) written as by
// launch_partition_topk.  No score buffer is written.  tickets (may be null):
// tickets_per_row merge tickets per row, zeroed for the fused kernel that follows.
hipError_t launch_partition_onepass(const void* q, void* label, const void* K, const int32_t* ch, int r, int is_bf16,
                                    int B, int Hq, int Hkv, int64_t T_cap, int64_t T, int64_t t_append, int64_t k,
                                    float* cand_score, int64_t cand_ld, int32_t* cand_id, uint16_t* cand_hist,
                                    unsigned* tickets, int tickets_per_row, hipStream_t s);

// Attention over given kept units; writes out directly when sp.n_split == 1,
// else partial states that launch_merge combines.
hipError_t launch_attention(const void* q, const void* K, const void* V, int is_bf16, int B, int Hq, int Hkv,
                            int64_t T_cap, int64_t T, int block, int64_t k_units, const int32_t* idx, float scale,
                            int64_t kv_virtual, const SplitPlan& sp, float* part_acc, float* part_ml, float* out,
                            hipStream_t s);

// Fused selection + attention (rows of at most kFusedMaxUnits units).
// tile_hist (may be null): the score kernel's per-tile histograms of this call.
// tickets: rows * sp.head_chunks merge tickets, zero on entry (left zero).
// seq_lens (may be null): device int32 [B]; sequence b holds seq_lens[b] tokens
// (clamped to [1, T]), keeps min(k_units, its unit count) units, and its index
// slots past that are set to -1.
// unit_ids (may be null): the scores are candidates [rows][pl.n_units] whose
// unit ids these are (ascending per row); kept candidates are written and
// gathered as those units.
// one (may be null): the one-pass form, for token-level rows that one
// workgroup handles alone (pl.sp.n_split == 1, pl.sp.head_chunks == 1) and
// label rows of 16 or 32 bytes (64 for fp32): the kernel scores each row from the label
// cache itself (rebuilding rows [t_append, T), or the last n_append of each
// sequence, from K first) and scores / tile_hist are not read.
struct OnePass {
  void* label;        // [B, Hkv, T_cap, r]
  const int32_t* ch;  // [Hkv, r]
  int r;
  int64_t t_append;
  int n_append;
};
hipError_t launch_select_attention(const void* q, const void* K, const void* V, int is_bf16, const float* scores,
                                   int64_t ld, const uint16_t* tile_hist, int Hq, int Hkv, int64_t T_cap, int64_t T,
                                   int block, int64_t k_units, float scale, const DecodePlan& pl, int32_t* indices,
                                   float* part_acc, float* part_ml, float* out, unsigned* tickets,
                                   const int32_t* seq_lens, float tau, int32_t* counts,
                                   const int32_t* unit_ids, hipStream_t s, const OnePass* one = nullptr);

// Selection + attention of token-level rows from the score kernel's sorted
// tile lists (pl.bucketed): per (row, head chunk, split), the top digit from
// the tiles' prefixes, the boundary digit's candidates refined to the exact
// threshold, this split's share of the kept tokens gathered and attended, its
// tiles' slices of the ascending index list written, and the splits merged.
// tickets: rows * head_chunks merge tickets, zero on entry (left zero).
hipError_t launch_bucket_attention(const void* q, const void* K, const void* V, int is_bf16, const uint32_t* slist,
                                   const uint16_t* tprefix, int Hq, int Hkv, int64_t T_cap,
                                   int64_t k_units, float scale, const DecodePlan& pl, int32_t* indices,
                                   float* part_acc, float* part_ml, float* out, unsigned* tickets, hipStream_t s);

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s);

// Hierarchical span search (rows of B * Hkv, k <= 1024 spans): writes the kept
// spans [rows][k][2] and the covered token ids [rows][cap], ascending, -1 after.
hipError_t launch_hip_search(const void* q, const void* K, int is_bf16, int B, int Hq, int Hkv, int64_t T_cap,
                             int64_t T, int k, int span, int rounds, int32_t* spans, int32_t* tokens, int64_t cap,
                             hipStream_t s);

// Log-sum-exp merge of n_split partial states per (sequence, query head).
hipError_t launch_merge(const float* part_acc, const float* part_ml, int64_t BH, int n_split, float* out,
                        hipStream_t s);

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

// Maximum over the 16 lanes of a DPP row; every lane of the row receives it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRor8>(v));
  return v;
}

}  // namespace ds
#endif
