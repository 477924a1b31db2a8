// C ABI entry points: argument validation, workspace planning, kernel launches.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and writes nothing.  No C++ exception leaves this file.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "ds.h"
#include "ds_common.h"

namespace {

thread_local std::string g_err;

ds_status fail(ds_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_block(int block) { return block >= 1 && block <= 64 && (block & (block - 1)) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

ds_status check_dtype(ds_dtype dt) {
  if (dt != DS_DTYPE_F32 && dt != DS_DTYPE_BF16) return fail(DS_ERR_INVALID_ARGUMENT, "dt: unknown dtype %d", int(dt));
  return DS_OK;
}

// Shape checks shared by the decode entry points.
ds_status check_decode_shape(int B, int Hq, int Hkv, int d, int64_t T_cap, int64_t T, int block, int64_t k_units) {
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(DS_ERR_INVALID_ARGUMENT, "B, Hq, Hkv must be >= 1 (got %d, %d, %d)", B, Hq, Hkv);
  if (Hq % Hkv != 0) return fail(DS_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != ds::kHeadDim) return fail(DS_ERR_UNSUPPORTED, "d = %d unsupported (only %d)", d, ds::kHeadDim);
  if (T < 1 || T > T_cap)
    return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= T <= T_cap (T = %lld, T_cap = %lld)", (long long)T,
                (long long)T_cap);
  if (T > INT32_MAX) return fail(DS_ERR_UNSUPPORTED, "T = %lld exceeds int32 token ids", (long long)T);
  if (!valid_block(block)) return fail(DS_ERR_INVALID_ARGUMENT, "block = %d must be a power of two in [1, 64]", block);
  const int64_t n_units = (T + block - 1) / block;
  if (k_units < 1 || k_units > n_units)
    return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= k_units <= ceil(T/block) = %lld (got %lld)",
                (long long)n_units, (long long)k_units);
  if (int64_t(B) * Hkv > 65535)
    return fail(DS_ERR_UNSUPPORTED, "B * Hkv = %lld exceeds 65535 rows", (long long)(int64_t(B) * Hkv));
  return DS_OK;
}

// Device scratch of ds_decode_sparse_attn_noalloc, for callers that cannot
// allocate: one copy per GPU, held until the process ends.  Host code never
// uses the array's name as an address: each device's copy is found once with
// hipGetSymbolAddress (with that device current) and that pointer is used.
// Every call on a GPU shares its copy, so calls that overlap on one GPU race.
constexpr size_t kScratchBytes = size_t(DS_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
char* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

ds_status scratch_for_current_device(char*& ptr) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
    return fail(DS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DS_ERR_UNSUPPORTED, "device %d: the static scratch supports devices 0..%d", dev, kMaxDevices - 1);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<char*>(p) : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return fail(DS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  ptr = g_scratch_ptr[dev];
  return DS_OK;
}

ds_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DS_OK;
}

}  // namespace

namespace ds {

void set_error(const char* msg) { g_err = msg; }

SplitPlan plan_split(int64_t rows, int G, int64_t kv_virtual, bool fused, bool wide = false) {
  SplitPlan sp{};
  // Fused workgroups are 1024 threads, one resident per CU, and aim at ~256 of
  // them (each repeats the row's selection, so fewer is cheaper, and a second
  // round of workgroups would pay it twice); separate attention workgroups are
  // 256 threads and aim at ~2048.  Every head chunk of a row is a workgroup of
  // its own.  Slices hold at least 64 kept positions, and a row is cut into
  // at most 1024 splits.  Fused workgroups take up to four heads, or up to
  // eight when `wide` (the long rows of the two-stage selection, whose kept
  // K/V rows the eight-head form reads once per group instead of twice).
  const int head_chunk = fused ? (wide ? head_chunk8(G) : head_chunk4(G)) : head_chunk8(G);
  const int64_t head_chunks = G / head_chunk;
  const int64_t target = fused ? 256 : 2048;
  int64_t chunk = (kv_virtual * rows * head_chunks + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  const int64_t min_for_cap = ((kv_virtual + 1023) / 1024 + 63) / 64 * 64;
  if (chunk < min_for_cap) chunk = min_for_cap;
  if (fused && chunk > kFusedMaxChunk) chunk = kFusedMaxChunk;
  sp.chunk = chunk;
  sp.n_split = int((kv_virtual + chunk - 1) / chunk);
  sp.head_chunk = head_chunk;
  sp.head_chunks = int(head_chunks);
  return sp;
}

DecodePlan plan_decode(int B, int Hq, int Hkv, int64_t T, int block, int64_t k_units) {
  DecodePlan p{};
  const int G = Hq / Hkv;
  p.rows = int64_t(B) * Hkv;
  p.n_units = (T + block - 1) / block;
  p.score_ld = (p.n_units + 63) / 64 * 64;
  p.kv_virtual = k_units * block;
  p.fused = p.n_units <= kFusedMaxUnits;
  // Longer rows: the top k of each partition, then the fused kernel over the
  // candidates, when those fit it.
  const int64_t parts = (p.n_units + kPartUnits - 1) / kPartUnits;
  p.partitioned = !p.fused && parts * k_units <= kFusedMaxUnits;
  p.n_cand = p.partitioned ? parts * k_units : 0;
  p.cand_ld = (p.n_cand + 63) / 64 * 64;
  p.sp = plan_split(p.rows, G, p.kv_virtual, p.fused || p.partitioned, p.partitioned);
  p.tiles = (T + kScoreTile - 1) / kScoreTile;
  // The fused kernel then reads the row's top-digit histogram instead of building it
  // (worth it for token-level rows; a tile of 64-token blocks holds only 32 units),
  // when several of its workgroups would each build it: a row that one workgroup
  // handles alone builds it once, for less than the histograms cost to write and
  // read back (batched_32k: 208.9 -> 201.4 us per step).
  // Token-level rows of the two-stage selection score their partitions from
  // the label cache inside the first stage (no score buffer, no tile
  // histograms; each partition builds its own histogram) and pass their
  // candidates' histograms on (at most kMaxHistTiles partitions).
  p.part_onepass = p.partitioned && block == 1;
  p.tile_hist = p.fused && p.tiles <= kMaxHistTiles && block <= 4 && p.sp.n_split * p.sp.head_chunks > 1;
  p.cand_hist = p.partitioned && block == 1 && parts <= kMaxHistTiles;
  // Token-level rows over several fused workgroups take the sorted tile lists
  // and the bucket kernel: a split then reads the tiles' prefixes, its share of
  // the kept ids and the boundary digit's candidates instead of the row.
  p.bucketed = p.fused && block == 1 && p.tile_hist;
  p.sp_idx = plan_split(p.rows, G, p.kv_virtual, false);
  const int max_split = p.sp.n_split > p.sp_idx.n_split ? p.sp.n_split : p.sp_idx.n_split;
  const int64_t bhs = int64_t(B) * Hq * max_split;
  size_t off = 0;
  p.off_scores = off;
  if (!p.part_onepass) off += round256(size_t(p.rows) * size_t(p.score_ld) * sizeof(float));
  p.off_tile_hist = off;
  if (p.tile_hist) off += round256(size_t(p.rows) * size_t(p.tiles) * kHistBins * sizeof(uint16_t));
  p.off_acc = off;
  off += round256(size_t(bhs) * kHeadDim * sizeof(float));
  p.off_ml = off;
  off += round256(size_t(bhs) * 2 * sizeof(float));
  p.off_tickets = off;
  off += round256(size_t(p.rows) * p.sp.head_chunks * sizeof(unsigned));
  p.off_cand_score = off;
  off += round256(size_t(p.rows) * size_t(p.cand_ld) * sizeof(float));
  p.off_cand_id = off;
  off += round256(size_t(p.rows) * size_t(p.n_cand) * sizeof(int32_t));
  p.off_cand_hist = off;
  if (p.cand_hist) off += round256(size_t(p.rows) * size_t(parts) * kHistBins * sizeof(uint16_t));
  p.total_bytes = off;
  return p;
}

}  // namespace ds

namespace {

// Attention over known kept units, then the merge when a row has several splits.
ds_status run_attention(const void* q, const void* K, const void* V, ds_dtype dt, int B, int Hq, int Hkv,
                        int64_t T_cap, int64_t T, int block, int64_t k_units, const int32_t* indices, float scale,
                        const ds::DecodePlan& pl, const ds::SplitPlan& sp, float* out, char* ws, hipStream_t s) {
  float* part_acc = reinterpret_cast<float*>(ws + pl.off_acc);
  float* part_ml = reinterpret_cast<float*>(ws + pl.off_ml);
  if (ds_status st = hip_status(ds::launch_attention(q, K, V, dt == DS_DTYPE_BF16, B, Hq, Hkv, T_cap, T, block,
                                                     k_units, indices, scale, pl.kv_virtual, sp, part_acc, part_ml,
                                                     out, s),
                                "attention launch"))
    return st;
  if (sp.n_split == 1) return DS_OK;
  return hip_status(ds::launch_merge(part_acc, part_ml, int64_t(B) * Hq, sp.n_split, out, s), "merge launch");
}

// Steps 2 and 3 of the decode step from a score buffer laid out as the plan says.
// tickets_zeroed: the score kernel of this call already cleared the merge tickets.
ds_status run_select_attend(const void* q, const void* K, const void* V, ds_dtype dt, int B, int Hq, int Hkv,
                            int64_t T_cap, int64_t T, int block, int64_t k_units, const float* scores, int64_t ld,
                            const uint16_t* tile_hist, bool tickets_zeroed, float scale, const ds::DecodePlan& pl,
                            float* out, int32_t* indices, char* ws, hipStream_t s,
                            const int32_t* seq_lens = nullptr, float tau = 0.f, int32_t* counts = nullptr,
                            bool cand_ready = false) {
  if (pl.fused || pl.partitioned) {
    float* part_acc = reinterpret_cast<float*>(ws + pl.off_acc);
    float* part_ml = reinterpret_cast<float*>(ws + pl.off_ml);
    unsigned* tickets = reinterpret_cast<unsigned*>(ws + pl.off_tickets);
    if (!tickets_zeroed && pl.sp.n_split > 1)
      if (ds_status st = hip_status(ds::launch_zero_u32(tickets, pl.rows * pl.sp.head_chunks, s), "ticket reset"))
        return st;
    if (pl.partitioned) {
      // Top k of each partition, then the fused kernel over the candidates.
      float* cand_score = reinterpret_cast<float*>(ws + pl.off_cand_score);
      int32_t* cand_id = reinterpret_cast<int32_t*>(ws + pl.off_cand_id);
      // cand_ready: the score phase's one-pass first stage already wrote the candidates.
      uint16_t* cand_hist = (tile_hist != nullptr || cand_ready) && pl.cand_hist
                                ? reinterpret_cast<uint16_t*>(ws + pl.off_cand_hist)
                                : nullptr;
      if (!cand_ready)
        if (ds_status st = hip_status(ds::launch_partition_topk(scores, pl.rows, pl.n_units, ld, k_units, cand_score,
                                                                pl.cand_ld, cand_id, tile_hist, pl.tiles, cand_hist, s),
                                      "partition select launch"))
          return st;
      ds::DecodePlan pc = pl;
      pc.n_units = pl.n_cand;
      pc.tile_hist = cand_hist != nullptr;
      pc.tiles = pl.n_cand / k_units;
      return hip_status(ds::launch_select_attention(q, K, V, dt == DS_DTYPE_BF16, cand_score, pl.cand_ld, cand_hist, Hq,
                                                    Hkv, T_cap, T, block, k_units, scale, pc, indices, part_acc,
                                                    part_ml, out, tickets, nullptr, 0.f, nullptr, cand_id, s),
                        "select-attention launch");
    }
    return hip_status(ds::launch_select_attention(q, K, V, dt == DS_DTYPE_BF16, scores, ld, tile_hist, Hq, Hkv, T_cap,
                                                  T, block, k_units, scale, pl, indices, part_acc, part_ml, out,
                                                  tickets, seq_lens, tau, counts, nullptr, s),
                      "select-attention launch");
  }
  if (ds_status st = hip_status(ds::launch_select(scores, pl.rows, pl.n_units, ld, k_units, indices, s),
                                "select launch"))
    return st;
  return run_attention(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, indices, scale, pl, pl.sp, out, ws, s);
}

}  // namespace

extern "C" {

const char* ds_last_error(void) { return g_err.c_str(); }

const char* ds_version(void) { return "dsparse 0.2.0 gfx950"; }

ds_status ds_build_label_cache(const void* K, ds_dtype dt, int32_t B, int32_t Hkv, int64_t T_cap, int32_t d,
                               const int32_t* channels_dev, int32_t r, int64_t t_begin, int64_t t_end,
                               void* label_out, void* stream) {
  g_err.clear();
  if (!K || !channels_dev || !label_out) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (B < 1 || Hkv < 1 || T_cap < 1) return fail(DS_ERR_INVALID_ARGUMENT, "B, Hkv, T_cap must be >= 1");
  if (T_cap > INT32_MAX) return fail(DS_ERR_UNSUPPORTED, "T_cap = %lld exceeds int32 token ids", (long long)T_cap);
  if (int64_t(B) * Hkv > 65535)
    return fail(DS_ERR_UNSUPPORTED, "B * Hkv = %lld exceeds 65535 rows", (long long)(int64_t(B) * Hkv));
  if (d != ds::kHeadDim) return fail(DS_ERR_UNSUPPORTED, "d = %d unsupported (only %d)", d, ds::kHeadDim);
  if (r < 1 || r > d) return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= r <= d (r = %d)", r);
  if (t_begin < 0 || t_begin > t_end || t_end > T_cap)
    return fail(DS_ERR_INVALID_ARGUMENT, "need 0 <= t_begin <= t_end <= T_cap (%lld, %lld, %lld)",
                (long long)t_begin, (long long)t_end, (long long)T_cap);
  if (!aligned(K, 16) || !aligned(label_out, 16) || !aligned(channels_dev, 4))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  return hip_status(ds::launch_pack(K, dt == DS_DTYPE_BF16, B, Hkv, T_cap, channels_dev, r, t_begin, t_end,
                                    label_out, static_cast<hipStream_t>(stream)),
                    "label pack launch");
}

size_t ds_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t block,
                                 int64_t k_units) {
  g_err.clear();
  if (check_decode_shape(B, Hq, Hkv, d, T, T, block, k_units) != DS_OK) return 0;
  return ds::plan_decode(B, Hq, Hkv, T, block, k_units).total_bytes;
}

ds_status ds_label_scores(const void* q, const void* label, const int32_t* channels_dev, int32_t r, ds_dtype dt,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block,
                          float* scores, int64_t ld, void* stream) {
  g_err.clear();
  if (!q || !label || !channels_dev || !scores) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, 1)) return st;
  if (r < 1 || r > d) return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= r <= d (r = %d)", r);
  const int64_t n_units = (T + block - 1) / block;
  if (ld < n_units || ld % 4 != 0)
    return fail(DS_ERR_INVALID_ARGUMENT, "ld = %lld must be >= %lld and a multiple of 4", (long long)ld,
                (long long)n_units);
  if (!aligned(q, 16) || !aligned(label, 16) || !aligned(scores, 16) || !aligned(channels_dev, 4))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  // No append: the label cache is only read.
  return hip_status(ds::launch_scores(q, const_cast<void*>(label), nullptr, channels_dev, r, dt == DS_DTYPE_BF16, B,
                                      Hq, Hkv, T_cap, T, T, block, scores, ld, nullptr, nullptr, 0, nullptr, 0,
                                      false, static_cast<hipStream_t>(stream)),
                    "score launch");
}

// Positive-only head aggregation (one double per (head, label channel) in the
// score kernel's LDS table, filled by one thread each).
static ds_status check_positive(int32_t Hq, int32_t Hkv, int32_t r) {
  const int G = Hq / Hkv;
  if (G > 8) return fail(DS_ERR_UNSUPPORTED, "positive-only aggregation needs Hq / Hkv <= 8 (got %d)", G);
  if (G * r > 512) return fail(DS_ERR_UNSUPPORTED, "positive-only aggregation needs (Hq / Hkv) * r <= 512 (got %d)",
                               G * r);
  return DS_OK;
}

ds_status ds_label_scores_positive(const void* q, const void* label, const int32_t* channels_dev, int32_t r,
                                   ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                   int64_t T, int32_t block, float* scores, int64_t ld, void* stream) {
  g_err.clear();
  if (!q || !label || !channels_dev || !scores) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, 1)) return st;
  if (r < 1 || r > d) return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= r <= d (r = %d)", r);
  if (ds_status st = check_positive(Hq, Hkv, r)) return st;
  const int64_t n_units = (T + block - 1) / block;
  if (ld < n_units || ld % 4 != 0)
    return fail(DS_ERR_INVALID_ARGUMENT, "ld = %lld must be >= %lld and a multiple of 4", (long long)ld,
                (long long)n_units);
  if (!aligned(q, 16) || !aligned(label, 16) || !aligned(scores, 16) || !aligned(channels_dev, 4))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  return hip_status(ds::launch_scores(q, const_cast<void*>(label), nullptr, channels_dev, r, dt == DS_DTYPE_BF16, B,
                                      Hq, Hkv, T_cap, T, T, block, scores, ld, nullptr, nullptr, 0, nullptr, 0,
                                      true, static_cast<hipStream_t>(stream)),
                    "score launch");
}

ds_status ds_topk_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx_out,
                         void* stream) {
  g_err.clear();
  if (!scores || !idx_out) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (rows < 1 || rows > INT32_MAX) return fail(DS_ERR_INVALID_ARGUMENT, "rows = %lld out of range", (long long)rows);
  if (n < 1 || n > INT32_MAX) return fail(DS_ERR_INVALID_ARGUMENT, "n = %lld out of range", (long long)n);
  if (k < 1 || k > n) return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= k <= n (k = %lld)", (long long)k);
  if (ld < n) return fail(DS_ERR_INVALID_ARGUMENT, "ld = %lld < n = %lld", (long long)ld, (long long)n);
  if (!aligned(scores, 4) || !aligned(idx_out, 4)) return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  return hip_status(ds::launch_select(scores, rows, n, ld, k, idx_out, static_cast<hipStream_t>(stream)),
                    "select launch");
}

ds_status ds_sparse_attn_from_indices(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                                      int32_t block, int64_t k_units, const int32_t* indices, float scale,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !K || !V || !indices || !out || !workspace) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, k_units)) return st;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16) || !aligned(indices, 4) ||
      !aligned(workspace, 256))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  const ds::DecodePlan pl = ds::plan_decode(B, Hq, Hkv, T, block, k_units);
  if (workspace_bytes < pl.total_bytes)
    return fail(DS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total_bytes);
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  return run_attention(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, indices, scale, pl, pl.sp_idx, out,
                       static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

// Shared validation of the decode calls; fills the plan on success.
static ds_status check_decode_call(const void* q, const void* K, const void* V, const void* label,
                                   const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append, int32_t block,
                                   int64_t k_units, const void* out, const int32_t* indices, const void* workspace,
                                   size_t workspace_bytes, bool need_label, bool need_out, ds::DecodePlan& pl) {
  if (!q || !K || !workspace || (need_label && (!label || !channels_dev)) || (need_out && (!V || !out || !indices)))
    return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, k_units)) return st;
  if (need_label && (r < 1 || r > d)) return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= r <= d (r = %d)", r);
  if (need_label && (t_append < 0 || t_append > T))
    return fail(DS_ERR_INVALID_ARGUMENT, "need 0 <= t_append <= T (t_append = %lld)", (long long)t_append);
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(workspace, 256) ||
      (need_label && (!aligned(label, 16) || !aligned(channels_dev, 4))) ||
      (need_out && (!aligned(V, 16) || !aligned(out, 16) || !aligned(indices, 4))))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  pl = ds::plan_decode(B, Hq, Hkv, T, block, k_units);
  if (workspace_bytes < pl.total_bytes)
    return fail(DS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total_bytes);
  return DS_OK;
}

static ds_status decode_score_stage(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                                    ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int64_t T_cap, int64_t T,
                                    int64_t t_append, int32_t block, const ds::DecodePlan& pl, char* ws,
                                    hipStream_t s, const int32_t* seq_lens = nullptr, int32_t n_append = 0,
                                    bool positive = false) {
  float* scores = reinterpret_cast<float*>(ws + pl.off_scores);
  uint16_t* tile_hist = pl.tile_hist ? reinterpret_cast<uint16_t*>(ws + pl.off_tile_hist) : nullptr;
  unsigned* tickets = pl.fused || pl.partitioned ? reinterpret_cast<unsigned*>(ws + pl.off_tickets) : nullptr;
  if (pl.part_onepass && seq_lens == nullptr && !positive)
    return hip_status(ds::launch_partition_onepass(
                          q, label, K, channels_dev, r, dt == DS_DTYPE_BF16, B, Hq, Hkv, T_cap, T, t_append,
                          pl.n_cand / ((pl.n_units + ds::kPartUnits - 1) / ds::kPartUnits),
                          reinterpret_cast<float*>(ws + pl.off_cand_score), pl.cand_ld,
                          reinterpret_cast<int32_t*>(ws + pl.off_cand_id),
                          pl.cand_hist ? reinterpret_cast<uint16_t*>(ws + pl.off_cand_hist) : nullptr, tickets,
                          pl.sp.head_chunks, s),
                      "one-pass partition launch");
  // The plain top-k step of bucketed shapes writes sorted tile lists; ragged and
  // threshold calls keep the unit-order scores and histograms.
  const bool sorted = pl.bucketed && seq_lens == nullptr && !positive;
  return hip_status(ds::launch_scores(q, label, K, channels_dev, r, dt == DS_DTYPE_BF16, B, Hq, Hkv, T_cap, T,
                                      t_append, block, scores, pl.score_ld, tile_hist, tickets, pl.sp.head_chunks,
                                      seq_lens, n_append, positive, s, sorted),
                    "score launch");
}

static ds_status decode_select_stage(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                                     int32_t Hkv, int64_t T_cap, int64_t T, int32_t block, int64_t k_units,
                                     float scale, const ds::DecodePlan& pl, float* out, int32_t* indices, char* ws,
                                     hipStream_t s, const int32_t* seq_lens = nullptr, float tau = 0.f,
                                     int32_t* counts = nullptr) {
  const float* scores = reinterpret_cast<const float*>(ws + pl.off_scores);
  const uint16_t* tile_hist = pl.tile_hist ? reinterpret_cast<const uint16_t*>(ws + pl.off_tile_hist) : nullptr;
  if (pl.bucketed && seq_lens == nullptr && counts == nullptr)
    return hip_status(
        ds::launch_bucket_attention(q, K, V, dt == DS_DTYPE_BF16, reinterpret_cast<const uint32_t*>(scores), tile_hist, Hq, Hkv, T_cap, k_units, scale, pl, indices,
                                    reinterpret_cast<float*>(ws + pl.off_acc), reinterpret_cast<float*>(ws + pl.off_ml),
                                    out, reinterpret_cast<unsigned*>(ws + pl.off_tickets), s),
        "bucket select-attention launch");
  return run_select_attend(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, scores, pl.score_ld, tile_hist, true,
                           scale, pl, out, indices, ws, s, seq_lens, tau, counts,
                           pl.part_onepass && seq_lens == nullptr && counts == nullptr);
}

// The one-pass form of the decode step, one kernel instead of two: token-level
// rows that one fused workgroup handles alone (one split, one head chunk),
// with label rows of 16 or 32 bytes (or 64 in fp32).  The kernel scores each row from the label
// cache itself, so the scores never go through memory.
static bool one_pass_ok(const ds::DecodePlan& pl, int32_t block, int32_t r, ds_dtype dt) {
  const int row_bytes = r * (dt == DS_DTYPE_BF16 ? 2 : 4);
  return pl.fused && block == 1 && pl.sp.n_split == 1 && pl.sp.head_chunks == 1 && !pl.tile_hist &&
         (row_bytes == 16 || row_bytes == 32 || (row_bytes == 64 && dt == DS_DTYPE_F32));
}

static ds_status decode_one_pass(const void* q, const void* K, const void* V, void* label,
                                 const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t Hq, int32_t Hkv,
                                 int64_t T_cap, int64_t T, int64_t t_append, int64_t k_units, float scale,
                                 const ds::DecodePlan& pl, float* out, int32_t* indices, char* ws, hipStream_t s,
                                 const int32_t* seq_lens = nullptr, int32_t n_append = 0) {
  const ds::OnePass one{label, channels_dev, r, t_append, n_append};
  return hip_status(
      ds::launch_select_attention(q, K, V, dt == DS_DTYPE_BF16, nullptr, pl.score_ld, nullptr, Hq, Hkv, T_cap, T, 1,
                                  k_units, scale, pl, indices, reinterpret_cast<float*>(ws + pl.off_acc),
                                  reinterpret_cast<float*>(ws + pl.off_ml), out,
                                  reinterpret_cast<unsigned*>(ws + pl.off_tickets), seq_lens, 0.f, nullptr, nullptr, s,
                                  &one),
      "one-pass decode launch");
}

int32_t ds_decode_is_one_pass(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t block,
                              int64_t k_units, int32_t r, ds_dtype dt) {
  g_err.clear();
  if (check_dtype(dt) != DS_OK || check_decode_shape(B, Hq, Hkv, d, T, T, block, k_units) != DS_OK) return -1;
  if (r < 1 || r > d) {
    fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= r <= d (r = %d)", r);
    return -1;
  }
  return one_pass_ok(ds::plan_decode(B, Hq, Hkv, T, block, k_units), block, r, dt) ? 1 : 0;
}

// The decode step's launches, once the call has been validated and planned.
static ds_status decode_step(const void* q, const void* K, const void* V, void* label, const int32_t* channels_dev,
                             int32_t r, ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                             int64_t T, int64_t t_append, int32_t block, int64_t k_units, float scale, float* out,
                             int32_t* indices, char* ws, const ds::DecodePlan& pl, hipStream_t s) {
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  if (one_pass_ok(pl, block, r, dt))
    return decode_one_pass(q, K, V, label, channels_dev, r, dt, Hq, Hkv, T_cap, T, t_append, k_units, scale, pl,
                           out, indices, ws, s);
  if (ds_status st = decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T, t_append, block, pl,
                                        ws, s))
    return st;
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, scale, pl, out, indices, ws, s);
}

ds_status ds_decode_sparse_attn(const void* q, const void* K, const void* V, void* label, const int32_t* channels_dev,
                                int32_t r, ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                int64_t T, int64_t t_append, int32_t block, int64_t k_units, float scale, float* out,
                                int32_t* indices, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block,
                                       k_units, out, indices, workspace, workspace_bytes, true, true, pl))
    return st;
  return decode_step(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block, k_units, scale,
                     out, indices, static_cast<char*>(workspace), pl, static_cast<hipStream_t>(stream));
}

ds_status ds_decode_sparse_attn_noalloc(const void* q, const void* K, const void* V, void* label,
                                        const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                        int32_t block, int64_t k_units, float scale, float* out, int32_t* indices,
                                        void* stream) {
  g_err.clear();
  // The shape's workspace must fit the scratch.  The placeholder workspace
  // pointer passed to the shared checks is only tested for null and alignment.
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, k_units)) return st;
  const size_t need = ds::plan_decode(B, Hq, Hkv, T, block, k_units).total_bytes;
  if (need > kScratchBytes)
    return fail(DS_ERR_WORKSPACE_TOO_SMALL,
                "this shape needs %zu bytes of workspace, more than the %zu-byte static device scratch of the "
                "no-allocation entry point; call ds_decode_sparse_attn with a workspace instead",
                need, kScratchBytes);
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block,
                                       k_units, out, indices, reinterpret_cast<void*>(uintptr_t(256)), kScratchBytes,
                                       true, true, pl))
    return st;
  char* ws = nullptr;
  if (ds_status st = scratch_for_current_device(ws)) return st;
  return decode_step(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block, k_units, scale,
                     out, indices, ws, pl, static_cast<hipStream_t>(stream));
}

// Validation shared by the ragged-length calls, after check_decode_call.
static ds_status check_ragged(const int32_t* seq_lens_dev, int32_t n_append, const ds::DecodePlan& pl) {
  if (!seq_lens_dev) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument (seq_lens)");
  if (!aligned(seq_lens_dev, 4)) return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer (seq_lens)");
  if (n_append < 0) return fail(DS_ERR_INVALID_ARGUMENT, "n_append = %d must be >= 0", int(n_append));
  if (!pl.fused)
    return fail(DS_ERR_UNSUPPORTED, "ragged lengths need ceil(T_max / block) <= %lld units per row (got %lld)",
                (long long)ds::kFusedMaxUnits, (long long)pl.n_units);
  return DS_OK;
}

ds_status ds_decode_sparse_attn_ragged(const void* q, const void* K, const void* V, void* label,
                                       const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                       int32_t Hkv, int32_t d, int64_t T_cap, int64_t T_max,
                                       const int32_t* seq_lens_dev, int32_t n_append, int32_t block, int64_t k_units,
                                       float scale, float* out, int32_t* indices, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T_max, T_max, block,
                                       k_units, out, indices, workspace, workspace_bytes, true, true, pl))
    return st;
  if (ds_status st = check_ragged(seq_lens_dev, n_append, pl)) return st;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (one_pass_ok(pl, block, r, dt))
    return decode_one_pass(q, K, V, label, channels_dev, r, dt, Hq, Hkv, T_cap, T_max, T_max, k_units, scale, pl,
                           out, indices, ws, s, seq_lens_dev, n_append);
  if (ds_status st = decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T_max, T_max, block, pl,
                                        ws, s, seq_lens_dev, n_append))
    return st;
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T_max, block, k_units, scale, pl, out, indices, ws, s,
                             seq_lens_dev);
}

ds_status ds_decode_score_ragged(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                                 ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                 int64_t T_max, const int32_t* seq_lens_dev, int32_t n_append, int32_t block,
                                 int64_t k_units, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, nullptr, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T_max, T_max,
                                       block, k_units, nullptr, nullptr, workspace, workspace_bytes, true, false, pl))
    return st;
  if (ds_status st = check_ragged(seq_lens_dev, n_append, pl)) return st;
  return decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T_max, T_max, block, pl,
                            static_cast<char*>(workspace), static_cast<hipStream_t>(stream), seq_lens_dev, n_append);
}

ds_status ds_decode_select_attend_ragged(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T_max,
                                         const int32_t* seq_lens_dev, int32_t block, int64_t k_units, float scale,
                                         float* out, int32_t* indices, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, nullptr, nullptr, 0, dt, B, Hq, Hkv, d, T_cap, T_max, T_max, block,
                                       k_units, out, indices, workspace, workspace_bytes, false, true, pl))
    return st;
  if (ds_status st = check_ragged(seq_lens_dev, 0, pl)) return st;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T_max, block, k_units, scale, pl, out, indices,
                             static_cast<char*>(workspace), static_cast<hipStream_t>(stream), seq_lens_dev);
}

// The device address of pinned host memory (allocated with hipHostMalloc or
// registered by the runtime); fails for any other pointer.
static ds_status host_pinned(const void* p, const char* name, const void*& dev) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the failed query
    return fail(DS_ERR_INVALID_ARGUMENT, "%s is not memory known to HIP (%s)", name, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeHost) return fail(DS_ERR_INVALID_ARGUMENT, "%s must be pinned host memory", name);
  dev = at.devicePointer ? at.devicePointer : p;
  return DS_OK;
}

ds_status ds_decode_sparse_attn_offload(const void* q, const void* K_host, const void* V_host, void* label,
                                        const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                        int32_t block, int64_t k_units, float scale, float* out, int32_t* indices,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K_host, V_host, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T,
                                       t_append, block, k_units, out, indices, workspace, workspace_bytes, true, true,
                                       pl))
    return st;
  const void* Kd = nullptr;
  const void* Vd = nullptr;
  if (ds_status st = host_pinned(K_host, "K", Kd)) return st;
  if (ds_status st = host_pinned(V_host, "V", Vd)) return st;
  if (!aligned(Kd, 16) || !aligned(Vd, 16)) return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device address of K or V");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (one_pass_ok(pl, block, r, dt))
    return decode_one_pass(q, Kd, Vd, label, channels_dev, r, dt, Hq, Hkv, T_cap, T, t_append, k_units, scale,
                           pl, out, indices, ws, s);
  if (ds_status st = decode_score_stage(q, Kd, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T, t_append, block, pl,
                                        ws, s))
    return st;
  return decode_select_stage(q, Kd, Vd, dt, B, Hq, Hkv, T_cap, T, block, k_units, scale, pl, out, indices, ws, s);
}

ds_status ds_decode_score(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                          ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                          int64_t t_append, int32_t block, int64_t k_units, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, nullptr, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append,
                                       block, k_units, nullptr, nullptr, workspace, workspace_bytes, true, false, pl))
    return st;
  return decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T, t_append, block, pl,
                            static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

ds_status ds_decode_select_attend(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block, int64_t k_units,
                                  float scale, float* out, int32_t* indices, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, nullptr, nullptr, 0, dt, B, Hq, Hkv, d, T_cap, T, T, block, k_units,
                                       out, indices, workspace, workspace_bytes, false, true, pl))
    return st;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, scale, pl, out, indices,
                             static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

// Validation shared by the threshold-rule calls, after check_decode_call.
static ds_status check_threshold(float tau, const int32_t* counts, bool need_counts, const ds::DecodePlan& pl) {
  if (std::isnan(tau)) return fail(DS_ERR_INVALID_ARGUMENT, "tau is NaN");
  if (need_counts && !counts) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument (counts)");
  if (need_counts && !aligned(counts, 4)) return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer (counts)");
  if (!pl.fused)
    return fail(DS_ERR_UNSUPPORTED, "the threshold rule needs ceil(T / block) <= %lld units per row (got %lld)",
                (long long)ds::kFusedMaxUnits, (long long)pl.n_units);
  return DS_OK;
}

ds_status ds_decode_sparse_attn_threshold(const void* q, const void* K, const void* V, void* label,
                                          const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                          int32_t block, int64_t k_max, float tau, float scale, float* out,
                                          int32_t* indices, int32_t* counts, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append, block,
                                       k_max, out, indices, workspace, workspace_bytes, true, true, pl))
    return st;
  if (ds_status st = check_positive(Hq, Hkv, r)) return st;
  if (ds_status st = check_threshold(tau, counts, true, pl)) return st;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (ds_status st = decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T, t_append, block, pl,
                                        ws, s, nullptr, 0, true))
    return st;
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_max, scale, pl, out, indices, ws, s, nullptr,
                             tau, counts);
}

ds_status ds_decode_score_threshold(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                                    ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                    int64_t T, int64_t t_append, int32_t block, int64_t k_max, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, nullptr, label, channels_dev, r, dt, B, Hq, Hkv, d, T_cap, T, t_append,
                                       block, k_max, nullptr, nullptr, workspace, workspace_bytes, true, false, pl))
    return st;
  if (ds_status st = check_positive(Hq, Hkv, r)) return st;
  if (ds_status st = check_threshold(0.f, nullptr, false, pl)) return st;
  return decode_score_stage(q, K, label, channels_dev, r, dt, B, Hq, Hkv, T_cap, T, t_append, block, pl,
                            static_cast<char*>(workspace), static_cast<hipStream_t>(stream), nullptr, 0, true);
}

ds_status ds_decode_select_attend_threshold(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                            int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                                            int32_t block, int64_t k_max, float tau, float scale, float* out,
                                            int32_t* indices, int32_t* counts, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  g_err.clear();
  ds::DecodePlan pl;
  if (ds_status st = check_decode_call(q, K, V, nullptr, nullptr, 0, dt, B, Hq, Hkv, d, T_cap, T, T, block, k_max,
                                       out, indices, workspace, workspace_bytes, false, true, pl))
    return st;
  if (ds_status st = check_threshold(tau, counts, true, pl)) return st;
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  return decode_select_stage(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_max, scale, pl, out, indices,
                             static_cast<char*>(workspace), static_cast<hipStream_t>(stream), nullptr, tau, counts);
}

// Hierarchical span search: rounds until no span is longer than `span`, and
// the token capacity of a row (k * span, or T when no round runs, in which
// case the first spans cover every token).
static int hip_rounds(int64_t T, int64_t k, int64_t span) {
  int64_t len = (T + k - 1) / k;
  int rounds = 0;
  while (len > span) {
    len = (len + 1) / 2;
    ++rounds;
  }
  return rounds;
}

static int64_t hip_capacity(int64_t T, int64_t k, int64_t span) {
  return hip_rounds(T, k, span) > 0 ? k * span : T;
}

static ds_status check_hip_shape(int B, int Hq, int Hkv, int d, int64_t T_cap, int64_t T, int64_t k, int64_t span) {
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, 1, 1)) return st;
  if (k < 1 || k > T || k > 1024)
    return fail(DS_ERR_INVALID_ARGUMENT, "need 1 <= k_spans <= min(T, 1024) (got %lld)", (long long)k);
  if (span < 1 || span > INT32_MAX) return fail(DS_ERR_INVALID_ARGUMENT, "span = %lld must be >= 1", (long long)span);
  return DS_OK;
}

// Workspace of ds_decode_hip_attn: the token list, then the attention splits.
static ds::DecodePlan plan_hip(int B, int Hq, int Hkv, int64_t T, int64_t k, int64_t span) {
  ds::DecodePlan p{};
  const int G = Hq / Hkv;
  p.rows = int64_t(B) * Hkv;
  p.n_units = T;
  p.kv_virtual = hip_capacity(T, k, span);
  p.sp = ds::plan_split(p.rows, G, p.kv_virtual, false);
  p.sp_idx = p.sp;
  size_t off = 0;
  p.off_scores = off;   // token list [rows][capacity] int32
  off += round256(size_t(p.rows) * size_t(p.kv_virtual) * sizeof(int32_t));
  const int64_t bhs = int64_t(B) * Hq * p.sp.n_split;
  p.off_acc = off;
  off += round256(size_t(bhs) * ds::kHeadDim * sizeof(float));
  p.off_ml = off;
  off += round256(size_t(bhs) * 2 * sizeof(float));
  p.total_bytes = off;
  return p;
}

int64_t ds_hip_token_capacity(int64_t T, int64_t k_spans, int64_t span) {
  g_err.clear();
  if (T < 1 || k_spans < 1 || k_spans > T || span < 1) {
    fail(DS_ERR_INVALID_ARGUMENT, "need T >= 1, 1 <= k_spans <= T, span >= 1");
    return 0;
  }
  return hip_capacity(T, k_spans, span);
}

size_t ds_hip_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t k_spans,
                              int32_t span) {
  g_err.clear();
  if (check_hip_shape(B, Hq, Hkv, d, T, T, k_spans, span) != DS_OK) return 0;
  return plan_hip(B, Hq, Hkv, T, k_spans, span).total_bytes;
}

ds_status ds_hip_search(const void* q, const void* K, ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                        int64_t T_cap, int64_t T, int32_t k_spans, int32_t span, int32_t* spans, int32_t* tokens,
                        void* stream) {
  g_err.clear();
  if (!q || !K || !spans || !tokens) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_hip_shape(B, Hq, Hkv, d, T_cap, T, k_spans, span)) return st;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(spans, 4) || !aligned(tokens, 4))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  return hip_status(ds::launch_hip_search(q, K, dt == DS_DTYPE_BF16, B, Hq, Hkv, T_cap, T, k_spans, span,
                                          hip_rounds(T, k_spans, span), spans, tokens,
                                          hip_capacity(T, k_spans, span), static_cast<hipStream_t>(stream)),
                    "search launch");
}

ds_status ds_decode_hip_attn(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t k_spans, int32_t span,
                             float scale, float* out, int32_t* spans, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_err.clear();
  if (!q || !K || !V || !out || !spans || !workspace) return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_hip_shape(B, Hq, Hkv, d, T_cap, T, k_spans, span)) return st;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16) || !aligned(spans, 4) ||
      !aligned(workspace, 256))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  const ds::DecodePlan pl = plan_hip(B, Hq, Hkv, T, k_spans, span);
  if (workspace_bytes < pl.total_bytes)
    return fail(DS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total_bytes);
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* tokens = reinterpret_cast<int32_t*>(ws + pl.off_scores);
  if (ds_status st = hip_status(ds::launch_hip_search(q, K, dt == DS_DTYPE_BF16, B, Hq, Hkv, T_cap, T, k_spans, span,
                                                      hip_rounds(T, k_spans, span), spans, tokens, pl.kv_virtual, s),
                                "search launch"))
    return st;
  return run_attention(q, K, V, dt, B, Hq, Hkv, T_cap, T, 1, pl.kv_virtual, tokens, scale, pl, pl.sp, out, ws, s);
}

ds_status ds_select_attention(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block, int64_t k_units,
                              const float* scores, int64_t ld, float scale, float* out, int32_t* indices,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !K || !V || !scores || !out || !indices || !workspace)
    return fail(DS_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (ds_status st = check_dtype(dt)) return st;
  if (ds_status st = check_decode_shape(B, Hq, Hkv, d, T_cap, T, block, k_units)) return st;
  const ds::DecodePlan pl = ds::plan_decode(B, Hq, Hkv, T, block, k_units);
  if (ld < pl.n_units || ld % 4 != 0)
    return fail(DS_ERR_INVALID_ARGUMENT, "ld = %lld must be >= %lld and a multiple of 4", (long long)ld,
                (long long)pl.n_units);
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(scores, 16) || !aligned(out, 16) ||
      !aligned(indices, 4) || !aligned(workspace, 256))
    return fail(DS_ERR_INVALID_ARGUMENT, "misaligned device pointer");
  if (workspace_bytes < pl.total_bytes)
    return fail(DS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total_bytes);
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(float(d));
  // Scores come from the caller here, so the fused kernel builds the top-digit histogram itself.
  return run_select_attend(q, K, V, dt, B, Hq, Hkv, T_cap, T, block, k_units, scores, ld, nullptr, false, scale, pl,
                           out, indices, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"
