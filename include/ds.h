/*
 * ds.h: C ABI of the Double Sparsity sparse-decode library for AMD MI355X (gfx950).
 *
 * One decode step of Double Sparsity ("Post-Training Sparse Attention with
 * Double Sparsity", method details and abstract): a small set of r "label"
 * channels of K, fixed offline by calibration, scores every cached token
 * approximately; the k highest-scoring tokens (or blocks of tokens, the
 * block-max variant of the Jenga page, core method item 1, and the top-k key
 * framing of the HiP page, abstract) are kept; exact softmax attention then
 * runs over the kept tokens' K and V rows only, read in place from the cache.
 *
 * Conventions shared by every entry point
 *   - Plain pointers and sizes only.  "Device" pointers are HIP device memory
 *     on the current device; "host" pointers are ordinary process memory.
 *   - The caller owns every buffer, the workspace included.  The library
 *     allocates no device memory and keeps no pointer after a call returns.
 *     Buffers passed to a GPU entry point must stay valid until the work
 *     queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  GPU
 *     entry points only enqueue work; they never synchronise.  A fault inside
 *     a kernel surfaces at the caller's next synchronisation.
 *   - Every argument is validated before any HIP call.  On failure nothing is
 *     written or enqueued, the status is returned, and ds_last_error() holds a
 *     message.  A failed kernel launch returns DS_ERR_HIP.  No C++ exception
 *     crosses the ABI.
 *   - Re-entrant; calls that run concurrently need distinct output and
 *     workspace buffers.
 *   - Element types: DS_DTYPE_F32 (float) or DS_DTYPE_BF16 (bfloat16 bits in
 *     uint16).  q, K, V and the label cache share one element type.  Scores
 *     and outputs are float32.
 *   - All device buffers must be 16-byte aligned, except int32 index buffers
 *     (4-byte) and the workspace (256-byte).
 *   - Head dimension d must be 128 (DS_ERR_UNSUPPORTED otherwise).  Any label
 *     width 1 <= r <= d works; r * element_size a multiple of 16 bytes takes
 *     the vectorised path.
 */
#ifndef DS_SPARSE_DECODE_H
#define DS_SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DS_OK = 0,
  DS_ERR_INVALID_ARGUMENT = 1,
  DS_ERR_UNSUPPORTED = 2,
  DS_ERR_WORKSPACE_TOO_SMALL = 3,
  DS_ERR_HIP = 4
} ds_status;

/* Element type of q, K, V and the label cache.  A plain 32-bit integer rather
 * than an enum type, so that any value a caller passes is a valid argument
 * (values other than these two are rejected with DS_ERR_INVALID_ARGUMENT). */
typedef int32_t ds_dtype;
enum { DS_DTYPE_F32 = 0, DS_DTYPE_BF16 = 1 };

/* Message of the last failed call on this thread ("" if none).  Valid until the
 * next ds_* call on the same thread. */
const char* ds_last_error(void);

/* Library version string, e.g. "dsparse 0.1.0 gfx950". */
const char* ds_version(void);

/*
 * Offline calibration of the label channels (CPU, synchronous, host memory).
 * Double Sparsity page, method details: the channel-sparsity pattern is close
 * to static, so it is fixed once from a small calibration set.  The page does
 * not give the rule; this library scores channel c of KV head g by
 *     mean over (n, query heads h of group g) of |q_cal[n, h, c]|
 *   * mean over n of |k_cal[g, n, c]|
 * (the mean of |q_c| * |k_c| over all query/key pairs) in double precision,
 * keeps the r highest (the lower channel id wins a tie) and writes them in
 * ascending order.
 *   q_cal        host float [n_q, Hq, d]
 *   k_cal        host float [Hkv, n_k, d]
 *   channels_out host int32 [Hkv, r], written only on success
 * Errors: null pointer, n_q or n_k < 1, Hq % Hkv != 0, r outside [1, d].
 */
ds_status ds_calibrate_channels(const float* q_cal, int64_t n_q, const float* k_cal, int64_t n_k,
                                int32_t Hq, int32_t Hkv, int32_t d, int32_t r, int32_t* channels_out);

/*
 * Label cache: label[b, g, t, j] = K[b, g, t, channels[g, j]] for t in
 * [t_begin, t_end) (GPU, async).  Bit copy, no arithmetic.  Run once over the
 * prefilled tokens, then for the one new row of each decode step (Double
 * Sparsity page, abstract: the important channels are used to identify the
 * important tokens, so only they are kept in a compact per-token row).
 *   K            device [B, Hkv, T_cap, d]
 *   channels_dev device int32 [Hkv, r], each in [0, d) (not checked)
 *   label_out    device [B, Hkv, T_cap, r]; rows outside [t_begin, t_end) are
 *                left untouched
 * Errors: null pointer, bad dtype, B/Hkv/T_cap < 1, r outside [1, d],
 * 0 <= t_begin <= t_end <= T_cap violated, misalignment, unsupported d.
 */
ds_status ds_build_label_cache(const void* K, ds_dtype dt, int32_t B, int32_t Hkv, int64_t T_cap, int32_t d,
                               const int32_t* channels_dev, int32_t r, int64_t t_begin, int64_t t_end,
                               void* label_out, void* stream);

/*
 * Workspace bytes that ds_decode_sparse_attn needs for this shape, or 0 (with
 * ds_last_error set) if the shape is invalid.  The amount does not depend on
 * the element type or r.
 */
size_t ds_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t block,
                                 int64_t k_units);

/*
 * Whether ds_decode_sparse_attn (and its ragged and offload forms) runs this
 * shape in one pass: 1 when it launches a single kernel that scores each row
 * from the label cache itself, then selects and attends, with no score buffer
 * in memory; 0 when it launches the score kernel and then the fused
 * select + attention kernel (the two phases below); -1 (with ds_last_error set)
 * for an invalid shape.  One pass is taken for token-level rows (block = 1)
 * of at most 32,768 tokens that one fused workgroup handles alone: a single
 * split of the kept set (which holds once B * Hkv reaches about 256, or for
 * k_units <= 64 on a few rows) and groups of 1, 2 or 4 query heads, with
 * label rows of 16 or 32 bytes (r = 8 or 16 for bf16, 4 or 8 for fp32) or,
 * for fp32, 64 bytes (r = 16).
 * Both forms give the same indices and outputs bit for bit.  Host only.
 */
int32_t ds_decode_is_one_pass(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t block,
                              int64_t k_units, int32_t r, ds_dtype dt);

/*
 * One Double Sparsity decode step for every (sequence b, KV head g) (GPU, async):
 *   0. label-row append: rows [t_append, T) of the label cache are rebuilt
 *      from K (as ds_build_label_cache would) before they are scored, so the
 *      newest tokens' rows need no separate call; t_append = T skips it;
 *   1. approximate score of each of the T valid tokens,
 *        u[b,g,t] = sum over query heads h of group g, sum over j < r, of
 *                   q[b,h,channels[g,j]] * label[b,g,t,j]
 *      accumulated in double precision and rounded once to float32;
 *      block > 1: the score of block i is the max of u over its tokens
 *      (Jenga page, core method item 1), the last block may be partial;
 *   2. keep the k_units highest-scoring tokens (block = 1) or blocks, the lower
 *      index winning a tie (Double Sparsity page, method details; HiP page,
 *      abstract), written ascending to `indices`; all query heads of a group
 *      share the group's set;
 *   3. for each query head, softmax(scale * q.K_t) over the kept tokens only
 *      and the weighted sum of their V rows, read in place from the cache
 *      (Jenga page, core method item 3), accumulated in float32.
 *   q            device [B, Hq, d]
 *   K, V         device [B, Hkv, T_cap, d]; rows >= T are never read
 *   label        device [B, Hkv, T_cap, r] (from ds_build_label_cache); rows
 *                [t_append, T) are written, the others only read
 *   channels_dev device int32 [Hkv, r]
 *   T            valid tokens, 1 <= T <= T_cap
 *   t_append     0 <= t_append <= T
 *   block        1, 2, 4, 8, 16, 32 or 64
 *   k_units      tokens or blocks kept, 1 <= k_units <= ceil(T / block)
 *   scale        softmax scale; <= 0 means 1/sqrt(d)
 *   out          device float [B, Hq, d]
 *   indices      device int32 [B, Hkv, k_units] (token ids, or block ids)
 *   workspace    device, >= ds_decode_workspace_bytes(...) bytes; contents on
 *                entry do not matter and are clobbered
 * Errors: null pointer, bad dtype, Hq % Hkv != 0, r outside [1, d], T,
 * t_append, k_units or block out of range, misalignment, unsupported d,
 * workspace too small (DS_ERR_WORKSPACE_TOO_SMALL).
 */
ds_status ds_decode_sparse_attn(const void* q, const void* K, const void* V, void* label, const int32_t* channels_dev,
                                int32_t r, ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                int64_t T, int64_t t_append, int32_t block, int64_t k_units, float scale, float* out,
                                int32_t* indices, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind ds_decode_sparse_attn_noalloc. */
#define DS_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * ds_decode_sparse_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  Same steps, kernels, arguments and results as
 * ds_decode_sparse_attn, without the workspace arguments: the workspace is a
 * static device array of DS_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * one copy per GPU, allocated when the library's device code is loaded onto
 * that GPU and held until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's copy once (hipGetSymbolAddress,
 * with the device current).  Shapes whose workspace
 * (ds_decode_workspace_bytes) exceeds DS_NOALLOC_SCRATCH_BYTES are rejected
 * with DS_ERR_WORKSPACE_TOO_SMALL before any HIP call.  Every call on a GPU
 * shares that GPU's scratch and leaves its contents behind (the kernels clear
 * what must start at zero), so calls that overlap on one GPU, on different
 * streams or threads, race; calls in order on one stream do not.
 * Errors: as ds_decode_sparse_attn, plus DS_ERR_HIP if the scratch cannot be
 * found on the current device.
 */
ds_status ds_decode_sparse_attn_noalloc(const void* q, const void* K, const void* V, void* label,
                                        const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                        int32_t block, int64_t k_units, float scale, float* out, int32_t* indices,
                                        void* stream);

/*
 * The decode step for a batch of sequences of unequal lengths (GPU, async): the
 * incremental decode loop of serving, where the Double Sparsity page's online
 * stage runs on sequences that each hold their own number of tokens.
 * Sequence b holds T_b = seq_lens[b] tokens; every step of
 * ds_decode_sparse_attn is applied to its rows with T replaced by T_b:
 *   0. its last n_append label rows, [T_b - n_append, T_b), are rebuilt from K;
 *   1. it scores its T_b tokens (or ceil(T_b / block) blocks);
 *   2. it keeps k_b = min(k_units, ceil(T_b / block)) units, written ascending
 *      to indices[b, g, 0 .. k_b); slots k_b .. k_units - 1 are set to -1;
 *   3. attention runs over its kept tokens below T_b.
 *   T_max        longest sequence, 1 <= T_max <= T_cap; sizes the workspace
 *                (ds_decode_workspace_bytes with T = T_max) and the score rows
 *   seq_lens_dev device int32 [B]; values are clamped to [1, T_max] on the device
 *   n_append     >= 0 (1 for one decode step; 0 skips the append)
 *   k_units      1 <= k_units <= ceil(T_max / block)
 *   other arguments as for ds_decode_sparse_attn (T = T_max).
 * Errors: as ds_decode_sparse_attn, plus a null or misaligned seq_lens_dev,
 * n_append < 0, and DS_ERR_UNSUPPORTED when ceil(T_max / block) > 32768.
 */
ds_status ds_decode_sparse_attn_ragged(const void* q, const void* K, const void* V, void* label,
                                       const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                       int32_t Hkv, int32_t d, int64_t T_cap, int64_t T_max,
                                       const int32_t* seq_lens_dev, int32_t n_append, int32_t block, int64_t k_units,
                                       float scale, float* out, int32_t* indices, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * The decode step with K and V offloaded to host memory (GPU, async).
 * Post-Training Sparse Attention with Double Sparsity, abstract: the method
 * combines with offloading to cut GPU memory use.  Only the label cache (r of
 * d channels), q, the outputs and the workspace stay in device memory; K and V
 * stay in host memory, and each step moves only the kept rows (and the
 * channels of the appended rows) across the host link, read in place by the
 * kernels.  Same steps, kernels and results as ds_decode_sparse_attn.
 *   K_host, V_host  [B, Hkv, T_cap, d] in pinned host memory that the device
 *                   can access (hipHostMalloc, or a pinned torch tensor)
 *   other arguments as for ds_decode_sparse_attn.
 * Errors: as ds_decode_sparse_attn, plus DS_ERR_INVALID_ARGUMENT when K_host or
 * V_host is not pinned host memory known to HIP.
 */
ds_status ds_decode_sparse_attn_offload(const void* q, const void* K_host, const void* V_host, void* label,
                                        const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                        int32_t block, int64_t k_units, float scale, float* out, int32_t* indices,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * ds_decode_sparse_attn in two phases through one workspace: ds_decode_score
 * runs steps 0 and 1 (label-row append and scoring) and leaves the scores and
 * their per-tile histograms in the workspace; ds_decode_select_attend runs
 * steps 2 and 3 from them.  Issued back to back on one stream with the same
 * shape and workspace, they launch exactly the kernels of
 * ds_decode_sparse_attn and give the same results; the split lets a caller
 * time or schedule the phases.  For a shape that ds_decode_sparse_attn runs
 * in one pass (ds_decode_is_one_pass), the phases still run the two kernels,
 * with the same results bit for bit.  Arguments as for ds_decode_sparse_attn; K and
 * V may also be pinned host memory the device can access, which is how the
 * phases of ds_decode_sparse_attn_offload are run on their own.
 */
ds_status ds_decode_score(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                          ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                          int64_t t_append, int32_t block, int64_t k_units, void* workspace, size_t workspace_bytes,
                          void* stream);

ds_status ds_decode_select_attend(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block, int64_t k_units,
                                  float scale, float* out, int32_t* indices, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * ds_decode_sparse_attn_ragged in the same two phases: ds_decode_score_ragged
 * runs its steps 0 and 1, ds_decode_select_attend_ragged its steps 2 and 3.
 * Issued back to back on one stream with the same shape, seq_lens and
 * workspace, they launch exactly the kernels of ds_decode_sparse_attn_ragged
 * and give the same results.  Arguments and errors as for that call; the
 * select phase reads seq_lens again, so it must not change in between.
 */
ds_status ds_decode_score_ragged(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                                 ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                 int64_t T_max, const int32_t* seq_lens_dev, int32_t n_append, int32_t block,
                                 int64_t k_units, void* workspace, size_t workspace_bytes, void* stream);

ds_status ds_decode_select_attend_ragged(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T_max,
                                         const int32_t* seq_lens_dev, int32_t block, int64_t k_units, float scale,
                                         float* out, int32_t* indices, void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * The decode step with the threshold rule instead of a fixed k (GPU, async).
 * Jenga: Enhancing LLM Long-Context Fine-tuning with Contextual Token Sparsity,
 * core method item 1: a token's informativeness sums the attention scores of
 * the heads, counting only positive ones; a block's is the maximum over its
 * tokens; blocks below a layer-specific threshold are eliminated.  Per row
 * (sequence b, KV head g), with the label approximation of each head's score
 * (Post-Training Sparse Attention with Double Sparsity, abstract):
 *   0. label rows [t_append, T) are rebuilt from K, as in ds_decode_sparse_attn;
 *   1. u[t] = sum over the group's query heads h of max(0, sum_j q[h, ch[g, j]]
 *      * label[t, j]) (float32 of a double-precision sum); block > 1: the
 *      maximum over the block's tokens;
 *   2. the units with score >= tau are kept; when more than k_max pass, the
 *      k_max largest of them (lower index first on ties).  Their number n goes
 *      to counts[b, g]; indices[b, g, 0 .. n) holds them ascending and slots
 *      n .. k_max - 1 are set to -1;
 *   3. attention over the kept tokens, as in ds_decode_sparse_attn; a row that
 *      keeps nothing writes a zero output.
 *   tau     float threshold (a layer's); NaN is rejected, -inf keeps the k_max
 *           largest, +inf keeps nothing
 *   k_max   1 <= k_max <= ceil(T / block): capacity of the index buffer
 *   counts  device int32 [B, Hkv], written by the call
 *   other arguments as for ds_decode_sparse_attn (k_units = k_max).
 * Errors: as ds_decode_sparse_attn, plus a null or misaligned counts, a NaN
 * tau, and DS_ERR_UNSUPPORTED when Hq / Hkv > 8, (Hq / Hkv) * r > 512 or
 * ceil(T / block) > 32768.
 */
ds_status ds_decode_sparse_attn_threshold(const void* q, const void* K, const void* V, void* label,
                                          const int32_t* channels_dev, int32_t r, ds_dtype dt, int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int64_t t_append,
                                          int32_t block, int64_t k_max, float tau, float scale, float* out,
                                          int32_t* indices, int32_t* counts, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * ds_decode_sparse_attn_threshold in two phases through one workspace:
 * ds_decode_score_threshold runs its steps 0 and 1, and
 * ds_decode_select_attend_threshold its steps 2 and 3.  Issued back to back on
 * one stream with the same shape and workspace, they launch exactly the
 * kernels of the one call and give the same results.  Arguments and errors as
 * for that call.
 */
ds_status ds_decode_score_threshold(const void* q, const void* K, void* label, const int32_t* channels_dev, int32_t r,
                                    ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                    int64_t T, int64_t t_append, int32_t block, int64_t k_max, void* workspace,
                                    size_t workspace_bytes, void* stream);

ds_status ds_decode_select_attend_threshold(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                            int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                                            int32_t block, int64_t k_max, float tau, float scale, float* out,
                                            int32_t* indices, int32_t* counts, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Decode with a hierarchical span search instead of label scores (GPU, async).
 * A Training-free Sub-quadratic Cost Transformer Model Serving Framework With
 * Hierarchically Pruned Attention, abstract: nearby key tokens tend to have
 * similar attention scores, so the top-k keys of a query can be estimated by a
 * tree-search-like procedure in O(log T) rounds.  The page gives no algorithm;
 * this library's, per row (sequence b, KV head g):
 *   0. k_spans spans split [0, T) evenly: span i = [floor(i T / k), floor((i+1) T / k));
 *   1. each round, every span longer than `span` tokens is cut into a left part
 *      of ceil(len / 2) tokens and the rest (shorter spans go on whole); each
 *      candidate is scored by its first token t, as the float32 of the exact
 *      double sum over the group's query heads of q_h . K[b, g, t]; the
 *      k_spans best candidates are kept, the lower start winning a tie;
 *   2. the rounds stop when no span is longer than `span` tokens;
 *   3. softmax attention (scale, 1/sqrt(d) when <= 0) over the tokens of the
 *      kept spans.
 *   k_spans  1 <= k_spans <= min(T, 1024)
 *   span     >= 1: longest span the search ends with
 *   out      device fp32 [B, Hq, d]
 *   spans    device int32 [B, Hkv, k_spans, 2]: kept (start, end) pairs, ascending
 *   workspace  ds_hip_workspace_bytes(...) bytes, 256-byte aligned
 * No label cache is used.  Errors: DS_ERR_INVALID_ARGUMENT / UNSUPPORTED as
 * for ds_decode_sparse_attn, DS_ERR_WORKSPACE_TOO_SMALL, DS_ERR_HIP.
 */
ds_status ds_decode_hip_attn(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t k_spans, int32_t span,
                             float scale, float* out, int32_t* spans, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes of ds_decode_hip_attn, or 0 (ds_last_error set) for an invalid shape. */
size_t ds_hip_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T, int32_t k_spans,
                              int32_t span);

/* Tokens one row of the search can cover: k_spans * span when a round runs,
 * else T (the first spans cover every token); 0 for invalid arguments. */
int64_t ds_hip_token_capacity(int64_t T, int64_t k_spans, int64_t span);

/* Steps 0-2 only: the kept spans [B, Hkv, k_spans, 2] and the covered token
 * ids tokens [B, Hkv, capacity] (int32, ascending, -1 after the last), with
 * capacity = ds_hip_token_capacity(T, k_spans, span).  Step 3 is then
 * ds_sparse_attn_from_indices with block = 1 and k_units = capacity. */
ds_status ds_hip_search(const void* q, const void* K, ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                        int64_t T_cap, int64_t T, int32_t k_spans, int32_t span, int32_t* spans, int32_t* tokens,
                        void* stream);

/*
 * Stages of the decode step fed from caller buffers, so each can be checked in
 * isolation against independently computed inputs.
 */

/* Step 1 only: scores[b, g, i] (float32) for i < ceil(T / block).
 *   scores  device float [B, Hkv, ld], ld >= ceil(T / block), ld % 4 == 0 */
ds_status ds_label_scores(const void* q, const void* label, const int32_t* channels_dev, int32_t r, ds_dtype dt,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block,
                          float* scores, int64_t ld, void* stream);

/* Step 1 of the threshold rule only: scores[b, g, i] = the positive-only
 * aggregation of ds_decode_sparse_attn_threshold, laid out as for
 * ds_label_scores.  DS_ERR_UNSUPPORTED when Hq / Hkv > 8 or (Hq / Hkv) * r > 512. */
ds_status ds_label_scores_positive(const void* q, const void* label, const int32_t* channels_dev, int32_t r,
                                   ds_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap,
                                   int64_t T, int32_t block, float* scores, int64_t ld, void* stream);

/* Step 2 only: per row of `scores` (rows x n, row stride ld floats), the k
 * largest values, the lower index winning a tie, written ascending to
 * idx_out [rows, k].  Values are compared as float32 (-0.0 equals +0.0);
 * NaN is not supported. */
ds_status ds_topk_select(const float* scores, int64_t rows, int64_t n, int64_t ld, int64_t k, int32_t* idx_out,
                         void* stream);

/* Steps 2 and 3 from given scores (laid out as ds_label_scores writes them):
 * selection and attention, exactly as ds_decode_sparse_attn runs them after
 * scoring.  Workspace as for ds_decode_sparse_attn. */
ds_status ds_select_attention(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t d, int64_t T_cap, int64_t T, int32_t block, int64_t k_units,
                              const float* scores, int64_t ld, float scale, float* out, int32_t* indices,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Step 3 only: attention over the units listed in `indices` (as
 * ds_decode_sparse_attn writes them: ascending, distinct, each < ceil(T/block);
 * entries of -1 are skipped, as ds_hip_search pads its token lists).
 * Workspace as for ds_decode_sparse_attn. */
ds_status ds_sparse_attn_from_indices(const void* q, const void* K, const void* V, ds_dtype dt, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t d, int64_t T_cap, int64_t T,
                                      int32_t block, int64_t k_units, const int32_t* indices, float scale,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DS_SPARSE_DECODE_H */
