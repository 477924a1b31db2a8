// Fused top-k selection and sparse attention, one launch per decode step.
// In its one-pass form (LNV > 0) the same kernel also scores the row from the
// label cache first, so that a step whose rows each fit one workgroup is a
// single launch with no score buffer in memory.
//
// Double Sparsity page, method details and abstract: keep the tokens with the
// highest approximate scores, then compute self-attention over those tokens
// only.  Jenga page, core method item 3: kept K/V rows are read in place from
// the cache by index.
//
// One workgroup per (row = b * Hkv + g, head chunk, split).  Every workgroup of
// a row reads the row's scores (from L2 / Infinity Cache: the row was just
// written by the score kernel) and finds the row's exact threshold itself, so
// no workgroup waits for another before its gather and the kept indices never
// make a round trip through memory.  Split s owns kept positions
// [s * chunk, (s + 1) * chunk) of the ascending kept list: it writes those
// indices, and gathers and attends over those rows only.  When a row has one
// split the workgroup writes the normalised output.  Otherwise it publishes
// its softmax state (m, l, unnormalised acc) and takes a ticket; the row's last
// workgroup merges the states by log-sum-exp and writes the output.
// Workgroups of a row may run on different XCDs, whose L2 caches are not kept
// coherent with each other, so the states go through agent-scope accesses
// (written through past the L2, read around it), and a workgroup's stores have
// completed (s_waitcnt) before its ticket is taken.  No cache-wide writeback
// or invalidate is needed.
//
// Selection (exact k largest, lower index wins a tie).  Thread t holds units
// [t * ITEMS, (t + 1) * ITEMS) of the row.  The top 11 bits of the
// order-preserving score key give the first radix digit; its histogram comes
// from the score kernel's per-tile histograms (or is built here), and one
// workgroup prefix sum over the bins, highest first, finds the digit d0 that
// holds the k-th largest key.  Every unit is then classified with two float
// comparisons against the bounds of d0 into two per-thread bit masks: "above
// d0" (always kept) and "in d0" (candidates).  Only the few candidates are
// revisited (bit scans over the mask, keys read back from LDS) for the 11-bit
// and, when still needed, the 10-bit radix passes.  A last prefix sum over the
// per-thread kept counts gives every kept unit its position in the ascending
// output list.
//
// Threshold rule (Jenga page, core method item 1), when a counts buffer is
// given: the units scoring at least tau are kept, at most k of them (the k
// largest when more pass).  Their number comes with the first prefix sum (a
// second 16-bit count packed beside the bin counts); when it is at most k the
// kept set is exactly the passing units, so the radix passes are skipped and
// the prefix sum over the pass masks alone places them.  Otherwise the top-k
// search runs as usual and every unit it keeps passes.
//
// Eight query heads per workgroup (GQA groups of 8 in bf16, the long rows of
// the two-stage selection): the attention runs on the matrix cores, so each
// kept K/V row is read once for all eight heads.  A wavefront takes 16 kept
// tokens per step.  S^T = K q^T (16 tokens x 16 head slots, eight used) comes
// from four v_mfma_f32_16x16x32_bf16 over the 128 channels, taken in an order
// in which every lane's share of a K row is 32 contiguous channels; the online
// softmax runs on that tile (a head's 16 tokens lie in one lane column of
// four lanes); O^T += V^T P^T is 16 v_mfma_f32_16x16x16_bf16 with P split
// into a bf16 head and remainder (each lane's share of a V row is 8
// contiguous channels, the output channels permuted to match).  The state then takes the lane path's way to LDS.
#include "fused_dev.h"
#include "label_dot.h"

DS_STAMP_BUFFER(selattn)

namespace ds {
namespace {

constexpr int kMaxChunk = int(kFusedMaxChunk);

template <int NT, int ITEMS, int HC>
struct FusedSmem {
  static constexpr int NW = NT / 64;
  union {
    float sc[NT * ITEMS];   // the row's scores, while the threshold is found
    struct {
      int32_t sel[kMaxChunk];                 // this split's kept unit ids
      float wacc[NW][HC][kHeadDim];           // per-wavefront attention states
    } a;
  } u;
  uint32_t hist1[2048];     // top-digit histogram (when built here), then bits 20..10 of the candidates
  uint32_t hist2[1024];     // bits 9..0
  uint32_t wsum[4][NW];     // one per prefix sum, so none needs a trailing barrier
  float wm[NW][HC], wl[NW][HC];
  __align__(16) float wf[HC][NW];   // each wavefront's weight in the combined state, per head
  float hm[HC], hl[HC];             // the combined maximum and denominator, per head
  uint32_t pick[3];         // digit, count above it, count in it
  unsigned ticket;
};

// Kernel arguments, with the derived sizes precomputed on the host so the
// kernel's prologue is a few 32-bit operations (passed to the kernel as
// separate scalars).
struct FusedArgs {
  const void* q;
  const void* K;
  const void* V;
  const float* scores;
  const uint16_t* tile_hist;   // null: the kernel builds the top-digit histogram itself
  int32_t* indices;
  float* part_acc;
  float* part_ml;
  float* out;
  unsigned* tickets;
  int64_t ld, T_cap;
  int32_t T, n_units, k_units, G, head_chunks, tiles;
  int32_t lb;                  // log2(block)
  int32_t kv_virtual, chunk, n_split;
  float scale;
  const int32_t* seq_lens;     // null: every sequence holds T tokens
  int32_t Hkv;
  float tau;                   // threshold rule: keep units scoring >= tau (at most k_units)
  int32_t* counts;             // threshold rule: kept units per row; null: plain top-k
  const int32_t* unit_ids;     // the units are candidates with these unit ids [rows][n_units]; null: identity
  int32_t xcd_rows;            // grid (8, n_split, rows * head_chunks / 8): row = 8 (z / head_chunks) + x
  // One pass (scores null): the kernel scores the row from its label rows
  // [rows][T_cap][r] with channels ch [Hkv][r], rebuilding rows [t_append, T)
  // (ragged: the last n_append of each sequence) from K first.
  void* label;
  const int32_t* ch;
  int32_t r, t_append, n_append;
};

// Scalar arguments, those of the first loads first: the first 15 dwords (up to
// lb_) are preloaded into SGPRs at wave launch where the firmware supports it.
// RAGGED: sequence b holds seq_lens[b] tokens (clamped to [1, T]) and keeps
// min(k_units, its unit count) units; index slots past that are set to -1.
// counts_ != null: the threshold rule with tau_ (index slots past a row's kept
// count are -1; a row that keeps nothing gets a zero output).
// LNV > 0: one pass, for token-level rows that one workgroup handles alone (a
// single split and head chunk): the row's scores are computed here from its
// label rows of LNV 16-byte words, with the score kernel's arithmetic, instead
// of being read from scores_; no tile histograms.
template <typename TE, int NT, int ITEMS, int HC, bool RAGGED, int LNV>
__global__ __launch_bounds__(NT) void selattn_kernel(
    const void* q_, const float* scores_, const uint16_t* tile_hist_, int64_t ld_, int32_t G_,
    int32_t head_chunks_, int32_t xcd_rows_, int32_t n_units_, int32_t tiles_, int32_t k_units_, int32_t lb_,
    const void* K_,
    const void* V_, int32_t* indices_, float* part_acc_, float* part_ml_, float* out_, unsigned* tickets_,
    int64_t T_cap_, int32_t T_, int32_t kv_virtual_, int32_t chunk_, int32_t n_split_, float scale_,
    const int32_t* seq_lens_, int32_t Hkv_, float tau_, int32_t* counts_, const int32_t* unit_ids_, void* label_,
    const int32_t* ch_, int32_t r_, int32_t t_append_, int32_t n_append_) {
  FusedArgs a;
  a.label = label_;
  a.ch = ch_;
  a.r = r_;
  a.t_append = t_append_;
  a.n_append = n_append_;
  a.q = q_;
  a.K = K_;
  a.V = V_;
  a.scores = scores_;
  a.tile_hist = tile_hist_;
  a.indices = indices_;
  a.part_acc = part_acc_;
  a.part_ml = part_ml_;
  a.out = out_;
  a.tickets = tickets_;
  a.ld = ld_;
  a.T_cap = T_cap_;
  a.T = T_;
  a.n_units = n_units_;
  a.k_units = k_units_;
  a.G = G_;
  a.head_chunks = head_chunks_;
  a.tiles = tiles_;
  a.lb = lb_;
  a.kv_virtual = kv_virtual_;
  a.chunk = chunk_;
  a.n_split = n_split_;
  a.scale = scale_;
  a.seq_lens = seq_lens_;
  a.Hkv = Hkv_;
  a.tau = tau_;
  a.counts = counts_;
  a.unit_ids = unit_ids_;
  a.xcd_rows = xcd_rows_;
  using LN = Lanes<TE, NT>;
  DS_STAMP_START(selattn);
  constexpr int NW = LN::NW, EPL = LN::EPL, LPT = LN::LPT, GPW = LN::GPW, NG = LN::NG, KU = LN::KU;
  constexpr int BPT1 = 2048 / NT, BPT2 = 1024 / NT;
  static_assert(ITEMS % 4 == 0 && ITEMS <= 32, "per-thread masks are 32 bits");
  static_assert(BPT2 >= 1 && (BPT1 & 1) == 0, "two or more top-digit bins per thread");
  __shared__ FusedSmem<NT, ITEMS, HC> sm;

  // Grid (8, n_split, rows * head_chunks / 8) when the row count is a
  // multiple of 8, else (rows * head_chunks, n_split, 1).  Workgroups are dealt
  // to the 8 XCDs round-robin by linear id (x fastest), so in the first layout
  // blockIdx.x is the XCD, row = 8 * (z / head_chunks) + x and the head chunk
  // is z % head_chunks: every split and every head chunk of a row lands on the
  // same XCD, whose L2 then serves the row's scores and histograms, and the
  // K/V rows that the head chunks of a GQA group all read, once.  Queries of
  // the row are heads row * G + [0, G).
  const uint32_t split = blockIdx.y;
  const uint32_t hcs = uint32_t(a.head_chunks);
  uint32_t row, hchunk;
  if (a.xcd_rows) {
    const uint32_t zr = hcs == 1 ? blockIdx.z : blockIdx.z / hcs;
    row = zr * kXcds + blockIdx.x;
    hchunk = blockIdx.z - zr * hcs;
  } else {
    row = hcs == 1 ? blockIdx.x : blockIdx.x / hcs;
    hchunk = blockIdx.x - row * hcs;
  }
  const uint32_t rc = row * hcs + hchunk;
  const int64_t bh0 = int64_t(row) * a.G + int64_t(hchunk) * HC;   // first (b, h) of this chunk
  const TE* __restrict__ q = static_cast<const TE*>(a.q);
  const TE* __restrict__ K = static_cast<const TE*>(a.K);
  const TE* __restrict__ V = static_cast<const TE*>(a.V);
  const int n_units = a.n_units, k_units = a.k_units, lb = a.lb, block = 1 << a.lb;
  const int n_split = a.n_split;
  // This row's token count and kept-unit count.
  int T_row = a.T, k_row = k_units;
  if constexpr (RAGGED) {
    const uint32_t b = row / uint32_t(a.Hkv);
    T_row = min(max(a.seq_lens[b], 1), a.T);
    k_row = min(k_units, (T_row + block - 1) >> lb);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPT, sub = lane % LPT;
  const int gid = wave * GPW + grp;

  // Loads first: q (consumed only after the selection), the thread's scores,
  // and the tile histograms of its top-digit bins.  The matrix-core path holds
  // q as the B operand of S^T = K q^T: lane (16 g + j) has channels
  // [32 g, 32 g + 32) of head j (zero for the padding heads j >= HC).
  constexpr bool kMfma = HC == 8 && sizeof(TE) == 2;
  constexpr int NQ = kMfma ? 4 : HC;
  uint4 qraw[NQ];
  if constexpr (kMfma) {
    const int hq = (lane & 15) < HC ? (lane & 15) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qraw[i] = *reinterpret_cast<const uint4*>(q + (bh0 + hq) * kHeadDim + 32 * (lane >> 4) + 8 * i);
    if ((lane & 15) >= HC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qraw[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
#pragma unroll
    for (int h = 0; h < HC; ++h)
      qraw[h] = *reinterpret_cast<const uint4*>(q + (bh0 + h) * kHeadDim + sub * EPL);
  }
  const int first = tid * ITEMS;
  float s[ITEMS];
  if constexpr (LNV > 0) {
    // One pass: score the row here.  Pass c covers units c * NT + tid (a
    // wavefront reads 64 consecutive label rows per load), each score going
    // to the LDS slot of its owner thread; the owners read them back below.
    constexpr int R = LNV * 16 / int(sizeof(TE));   // label channels
    // Passes whose label rows are requested together (64 bytes per thread:
    // measured faster than 128 or 32, the other wavefronts covering the
    // latency), never more than the ITEMS passes there are: a unit of a pass
    // past ITEMS would have no slot.
    constexpr int CB0 = LNV == 1 ? 4 : LNV == 2 ? 2 : 1;
    constexpr int CB = CB0 < ITEMS ? CB0 : ITEMS;
    static_assert(ITEMS % CB == 0, "whole batches of passes");
    __shared__ double qs_l[R];
    __shared__ int ch_l[R];
    const int g = int(row % uint32_t(a.Hkv));
    if (tid < R) {
      const int cj = a.ch[g * R + tid];
      qs_l[tid] = group_q_sum(q + int64_t(row) * a.G * kHeadDim, a.G, cj);
      ch_l[tid] = cj;
    }
    TE* lab = static_cast<TE*>(a.label) + int64_t(row) * a.T_cap * R;
    // Label rows are read once per call.  When the call's label rows exceed
    // the XCDs' combined L2 (8 x 4 MB) they cannot stay cached from one call
    // to the next, and they are streamed with non-temporal loads (measured
    // faster on the 268 MB and 67 MB streams of the batched and ragged
    // workloads); a smaller set is read through the caches, where a repeated
    // call may find it (a single 1024-token row: 7.2 against 8.9 us).
    const int64_t n_rows = int64_t(gridDim.x) * gridDim.z / a.head_chunks;
    const bool nt_labels = n_rows * int64_t(a.T) * R * int64_t(sizeof(TE)) >= (int64_t(32) << 20);
    const int ta = RAGGED ? max(T_row - a.n_append, 0) : a.t_append;   // rows rebuilt from K
    // The top-digit histogram is built as the scores come in, its LDS atomics
    // overlapping the next passes' label loads.
#pragma unroll
    for (int i = 0; i < BPT1; ++i) sm.hist1[i * NT + tid] = 0u;
    __syncthreads();
    double qr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qr[j] = qs_l[j];
    for (int c0 = 0; c0 < ITEMS; c0 += CB) {
      if (c0 * NT >= T_row) {   // (uniform) passes wholly past the sequence: no loads, -inf scores
#pragma unroll
        for (int i = 0; i < CB; ++i) {
          const int u = (c0 + i) * NT + tid;
          const int ut = u / ITEMS, uj = u % ITEMS;
          sm.u.sc[((uj >> 2) * NT + ut) * 4 + (uj & 3)] = -INFINITY;
        }
        continue;
      }
      uint4 raw[CB][LNV];
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int u = (c0 + i) * NT + tid;
        const uint4* p = reinterpret_cast<const uint4*>(lab + int64_t(u < T_row ? u : 0) * R);   // row 0 exists
#pragma unroll
        for (int v = 0; v < LNV; ++v) {
          if (nt_labels) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + v));
            raw[i][v] = make_uint4(x.x, x.y, x.z, x.w);
          } else {
            raw[i][v] = p[v];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int u = (c0 + i) * NT + tid;
        float sv;
        if (u >= T_row) sv = -INFINITY;   // past the sequence (and the row's units)
        else if (u >= ta)
          sv = append_row(K + (int64_t(row) * a.T_cap + u) * kHeadDim, lab + int64_t(u) * R, ch_l, qs_l, R);
        else sv = float(dot_label<LNV>(raw[i], qr, TE()));
        if (u < T_row) atomicAdd(&sm.hist1[float_key(sv) >> 21], 1u);   // the sequence's units only
        const int ut = u / ITEMS, uj = u % ITEMS;
        sm.u.sc[((uj >> 2) * NT + ut) * 4 + (uj & 3)] = sv;
      }
    }
    __syncthreads();
    DS_STAMP(selattn, 16);   // one pass: the row's label rows scored
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) s[j] = sm.u.sc[((j >> 2) * NT + tid) * 4 + (j & 3)];
  } else if (first + ITEMS <= n_units) {
    const float* srow = a.scores + int64_t(row) * a.ld;   // 16-byte aligned: ld is a multiple of 4
#pragma unroll
    for (int v = 0; v < ITEMS / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(srow + first + 4 * v);
      s[4 * v + 0] = f.x;
      s[4 * v + 1] = f.y;
      s[4 * v + 2] = f.z;
      s[4 * v + 3] = f.w;
    }
  } else {
    const float* srow = a.scores + int64_t(row) * a.ld;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) s[j] = first + j < n_units ? srow[first + j] : -INFINITY;
  }
  // Packed pairs of 16-bit bin counts; a bin's total over the row is at most
  // n_units <= 32768, so the packed sums never carry between halves.
  uint32_t hw[BPT1 / 2];
#pragma unroll
  for (int i = 0; i < BPT1 / 2; ++i) hw[i] = 0u;
  const int tiles = a.tiles;
  if (a.tile_hist != nullptr) {
    const uint32_t* th = reinterpret_cast<const uint32_t*>(a.tile_hist + int64_t(row) * tiles * kHistBins) +
                         (kHistBins - BPT1 * (tid + 1)) / 2;
    // Every load is issued unconditionally (tile index clamped, value masked):
    // a load inside a branch makes the compiler wait for it at the join.
    uint32_t w[kMaxHistTiles][BPT1 / 2];
#pragma unroll
    for (int t = 0; t < int(kMaxHistTiles); ++t)
#pragma unroll
      for (int i = 0; i < BPT1 / 2; ++i) w[t][i] = th[(t < tiles ? t : 0) * (kHistBins / 2) + i];
#pragma unroll
    for (int t = 0; t < int(kMaxHistTiles); ++t)
#pragma unroll
      for (int i = 0; i < BPT1 / 2; ++i) hw[i] += t < tiles ? w[t][i] : 0u;
  }

  // The scores go to LDS as well, for the candidate passes' indexed reads of
  // a thread's own units (a register array cannot be indexed at run time).
  // Thread t's units 4v .. 4v + 3 sit in 16-byte slot v * NT + t, so a
  // wavefront's stores cover consecutive slots: written at the thread's own
  // 64-byte stride instead, all 64 lanes of a store hit the same few banks
  // and the stores took ~6K clocks per workgroup.
  // (One pass: they are there already.)
  const auto sc_at = [&](int j) -> float { return sm.u.sc[((j >> 2) * NT + tid) * 4 + (j & 3)]; };
  if constexpr (LNV == 0) {
#pragma unroll
    for (int v = 0; v < ITEMS / 4; ++v)
      *reinterpret_cast<float4*>(&sm.u.sc[(v * NT + tid) * 4]) =
          make_float4(s[4 * v], s[4 * v + 1], s[4 * v + 2], s[4 * v + 3]);
  }
  uint32_t c1[BPT1];
  if (a.tile_hist != nullptr) {
#pragma unroll
    for (int i = 0; i < BPT1; ++i) sm.hist1[i * NT + tid] = 0u;
    // Word i holds bins lo + 2i (low half) and lo + 2i + 1 (high half).
#pragma unroll
    for (int i = 0; i < BPT1 / 2; ++i) {
      c1[BPT1 - 1 - 2 * i] = hw[i] & 0xFFFFu;
      c1[BPT1 - 2 - 2 * i] = hw[i] >> 16;
    }
  } else {
    if constexpr (LNV == 0) {   // (one pass: built while scoring)
      // The units of this sequence only (a short one's padding would pile onto one bin).
      const int nu_hist = RAGGED ? ((T_row + block - 1) >> lb) : n_units;
#pragma unroll
      for (int i = 0; i < BPT1; ++i) sm.hist1[i * NT + tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (first + j < nu_hist) atomicAdd(&sm.hist1[float_key(s[j]) >> 21], 1u);
      __syncthreads();
    }
    read_bins<NT, 2048>(sm.hist1, c1);
    // Each bin is read by exactly one thread, which clears it for pass 1.
    const int lo = 2048 - BPT1 * (tid + 1);
#pragma unroll
    for (int i = 0; i < BPT1; ++i) sm.hist1[lo + i] = 0u;
  }
#pragma unroll
  for (int i = 0; i < BPT2; ++i) sm.hist2[i * NT + tid] = 0u;

  // Threshold rule: this thread's units scoring at least tau (-inf padding and
  // units past a short sequence never count).
  DS_STAMP(selattn, 2);   // scores and top-digit counts in
  const bool thresh = a.counts != nullptr;
  uint32_t passm = 0u;
  if (thresh) {
    const int nu_row = RAGGED ? ((T_row + block - 1) >> lb) : n_units;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) passm |= uint32_t(first + j < nu_row && s[j] >= a.tau) << j;
  }

  // Pass 0: the top digit d0 holding the k-th largest key (and the number of
  // units passing the threshold).
  const uint32_t k = uint32_t(k_row);
  const uint32_t n_pass = pick_bin<NT, 2048>(c1, k, sm.wsum[0], sm.pick, uint32_t(__popc(passm)));
  __syncthreads();
  DS_STAMP(selattn, 3);   // d0
  // Kept units of the row; with the threshold rule, when no more than k pass,
  // they are exactly the passing ones and the search below is skipped.
  int k_keep = k_row;
  bool compact = false;
  if (thresh) {
    k_keep = min(k_row, int(n_pass));
    compact = int(n_pass) <= k_row;
  }
  uint32_t keepm = passm, eqm = 0u, eq_take = 0u;
  if (!compact) {
    const uint32_t d0 = sm.pick[0];
    uint32_t kk = k - sm.pick[1];   // keys still needed from digit d0
    const uint32_t cnt0 = sm.pick[2];

    // Classify: finite scores have keys in [0x00800000, 0xFF7FFFFF], so
    // 4 <= d0 <= 2043 and both bounds are non-NaN floats; comparing floats is
    // comparing keys (-0.0 and +0.0 share a key and compare equal).  Padding
    // units hold -inf, below every bound.
    const float f_lo = key_float(d0 << 21), f_hi = key_float((d0 + 1u) << 21);
    uint32_t gtm = 0u, cm = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const bool hi = s[j] >= f_hi;
      const bool in = s[j] >= f_lo && !hi;
      gtm |= uint32_t(hi) << j;
      cm |= uint32_t(in) << j;
    }

    // Narrow the threshold inside d0: thr is a key, eq_take the number of keys
    // equal to thr to keep (lowest unit ids first), all_eq when that is all of them.
    DS_STAMP(selattn, 4);   // units classified against d0
    uint32_t thr = d0 << 21;
    bool all_eq = true;
    bool settled = kk == cnt0;   // every key of digit d0 is needed
    if (!settled) {
      for (uint32_t m = cm; m != 0u; m &= m - 1u) {
        const uint32_t key = float_key(sc_at(__builtin_ctz(m)));
        atomicAdd(&sm.hist1[(key >> 10) & 2047u], 1u);
      }
      __syncthreads();
      uint32_t c[BPT1];
      read_bins<NT, 2048>(sm.hist1, c);
      DS_STAMP(selattn, 5);   // first candidate pass's histogram
      pick_bin<NT, 2048>(c, kk, sm.wsum[1], sm.pick);
      __syncthreads();
      thr |= sm.pick[0] << 10;
      kk -= sm.pick[1];
      settled = kk == sm.pick[2];
      if (!settled) {
        for (uint32_t m = cm; m != 0u; m &= m - 1u) {
          const uint32_t key = float_key(sc_at(__builtin_ctz(m)));
          if ((key & 0xFFFFFC00u) == thr) atomicAdd(&sm.hist2[key & 1023u], 1u);
        }
        __syncthreads();
        uint32_t c2[BPT2];
        read_bins<NT, 1024>(sm.hist2, c2);
        DS_STAMP(selattn, 6);   // second candidate pass's histogram
        pick_bin<NT, 1024>(c2, kk, sm.wsum[2], sm.pick);
        __syncthreads();
        thr |= sm.pick[0];
        kk -= sm.pick[1];
        all_eq = kk == sm.pick[2];
        eq_take = kk;
      }
    }

    // Kept units of this thread: above d0, plus candidates at or above thr (when
    // all keys equal to a full-precision thr are kept), or above thr and the
    // first eq_take equal ones in unit order.
    DS_STAMP(selattn, 7);   // exact threshold
    keepm = gtm;
    if (thr == (d0 << 21) && all_eq) {
      keepm |= cm;
    } else {
      for (uint32_t m = cm; m != 0u; m &= m - 1u) {
        const int j = __builtin_ctz(m);
        const uint32_t key = float_key(sc_at(j));
        if (key > thr || (all_eq && key == thr)) keepm |= 1u << j;
        else if (key == thr) eqm |= 1u << j;
      }
    }
  }   // !compact
  DS_STAMP(selattn, 8);   // kept units classified
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan1<NT>((uint32_t(__popc(keepm)) << 16) | uint32_t(__popc(eqm)),
                                                sm.wsum[3], tot);
  // Past this barrier (inside the scan) the scores in LDS are dead: sel reuses them.
  const int p_begin = int(split) * a.chunk;   // virtual positions of this split
  const int p_end = min(min(p_begin + a.chunk, a.kv_virtual), k_keep << lb);
  const int u_lo = p_begin >> lb;
  const int u_hi = (min(p_begin + a.chunk, a.kv_virtual) + block - 1) >> lb;   // kept-list slots of this split
  {
    // This thread's kept units: keepm, plus its first n_eq units equal to the
    // threshold (the tied units kept go lowest unit first across the row).
    // They take positions [pos, pos + popc(takem)) in unit order; only a thread
    // whose range meets this split's slots walks them.
    const uint32_t eq_seen = ex & 0xFFFFu;
    int pos = int(ex >> 16) + int(min(eq_seen, eq_take));
    const uint32_t n_eq = min(uint32_t(__popc(eqm)), eq_take > eq_seen ? eq_take - eq_seen : 0u);
    uint32_t takem = keepm;
    if (n_eq == uint32_t(__popc(eqm))) {
      takem |= eqm;
    } else {
      uint32_t m = eqm;
      for (uint32_t i = 0; i < n_eq; ++i, m &= m - 1u) takem |= m & (0u - m);
    }
    if (pos < u_hi && pos + __popc(takem) > u_lo)
      for (uint32_t m = takem; m != 0u; m &= m - 1u, ++pos)
        if (pos >= u_lo && pos < u_hi) sm.u.a.sel[pos - u_lo] = first + __builtin_ctz(m);
  }
  __syncthreads();
  DS_STAMP(selattn, 9);   // the split's kept list in LDS
  if (a.unit_ids != nullptr) {
    // Candidates of a long row: their kept slots become the units they stand for.
    const int32_t* ids = a.unit_ids + int64_t(row) * n_units;
    for (int i = tid; i < u_hi - u_lo; i += NT)
      if (u_lo + i < k_keep) sm.u.a.sel[i] = ids[sm.u.a.sel[i]];
    __syncthreads();
  }
  DS_STAMP(selattn, 10);   // candidate slots mapped to units
  if (hchunk == 0) {
    int32_t* ridx = a.indices + int64_t(row) * k_units + u_lo;
    for (int i = tid; i < u_hi - u_lo; i += NT) ridx[i] = u_lo + i < k_keep ? sm.u.a.sel[i] : -1;
    if (thresh && split == 0 && tid == 0) a.counts[row] = k_keep;
  }

  DS_STAMP(selattn, 11);   // indices written
  // Attention over the split's kept rows.
  if constexpr (kMfma) {
    // Kept position p of this split: its token, and whether it is one.
    const auto token_at = [&](int p, bool& ok) -> int64_t {
      const bool in = p < p_end;
      const int rel = in ? p - p_begin : 0;
      const int unit = in ? sm.u.a.sel[rel >> lb] : 0;
      const int64_t t = (int64_t(unit) << lb) + (rel & (block - 1));
      ok = in && unit >= 0 && t < T_row;
      return ok ? t : 0;
    };
    const int g = lane >> 4, j = lane & 15;
    bf16x8_t qb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = __builtin_bit_cast(bf16x8_t, qraw[i]);
    const TE* Kb = K + int64_t(row) * a.T_cap * kHeadDim;
    const TE* Vb = V + int64_t(row) * a.T_cap * kHeadDim;
    float M = -INFINITY, L = 0.f;   // head j's running maximum and denominator
    f32x4_t o[8];                   // O^T rows 4 g + r of channel tile c: channel 8 (4 g + r) + c, head j
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int base = p_begin; base < p_end; base += NW * 16) {
      const int pw = base + wave * 16;   // this wavefront's 16 positions
      bool okk, okv[4];
      const int64_t tk = token_at(pw + j, okk);   // K row of slot j
      int64_t tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[i] = token_at(pw + 4 * g + i, okv[i]);   // V rows of slots 4 g + i
      // Unconditional loads (a slot that is not kept reads token 0 and is masked).
      uint4 kq[4], vq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kq[i] = *reinterpret_cast<const uint4*>(Kb + tk * kHeadDim + 32 * g + 8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) vq[i] = *reinterpret_cast<const uint4*>(Vb + tv[i] * kHeadDim + 8 * j);
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};   // S^T rows 4 g + r (slots), column j (head)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[i]), qb[i], d, 0, 0, 0);
      float z[4], mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = okv[r] ? d[r] * a.scale : -INFINITY;
        mt = fmaxf(mt, z[r]);
      }
      float m16, m32;
      pair_values<16>(mt, m16, m32);
      mt = fmaxf(m16, m32);
      pair_values<32>(mt, m16, m32);
      mt = fmaxf(m16, m32);   // head j's maximum over the 16 slots
      const float Mn = fmaxf(M, mt);
      const float alpha = Mn == -INFINITY ? 1.f : __expf(M - Mn);
      float pr[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = z[r] == -INFINITY ? 0.f : __expf(z[r] - Mn);
        ps += pr[r];
      }
      float s16, s32;
      pair_values<16>(ps, s16, s32);
      ps = s16 + s32;
      pair_values<32>(ps, s16, s32);
      ps = s16 + s32;
      L = L * alpha + ps;
      M = Mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] *= alpha;
      // O^T += V^T P^T over the 16 slots: per channel tile c, A = V^T (lane
      // 16 g + j: channel 8 j + c of slots 4 g .. 4 g + 3, exact in bf16) and
      // B = P^T (the lane's own four slots of head j), P being split into a
      // bf16 head and a bf16 remainder (P = hi + lo to about 2^-16 relative),
      // so two bf16 products give P V in fp32 accumulation.
      uint32_t phi[2], plo[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t a = bf16_rne(pr[2 * h2]), b = bf16_rne(pr[2 * h2 + 1]);
        phi[h2] = a | (b << 16);
        const uint32_t ra = bf16_rne(pr[2 * h2] - __uint_as_float(a << 16));
        const uint32_t rb = bf16_rne(pr[2 * h2 + 1] - __uint_as_float(b << 16));
        plo[h2] = ra | (rb << 16);
      }
      const bf16x4_t bh = __builtin_bit_cast(bf16x4_t, make_uint2(phi[0], phi[1]));
      const bf16x4_t bl = __builtin_bit_cast(bf16x4_t, make_uint2(plo[0], plo[1]));
      const uint32_t vw[4][4] = {{vq[0].x, vq[0].y, vq[0].z, vq[0].w}, {vq[1].x, vq[1].y, vq[1].z, vq[1].w},
                                 {vq[2].x, vq[2].y, vq[2].z, vq[2].w}, {vq[3].x, vq[3].y, vq[3].z, vq[3].w}};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // bf16 element c of each slot's 8 channels: half (c & 1) of word c / 2.
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(vw[1][c >> 1], vw[0][c >> 1], sel);
        const uint32_t hi = __builtin_amdgcn_perm(vw[3][c >> 1], vw[2][c >> 1], sel);
        const bf16x4_t av = __builtin_bit_cast(bf16x4_t, make_uint2(lo, hi));
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bh, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bl, o[c], 0, 0, 0);
      }
    }
    DS_STAMP(selattn, 12);   // wavefront 0's gather
    if (j < HC) {
      if (g == 0) {
        sm.wm[wave][j] = M;
        sm.wl[wave][j] = L;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.u.a.wacc[wave][j][8 * (4 * g + r) + c] = o[c][r];
    }
  } else {
    float qv[HC][EPL];
  #pragma unroll
    for (int h = 0; h < HC; ++h) {
      unpack(qraw[h], qv[h], TE());
  #pragma unroll
      for (int e = 0; e < EPL; ++e) qv[h][e] *= a.scale;
    }
    float m[HC], l[HC], acc[HC][EPL];
  #pragma unroll
    for (int h = 0; h < HC; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
  #pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
    const TE* Kr = K + int64_t(row) * a.T_cap * kHeadDim + sub * EPL;
    const TE* Vr = V + int64_t(row) * a.T_cap * kHeadDim + sub * EPL;
    for (int base = p_begin; base < p_end; base += NG * KU) {
      // Loads are unconditional: a position past the split or an invalid entry
      // reads token 0 of the row (which exists) and is masked out of the
      // softmax; a load inside a branch would make the compiler wait for it
      // where the branches join.
      int64_t tok[KU];
      bool ok[KU];
  #pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int p = base + gid * KU + u;
        const bool in = p < p_end;
        const int rel = in ? p - p_begin : 0;
        const int unit = in ? sm.u.a.sel[rel >> lb] : 0;
        const int64_t t = (int64_t(unit) << lb) + (rel & (block - 1));
        ok[u] = in && unit >= 0 && t < T_row;   // always true for p < p_end when the kept list is whole
        tok[u] = ok[u] ? t : 0;
      }
      uint4 kr[KU], vr[KU];
  #pragma unroll
      for (int u = 0; u < KU; ++u) {
        kr[u] = *reinterpret_cast<const uint4*>(Kr + tok[u] * kHeadDim);
        vr[u] = *reinterpret_cast<const uint4*>(Vr + tok[u] * kHeadDim);
      }
      float kf[KU][EPL], vf[KU][EPL];
  #pragma unroll
      for (int u = 0; u < KU; ++u) {
        unpack(kr[u], kf[u], TE());
        unpack(vr[u], vf[u], TE());
      }
  #pragma unroll
      for (int h = 0; h < HC; ++h) {
        float z[KU];
  #pragma unroll
        for (int u = 0; u < KU; ++u) {
          float d = 0.f;
  #pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qv[h][e], kf[u][e], d);
          d = group_sum<TE, NT>(d);
          z[u] = ok[u] ? d : -INFINITY;
        }
        float mx = m[h];
  #pragma unroll
        for (int u = 0; u < KU; ++u) mx = fmaxf(mx, z[u]);
        if (mx == -INFINITY) continue;   // uniform across the lane group
        const float alpha = __expf(m[h] - mx);
        float p[KU], psum = 0.f;
  #pragma unroll
        for (int u = 0; u < KU; ++u) {
          p[u] = __expf(z[u] - mx);
          psum += p[u];
        }
        l[h] = l[h] * alpha + psum;
  #pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float a = acc[h][e] * alpha;
  #pragma unroll
          for (int u = 0; u < KU; ++u) a = fmaf(p[u], vf[u][e], a);
          acc[h][e] = a;
        }
        m[h] = mx;
      }
    }

    DS_STAMP(selattn, 12);   // wavefront 0's gather
    // Merge the lane groups of each wavefront (pairwise lane swaps); the
    // wavefronts' states then go through LDS.
    if constexpr (LPT == 16) merge_pairs<16, HC, EPL>(m, l, acc);
    merge_pairs<32, HC, EPL>(m, l, acc);
    if (grp == 0) {
  #pragma unroll
      for (int h = 0; h < HC; ++h) {
        if (sub == 0) {
          sm.wm[wave][h] = m[h];
          sm.wl[wave][h] = l[h];
        }
  #pragma unroll
        for (int e = 0; e < EPL; ++e) sm.u.a.wacc[wave][h][sub * EPL + e] = acc[h][e];
      }
    }
  }
  __syncthreads();
  // Each wavefront's weight in the combined state, once per head: lane
  // 16 (h % 4) + w of wavefront h / 4 (one 16-lane row per head).  Then every
  // output channel sums the weighted wavefront states (independent LDS reads).
  static_assert(NW == 16, "one 16-lane row per head");
  if (wave < (HC + 3) / 4) {
    const int hh = wave * 4 + lane / 16, w = lane % 16;
    const bool in = hh < HC;
    const int h = in ? hh : 0;
    const float mw = in ? sm.wm[w][h] : -INFINITY;
    const float M = row16_max(mw);
    const float f = M == -INFINITY ? 0.f : __expf(mw - M);   // empty wavefronts: 0
    const float Ls = row16_sum(in ? sm.wl[w][h] * f : 0.f);
    if (in) {
      sm.wf[h][w] = f;
      if (w == 0) {
        sm.hm[h] = M;
        sm.hl[h] = Ls;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < HC * kHeadDim; i += NT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    float A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) A = fmaf(sm.u.a.wacc[w][h][c], sm.wf[h][w], A);
    const float M = sm.hm[h], Ls = sm.hl[h];
    const int64_t bh = bh0 + h;
    if (n_split == 1) {
      a.out[bh * kHeadDim + c] = Ls > 0.f ? A / Ls : 0.f;   // nothing kept (threshold rule): zero
    } else {
      __hip_atomic_store(&a.part_acc[(bh * n_split + split) * kHeadDim + c], A, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) {
        __hip_atomic_store(&a.part_ml[(bh * n_split + split) * 2 + 0], M, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.part_ml[(bh * n_split + split) * 2 + 1], Ls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  DS_STAMP(selattn, 13);   // output or split state stored
  if (n_split == 1) {
    DS_STAMP_END(selattn);
    return;
  }

  // The row's last workgroup merges the splits.
  __builtin_amdgcn_s_waitcnt(0);   // this thread's state stores have completed
  __syncthreads();
  unsigned* ticket = a.tickets + rc;
  if (tid == 0) sm.ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  DS_STAMP(selattn, 14);   // ticket
  if (sm.ticket != unsigned(n_split - 1)) {
    DS_STAMP_END(selattn);
    return;
  }
  constexpr int kBatch = 8;   // splits whose states are requested together
  for (int i = tid; i < HC * kHeadDim; i += NT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    const int64_t bh = bh0 + h;
    const float* ml = a.part_ml + bh * n_split * 2;
    const float* pa = a.part_acc + bh * n_split * kHeadDim + c;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += kBatch) {
      float mb[kBatch], lb[kBatch], ab[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {   // unconditional loads (index clamped), then masked
        const bool in = s0 + u < n_split;
        const int sp = in ? s0 + u : 0;
        mb[u] = __hip_atomic_load(&ml[2 * sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lb[u] = __hip_atomic_load(&ml[2 * sp + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ab[u] = __hip_atomic_load(&pa[int64_t(sp) * kHeadDim], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!in) {
          mb[u] = -INFINITY;
          lb[u] = 0.f;
          ab[u] = 0.f;
        }
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, mb[u]);
      if (Mb == -INFINITY) continue;   // only empty splits so far
      const float f = __expf(M - Mb);  // M = -inf gives 0
      L *= f;
      A *= f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float e = __expf(mb[u] - Mb);   // an empty split has m = -inf: 0
        L = fmaf(lb[u], e, L);
        A = fmaf(ab[u], e, A);
      }
      M = Mb;
    }
    a.out[bh * kHeadDim + c] = L > 0.f ? A / L : 0.f;   // nothing kept (threshold rule): zero
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  DS_STAMP(selattn, 15);   // splits merged
  DS_STAMP_END(selattn);
}

template <typename TE, int NT, int ITEMS, int HC, bool RAGGED, int LNV>
hipError_t launch_kernel(const FusedArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((selattn_kernel<TE, NT, ITEMS, HC, RAGGED, LNV>), grid, dim3(NT), 0, s, a.q, a.scores,
                     a.tile_hist, a.ld, a.G, a.head_chunks, a.xcd_rows, a.n_units, a.tiles, a.k_units, a.lb, a.K, a.V,
                     a.indices, a.part_acc, a.part_ml, a.out, a.tickets, a.T_cap, a.T, a.kv_virtual, a.chunk,
                     a.n_split, a.scale, a.seq_lens, a.Hkv, a.tau, a.counts, a.unit_ids, a.label, a.ch, a.r,
                     a.t_append, a.n_append);
  return hipGetLastError();
}

// One pass when a label cache is given: LNV 16-byte words per label row (1 or
// 2; 4 for fp32).
template <typename TE, int NT, int ITEMS, int HC>
hipError_t launch_one(const FusedArgs& a, dim3 grid, hipStream_t s) {
  const int lnv = a.label == nullptr ? 0 : a.r * int(sizeof(TE)) / 16;
  if (a.seq_lens != nullptr) {
    if (lnv == 1) return launch_kernel<TE, NT, ITEMS, HC, true, 1>(a, grid, s);
    if (lnv == 2) return launch_kernel<TE, NT, ITEMS, HC, true, 2>(a, grid, s);
    if constexpr (sizeof(TE) == 4)   // 64-byte rows (fp32, r = 16); in bf16 (r = 32) the kernel would spill
      if (lnv == 4) return launch_kernel<TE, NT, ITEMS, HC, true, 4>(a, grid, s);
    return launch_kernel<TE, NT, ITEMS, HC, true, 0>(a, grid, s);
  }
  if (lnv == 1) return launch_kernel<TE, NT, ITEMS, HC, false, 1>(a, grid, s);
  if (lnv == 2) return launch_kernel<TE, NT, ITEMS, HC, false, 2>(a, grid, s);
  if constexpr (sizeof(TE) == 4)
    if (lnv == 4) return launch_kernel<TE, NT, ITEMS, HC, false, 4>(a, grid, s);
  return launch_kernel<TE, NT, ITEMS, HC, false, 0>(a, grid, s);
}

template <typename TE, int HC>
hipError_t dispatch_items(const FusedArgs& a, dim3 grid, hipStream_t s) {
  const int n = a.n_units;
  if (n <= 1024 * 4) return launch_one<TE, 1024, 4, HC>(a, grid, s);
  if (n <= 1024 * 8) return launch_one<TE, 1024, 8, HC>(a, grid, s);
  if (n <= 1024 * 16) return launch_one<TE, 1024, 16, HC>(a, grid, s);
  return launch_one<TE, 1024, 32, HC>(a, grid, s);
}

// Eight heads per workgroup: only the long rows of the two-stage selection
// (never ragged, one pass or the threshold rule).
template <typename TE>
hipError_t dispatch_wide(const FusedArgs& a, dim3 grid, hipStream_t s) {
  if (a.seq_lens != nullptr || a.label != nullptr || a.counts != nullptr) return hipErrorInvalidValue;
  const int n = a.n_units;
  if (n <= 1024 * 4) return launch_kernel<TE, 1024, 4, 8, false, 0>(a, grid, s);
  if (n <= 1024 * 8) return launch_kernel<TE, 1024, 8, 8, false, 0>(a, grid, s);
  if (n <= 1024 * 16) return launch_kernel<TE, 1024, 16, 8, false, 0>(a, grid, s);
  return launch_kernel<TE, 1024, 32, 8, false, 0>(a, grid, s);
}

template <typename TE>
hipError_t dispatch(const FusedArgs& a, int head_chunk, dim3 grid, hipStream_t s) {
  switch (head_chunk) {
    case 8: return dispatch_wide<TE>(a, grid, s);
    case 4: return dispatch_items<TE, 4>(a, grid, s);
    case 2: return dispatch_items<TE, 2>(a, grid, s);
    default: return dispatch_items<TE, 1>(a, grid, s);
  }
}

}  // namespace

hipError_t launch_select_attention(const void* q, const void* K, const void* V, int is_bf16, const float* scores,
                                   int64_t ld, const uint16_t* tile_hist, int Hq, int Hkv, int64_t T_cap, int64_t T,
                                   int block, int64_t k_units, float scale, const DecodePlan& pl, int32_t* indices,
                                   float* part_acc, float* part_ml, float* out, unsigned* tickets,
                                   const int32_t* seq_lens, float tau, int32_t* counts,
                                   const int32_t* unit_ids, hipStream_t s, const OnePass* one) {
  FusedArgs a{};
  if (one != nullptr) {
    a.label = one->label;
    a.ch = one->ch;
    a.r = one->r;
    a.t_append = int32_t(one->t_append);
    a.n_append = one->n_append;
  }
  a.unit_ids = unit_ids;
  a.seq_lens = seq_lens;
  a.tau = tau;
  a.counts = counts;
  a.Hkv = Hkv;
  a.q = q;
  a.K = K;
  a.V = V;
  a.scores = scores;
  a.tile_hist = tile_hist;
  a.indices = indices;
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  a.out = out;
  a.tickets = tickets;
  a.ld = ld;
  a.T_cap = T_cap;
  a.T = int32_t(T);
  a.n_units = int32_t(pl.n_units);
  a.k_units = int32_t(k_units);
  a.G = Hq / Hkv;
  a.head_chunks = pl.sp.head_chunks;
  a.tiles = int32_t(pl.tiles);
  a.lb = __builtin_ctz(unsigned(block));
  a.kv_virtual = int32_t(pl.kv_virtual);
  a.chunk = int32_t(pl.sp.chunk);
  a.n_split = pl.sp.n_split;
  a.scale = scale;
  // XCD-grouped layout when the rows come in eights and fit the grid limits,
  // else (rows * head_chunks, n_split, 1).
  const unsigned n_rc = unsigned(pl.rows * pl.sp.head_chunks);
  const bool grouped = pl.rows % kXcds == 0 && n_rc / kXcds <= 65535u;
  a.xcd_rows = grouped ? 1 : 0;
  const dim3 grid = grouped ? dim3(unsigned(kXcds), unsigned(pl.sp.n_split), n_rc / kXcds)
                            : dim3(n_rc, unsigned(pl.sp.n_split), 1u);
  if (is_bf16) return dispatch<uint16_t>(a, pl.sp.head_chunk, grid, s);
  return dispatch<float>(a, pl.sp.head_chunk, grid, s);
}

}  // namespace ds
