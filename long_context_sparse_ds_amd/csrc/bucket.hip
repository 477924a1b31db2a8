// Selection and sparse attention of token-level rows from the score kernel's
// sorted tile lists.
//
// Double Sparsity page, method details and abstract: keep the tokens with the
// highest approximate scores, then compute self-attention over those tokens
// only.  Jenga page, core method item 3: the kept K/V rows are read in place.
//
// The score kernel has written, for every tile of 2048 tokens of a row, its
// tokens in descending order of the top 11 bits of their score keys (one
// 32-bit word each: key bits 20..0 above the 11-bit tile-local id) and the
// tile's exclusive descending prefix P[b] (tokens whose top digit exceeds b).
// One workgroup per (row, head chunk, split):
//  A. One round of loads: every tile's prefix word of thread t's two digits
//     (2047 - 2t, 2046 - 2t), summed into the row's cumulative counts R[b]
//     (tokens whose top digit exceeds b), and the head of every tile's list
//     (its first 2048 / tiles entries, two per thread), where the tokens that
//     matter almost always are.
//  B. d0, the digit holding the k-th largest key, is the one digit with
//     R[d0] < k <= R[d0 - 1]: each thread tests its two digits (no scan).  A
//     = R[d0] tokens lie above it, R[d0 - 1] - R[d0] in it.  One wavefront
//     then forms each tile's slices: [0, above_i) of its list above d0, the
//     next in_i in d0.
//  C. Each thread sorts out its two prefetched entries: a token above d0
//     (kept for certain) goes into an LDS map of the row's kept tokens, one
//     bit per token; a candidate in d0 stays in registers with its full key
//     (digit d0 and the stored low bits).  Entries past the prefetched heads
//     (rare) are read in extra rounds.
//  D. 11-bit then 10-bit radix passes over the candidates (histogram atomics
//     by all threads, each digit found by one wavefront's lane scans) give the
//     exact threshold key and how many keys equal to it are kept; equal keys
//     are kept lowest token id first.  The kept candidates join the map.  One
//     prefix sum over the map's words gives every kept token its position in
//     the ascending list.  Split s takes positions [s chunk, (s + 1) chunk):
//     it writes those indices and gathers those rows in ascending order, so
//     the result does not depend on the order of the tiles' lists within a
//     digit (which the score kernel's atomics leave arbitrary).
//  E. Online softmax over the split's rows per query head; the splits' states
//     are merged by log-sum-exp in the row's last-arriving workgroup.
// No workgroup reads the row's full score list: a split reads the tiles'
// prefixes and the heads of their lists (12 KB on the 16K-token shape, in one
// round of loads), against the whole row's scores and histograms (96 KB) in
// the fused kernel of selattn.hip.
//
// Merge ordering.  The split states are written with agent-scope atomic stores
// and read by the merging workgroup with agent-scope atomic loads: on gfx950
// these are global stores and loads with the sc1 bit, which write through the
// XCD's L2 to memory and miss in the reader's L2, so every access goes to the
// memory-side point of coherence shared by all XCDs.  Each wavefront then
// waits for its stores to complete (s_waitcnt vmcnt(0)) before the workgroup
// barrier, and only after that barrier does one thread take the row's ticket
// with an agent-scope atomic, which is performed at the same point of
// coherence.  So a workgroup that draws the last ticket reads states that all
// completed before their tickets were taken.  These are the steps the
// compiler emits for an agent-scope release and acquire, minus the L2
// writeback and invalidate (buffer_wbl2, buffer_inv) that only cached data
// needs; an acquire-release ticket with plain stores and loads measured about
// 3 us slower per step on the 16K-token, 32-head shape.
#include "fused_dev.h"

DS_STAMP_BUFFER(bucket)

namespace ds {
namespace {

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;
constexpr int kTileU = int(kScoreTile);     // tokens per tile
constexpr int kMaxTiles = int(kMaxHistTiles);
constexpr int kSelCap = int(kFusedMaxChunk) + 64;

template <int HC>
struct BucketSmem {
  uint32_t h1[2048];             // candidates: bits 20..10
  uint32_t h2[1024];             // candidates: bits 9..0
  uint32_t map[1024];            // the row's kept tokens, one bit each (32768 tokens)
  uint32_t eq[1024];             // ties at the threshold: map of the tied candidates
  uint32_t eqpre[1024];          // ties: tied candidates before each map word
  uint32_t wsum[kNW];
  uint32_t info[4];              // a digit, the count above it, its count
  uint32_t seam_lo[kNW], seam_hi[kNW];   // R[b_lo] of each wavefront's lane 63, R[b_hi] of its lane 0
  union {
    uint32_t pw[kMaxTiles][1024];   // the tiles' prefix words, until the tiles' slices are known
    struct {
      int32_t sel[kSelCap];         // this split's kept token ids, ascending
      float wacc[kNW][HC][kHeadDim];   // per-wavefront attention states
    } a;
  } u;
  float wm[kNW][HC], wl[kNW][HC];
  __align__(16) float wf[HC][kNW];   // each wavefront's weight in the combined state, per head
  float hm[HC], hl[HC];              // the combined maximum and denominator, per head
  unsigned ticket;
};

// Within one wavefront, with no barrier: the digit of an LDS histogram of nb
// bins (2048 or 1024) holding the kk-th largest key.  Lane l sums the nb / 64
// bins below nb - l nb / 64 (highest first); a lane scan finds the lane whose
// bins hold the kk-th key; that lane's bins are spread over the lanes and
// scanned again.  Every lane receives the digit, the count above it and its
// count.  (Lanes are clamped so that an inconsistent histogram cannot send an
// access out of range.)
__device__ __forceinline__ void wave_pick(const uint32_t* hist, int nb, uint32_t kk, uint32_t& digit,
                                          uint32_t& above, uint32_t& count) {
  const int lane = threadIdx.x & 63;
  const int per = nb >> 6;                                   // 32 or 16
  const uint4* hv = reinterpret_cast<const uint4*>(hist + (nb - (lane + 1) * per));
  uint32_t sum = 0u;
  for (int i = 0; i < per / 4; ++i) {
    const uint4 v = hv[(i + lane) & (per / 4 - 1)];        // lane-rotated: fewer bank conflicts
    sum += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_inclusive_scan(sum);
  const int L = min(max(first_lane_reaching(incl, kk), 0), 63);
  const uint32_t above_L = uint32_t(__builtin_amdgcn_readlane(int(incl - sum), L));
  const int topL = nb - 1 - L * per;
  const uint32_t c = lane < per ? hist[topL - lane] : 0u;
  const uint32_t incl2 = wave_inclusive_scan(c) + above_L;
  const int J = min(max(first_lane_reaching(incl2, kk), 0), per - 1);
  digit = uint32_t(topL - J);
  above = uint32_t(__builtin_amdgcn_readlane(int(incl2 - c), J));
  count = uint32_t(__builtin_amdgcn_readlane(int(c), J));
}

// The tile holding position p of a concatenation whose tile offsets are
// pre[0 .. tiles] (pre[0] = 0, non-decreasing), and that tile's offset: the
// last tile whose offset is <= p (selects over registers, no indexing).
template <int MT>
__device__ __forceinline__ int tile_of(const uint32_t (&pre)[MT + 1], int tiles, uint32_t p, uint32_t& off) {
  int t = 0;
  off = 0u;
#pragma unroll
  for (int i = 1; i < MT; ++i) {
    const bool ge = i < tiles && pre[i] <= p;
    t = ge ? i : t;
    off = ge ? pre[i] : off;
  }
  return t;
}

// Scalar arguments, those of the first loads first (the first dwords are
// preloaded into SGPRs at wave launch).  MT: tiles per row, at most (8 or 16).
template <typename TE, int HC, int MT>
__global__ __launch_bounds__(kNT) void bucket_attn_kernel(
    const void* q_, const uint16_t* tprefix_, int32_t tiles_, int32_t xcd_rows_, int32_t head_chunks_, int32_t G_,
    int32_t n_units_, int32_t k_units_, int32_t n_split_, int32_t chunk_, const uint32_t* slist_, int64_t ld_, const void* K_, const void* V_, int64_t T_cap_, float scale_, int32_t* indices_, float* part_acc_,
    float* part_ml_, float* out_, unsigned* tickets_) {
  using LN = Lanes<TE, kNT>;
  constexpr int EPL = LN::EPL, LPT = LN::LPT, GPW = LN::GPW, NG = LN::NG, KU = LN::KU;
  __shared__ BucketSmem<HC> sm;
  DS_STAMP_START(bucket);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPT, sub = lane % LPT;
  const int gid = wave * GPW + grp;
  const int tiles = tiles_, n_split = n_split_, n_units = n_units_;
  const uint32_t split = blockIdx.y;
  const uint32_t hcs = uint32_t(head_chunks_);
  uint32_t row, hchunk;
  if (xcd_rows_) {
    const uint32_t zr = hcs == 1 ? blockIdx.z : blockIdx.z / hcs;
    row = zr * kXcds + blockIdx.x;
    hchunk = blockIdx.z - zr * hcs;
  } else {
    row = hcs == 1 ? blockIdx.x : blockIdx.x / hcs;
    hchunk = blockIdx.x - row * hcs;
  }
  const uint32_t rc = row * hcs + hchunk;
  const int64_t bh0 = int64_t(row) * G_ + int64_t(hchunk) * HC;   // first (b, h) of this chunk
  const TE* __restrict__ q = static_cast<const TE*>(q_);
  const uint32_t k = uint32_t(k_units_);
  const auto tile_count = [&](int t) -> uint32_t { return uint32_t(min(kTileU, n_units - t * kTileU)); };

  // A. Loads first: q (used only by the attention) and the tiles' prefix words,
  // unconditionally (tile index clamped; a load inside a branch is waited for
  // at once).  Thread t owns digits b_hi = 2047 - 2t and b_lo = 2046 - 2t: word
  // 1023 - t of a tile holds P[b_lo] (low half) and P[b_hi].
  uint4 qraw[HC];
#pragma unroll
  for (int h = 0; h < HC; ++h) qraw[h] = *reinterpret_cast<const uint4*>(q + (bh0 + h) * kHeadDim + sub * EPL);
  const uint32_t* tp = reinterpret_cast<const uint32_t*>(tprefix_ + int64_t(row) * tiles * kHistBins);
  uint32_t w0[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) w0[t] = tp[min(t, tiles - 1) * (kHistBins / 2) + (kNT - 1 - tid)];
  // In the same round of loads, the head of every tile's list (its first W
  // entries): the tokens above d0 and the candidates in d0 are almost always
  // among them.  Entry e of the window array is entry e % W of tile e / W.
  constexpr int W = 2 * kNT / MT;
  const int64_t lrow = int64_t(row) * ld_;   // this row's sorted lists
  uint32_t pf[2];
  bool pf_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid + j * kNT, t = e / W, pos = e % W;
    pf_ok[j] = t < tiles && pos < int(tile_count(t));
    pf[j] = slist_[pf_ok[j] ? lrow + t * kTileU + pos : lrow];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) sm.h1[i * kNT + tid] = 0u;
  sm.h2[tid] = 0u;
  sm.map[tid] = 0u;
  uint32_t R_hi = 0u, R_lo = 0u;   // the row's tokens whose top digit exceeds b_hi, b_lo
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const bool in = t < tiles;
    R_hi += in ? w0[t] >> 16 : 0u;
    R_lo += in ? w0[t] & 0xFFFFu : 0u;
    if (in) sm.u.pw[t][kNT - 1 - tid] = w0[t];
  }
  // B. d0: R[d0] < k <= R[d0 - 1] (R[-1] = every unit).  Exactly one digit
  // qualifies (R[2047] = 0 < k <= n_units).  Thread t tests b_hi, and b_lo
  // with the next lane's R[b_hi] (DPP wave_shl:1), before the first barrier;
  // the digit between two wavefronts (lane 63's b_lo) is tested after it by
  // every wavefront, from the two counts its edge lanes leave in LDS.
  {
    constexpr int kDppWaveShl1 = 0x130;
    const uint32_t R_next = uint32_t(__builtin_amdgcn_update_dpp(0, int(R_hi), kDppWaveShl1, 0xF, 0xF, false));
    const uint32_t R_lm1 = tid == kNT - 1 ? uint32_t(n_units) : R_next;
    const uint32_t b_hi = 2047u - 2u * uint32_t(tid);
    if (R_hi < k && R_lo >= k) {
      sm.info[0] = b_hi;
      sm.info[1] = R_hi;
      sm.info[2] = R_lo - R_hi;
    } else if ((lane < 63 || tid == kNT - 1) && R_lo < k && R_lm1 >= k) {
      sm.info[0] = b_hi - 1u;
      sm.info[1] = R_lo;
      sm.info[2] = R_lm1 - R_lo;
    }
    if (lane == 63) sm.seam_lo[wave] = R_lo;
    if (lane == 0) sm.seam_hi[wave] = R_hi;
  }
  __syncthreads();
  DS_STAMP(bucket, 2);   // prefix words and list heads in
  uint32_t d0, A, cnt0;
  {
    // Seam w: b_lo of thread 64 w + 63 (digit 1920 - 128 w), whose R[b_lo - 1]
    // is thread 64 (w + 1)'s R[b_hi].  Otherwise a thread's own test wrote info.
    const bool lv = lane < kNW - 1;
    const uint32_t slo = lv ? sm.seam_lo[lane] : 0u, shi = lv ? sm.seam_hi[lane + 1] : 0u;
    const uint64_t hit = __ballot(lv && slo < k && shi >= k);
    if (hit != 0u) {
      const int w = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(slo), w));
      const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(shi), w));
      d0 = 1920u - 128u * uint32_t(w);
      A = lo;
      cnt0 = hi - lo;
    } else {
      d0 = sm.info[0];
      A = sm.info[1];
      cnt0 = sm.info[2];
    }
  }
  DS_STAMP(bucket, 3);   // d0
  // (Counts are bounded by the row's units, and d0 by the digit range, so that
  // lists inconsistent with their prefixes cannot send a loop or an access out
  // of range.)
  d0 &= 2047u;
  A = min(A, k);
  cnt0 = min(cnt0, uint32_t(n_units));
  // Tokens of tile t above d0 (the head of its list), from its prefix words.
  const auto above_of = [&](int t) -> uint32_t {
    return min((sm.u.pw[t][d0 >> 1] >> ((d0 & 1u) * 16)) & 0xFFFFu, tile_count(t));
  };
  // Every wavefront forms the tiles' slices itself (lane i: tile i), so no
  // barrier is needed before the classification.
  uint32_t above = 0u, in = 0u;
  if (lane < tiles) {
    above = above_of(lane);
    const uint32_t pm1 = d0 == 0u ? tile_count(lane) : (sm.u.pw[lane][(d0 - 1u) >> 1] >> (((d0 - 1u) & 1u) * 16)) & 0xFFFFu;
    in = min(pm1 - min(pm1, above), tile_count(lane) - above);
  }
  // Past the window (rare): tokens above d0 at [W, above), candidates at [ci0, above + in).
  const uint32_t cr = above > uint32_t(W) ? above - uint32_t(W) : 0u;
  const uint32_t ci0_l = max(above, uint32_t(W));
  const uint32_t ci = above + in > ci0_l ? above + in - ci0_l : 0u;
  const uint32_t ir = wave_inclusive_scan(cr), ic = wave_inclusive_scan(ci);
  uint32_t pr[MT + 1], pc[MT + 1];   // exclusive offsets; lanes past the tiles hold the totals
#pragma unroll
  for (int i = 0; i <= MT; ++i) {
    pr[i] = uint32_t(__builtin_amdgcn_readlane(int(ir - cr), i));
    pc[i] = uint32_t(__builtin_amdgcn_readlane(int(ic - ci), i));
  }
  DS_STAMP(bucket, 4);   // the tiles' slices
  // A tile-local id read from a list, as a token of tile t (masked into the tile).
  const auto token_of = [&](int t, uint32_t id) -> int { return t * kTileU + int(min(id, tile_count(t) - 1u)); };
  const auto mark = [&](uint32_t* m, int tok) { atomicOr(&m[uint32_t(tok) >> 5], 1u << (tok & 31)); };

  // C. The prefetched entries: tokens above d0 into the map, candidates (in d0)
  // kept in registers with their key, counted into the first pass's histogram.
  // An entry's tile is the same for the whole wavefront (W >= 64).
  uint32_t ck[2];
  int ct[2];
  bool cv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid + j * kNT;
    const int t = __builtin_amdgcn_readfirstlane(min((wave * 64 + j * kNT) / W, tiles - 1));
    const uint32_t pos = uint32_t(e % W);
    const uint32_t ab = uint32_t(__builtin_amdgcn_readlane(int(above), t));
    const uint32_t in_t = uint32_t(__builtin_amdgcn_readlane(int(in), t));
    const int tok = token_of(t, pf[j] & 2047u);
    ck[j] = (d0 << 21) | (pf[j] >> 11);
    ct[j] = tok;
    cv[j] = pf_ok[j] && pos >= ab && pos < ab + in_t;
    if (pf_ok[j] && pos < ab) mark(sm.map, tok);
    if (cv[j]) atomicAdd(&sm.h1[(ck[j] >> 10) & 2047u], 1u);
  }
  // Entries past the window, if any (rare): loops with no iteration otherwise.
  const uint32_t n_cr = pr[MT] , n_ci = pc[MT];   // (entries MT hold the totals)
  const auto cand_load = [&](uint32_t c, uint32_t& key, int& tok) {
    uint32_t off;
    const int t = tile_of<MT>(pc, tiles, c, off);
    const uint32_t ci0 = max(above_of(t), uint32_t(W));
    const uint32_t e = slist_[lrow + int64_t(t) * kTileU + min(ci0 + (c - off), tile_count(t) - 1u)];
    key = (d0 << 21) | (e >> 11);
    tok = token_of(t, e & 2047u);
  };
  for (uint32_t p = uint32_t(tid); p < n_cr; p += kNT) {
    uint32_t off;
    const int t = tile_of<MT>(pr, tiles, p, off);
    mark(sm.map, token_of(t, slist_[lrow + t * kTileU + min(uint32_t(W) + (p - off), tile_count(t) - 1u)] & 2047u));
  }
  for (uint32_t c = uint32_t(tid); c < n_ci; c += kNT) {
    uint32_t key;
    int tok;
    cand_load(c, key, tok);
    atomicAdd(&sm.h1[(key >> 10) & 2047u], 1u);
  }
  // f(key, token) over this thread's candidates (those past the window read again).
  const auto for_cands = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (cv[j]) f(ck[j], ct[j]);
    for (uint32_t c = uint32_t(tid); c < n_ci; c += kNT) {
      uint32_t key;
      int tok;
      cand_load(c, key, tok);
      f(key, tok);
    }
  };
  __syncthreads();
  DS_STAMP(bucket, 5);   // candidates classified

  // D. Narrow the threshold inside d0: thr is a key, eq_take the number of keys
  // equal to thr to keep (lowest token ids first), all_eq when that is all of them.
  uint32_t kk = k - A;   // keys still needed from digit d0
  uint32_t thr = d0 << 21, eq_take = 0u;
  bool all_eq = true;
  if (kk != cnt0) {   // uniform
    if (wave == 0) {
      uint32_t dg, ab, cn;
      wave_pick(sm.h1, 2048, kk, dg, ab, cn);
      if (lane == 0) {
        sm.info[0] = dg;
        sm.info[1] = ab;
        sm.info[2] = cn;
      }
    }
    __syncthreads();
    thr |= sm.info[0] << 10;
    kk -= sm.info[1];
    if (kk != sm.info[2]) {
      for_cands([&](uint32_t key, int) {
        if ((key & 0xFFFFFC00u) == thr) atomicAdd(&sm.h2[key & 1023u], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        uint32_t dg, ab, cn;
        wave_pick(sm.h2, 1024, kk, dg, ab, cn);
        if (lane == 0) {
          sm.info[0] = dg;
          sm.info[1] = ab;
          sm.info[2] = cn;
        }
      }
      __syncthreads();
      thr |= sm.info[0];
      kk -= sm.info[1];
      all_eq = kk == sm.info[2];
      eq_take = kk;
    }
  }
  if (!all_eq) {   // uniform: rank the candidates whose key equals thr by token id
    sm.eq[tid] = 0u;
    __syncthreads();
    for_cands([&](uint32_t key, int tok) {
      if (key == thr) mark(sm.eq, tok);
    });
    __syncthreads();
    uint32_t tot;
    sm.eqpre[tid] = block_exclusive_scan1<kNT>(uint32_t(__popc(sm.eq[tid])), sm.wsum, tot);
    __syncthreads();
  }
  // The kept candidates join the map.
  for_cands([&](uint32_t key, int tok) {
    bool keep = key > thr;
    if (key == thr) {
      const uint32_t w = uint32_t(tok) >> 5;
      keep = all_eq || sm.eqpre[w] + uint32_t(__popc(sm.eq[w] & ((1u << (tok & 31)) - 1u))) < eq_take;
    }
    if (keep) mark(sm.map, tok);
  });
  __syncthreads();
  DS_STAMP(bucket, 6);   // radix passes and join

  // Ascending positions: thread w holds map word w.  Split s takes positions
  // [p0, p1): it writes those indices (one head chunk does) and keeps their tokens.
  const uint32_t word = sm.map[tid];
  const uint32_t cnt = uint32_t(__popc(word));
  uint32_t total;
  uint32_t pos = block_exclusive_scan1<kNT>(cnt, sm.wsum, total);   // total = k
  const uint32_t p0 = split * uint32_t(chunk_), p1 = min(p0 + uint32_t(chunk_), k);
  const int n_sel = p0 < p1 ? int(p1 - p0) : 0;
  DS_STAMP(bucket, 7);   // position scan
  if (pos < p1 && pos + cnt > p0) {
    for (uint32_t w = word; w != 0u; w &= w - 1u, ++pos) {
      if (pos < p0 || pos >= p1) continue;
      sm.u.a.sel[pos - p0] = tid * 32 + __builtin_ctz(w);
    }
  }
  __syncthreads();
  DS_STAMP(bucket, 8);   // the split's kept list in LDS
  // The split's slice of the indices, from the list (coalesced), after the
  // barrier: a barrier waits for the workgroup's outstanding global stores.
  if (hchunk == 0) {
    int32_t* ridx = indices_ + int64_t(row) * k_units_ + p0;
    for (int i = tid; i < n_sel; i += kNT) ridx[i] = sm.u.a.sel[i];
  }

  // E. Attention over the split's kept rows.
  const TE* __restrict__ K = static_cast<const TE*>(K_);
  const TE* __restrict__ V = static_cast<const TE*>(V_);
  float qv[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    unpack(qraw[h], qv[h], TE());
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[h][e] *= scale_;
  }
  float m[HC], l[HC], acc[HC][EPL];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const TE* Kr = K + int64_t(row) * T_cap_ * kHeadDim + sub * EPL;
  const TE* Vr = V + int64_t(row) * T_cap_ * kHeadDim + sub * EPL;
  for (int base = 0; base < n_sel; base += NG * KU) {
    // Unconditional loads: a slot past the split's rows reads token 0 of the
    // row (which exists) and is masked out of the softmax.
    int64_t tok[KU];
    bool ok[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int p = base + gid * KU + u;
      ok[u] = p < n_sel;
      tok[u] = ok[u] ? min(max(sm.u.a.sel[p], 0), n_units - 1) : 0;
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
        d = group_sum<TE, kNT>(d);
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

  // Lane groups of each wavefront (pairwise lane swaps); the wavefronts'
  // states then go through LDS.
  if constexpr (LPT == 16) merge_pairs<16, HC, EPL>(m, l, acc);
  merge_pairs<32, HC, EPL>(m, l, acc);
  DS_STAMP(bucket, 9);   // wavefront 0's gather and lane-group merge
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
  __syncthreads();
  DS_STAMP(bucket, 10);   // every wavefront's state in LDS
  // Each wavefront's weight in the combined state, once per head: lane
  // 16 (h % 4) + w of wavefront h / 4 (one 16-lane row per head).  Then every
  // output channel sums the weighted wavefront states (independent LDS reads);
  // the same arithmetic as the fused kernel's, so both give equal outputs.
  static_assert(kNW == 16, "one 16-lane row per head");
  // The state (Acc, M, Ls) of output channel c of head h, and where it goes.
  const auto emit = [&](int h, int c, float Acc, float M, float Ls) {
    const int64_t bh = bh0 + h;
    if (n_split == 1) {
      out_[bh * kHeadDim + c] = Acc / Ls;
    } else {
      __hip_atomic_store(&part_acc_[(bh * n_split + split) * kHeadDim + c], Acc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) {
        __hip_atomic_store(&part_ml_[(bh * n_split + split) * 2 + 0], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&part_ml_[(bh * n_split + split) * 2 + 1], Ls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  if constexpr (HC == 1) {
    // One head: each of the 128 output threads forms the wavefronts' weights
    // exp(m_w - M) and the combined denominator itself (broadcast LDS reads),
    // with no barrier between the weights and the sums.
    if (tid < kHeadDim) {
      float mw[kNW], f[kNW];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        mw[w] = sm.wm[w][0];
        M = fmaxf(M, mw[w]);
      }
      float Ls = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        f[w] = M == -INFINITY ? 0.f : __expf(mw[w] - M);   // empty wavefronts: 0
        Ls = fmaf(sm.wl[w][0], f[w], Ls);
      }
      float Acc = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) Acc = fmaf(sm.u.a.wacc[w][0][tid], f[w], Acc);
      DS_STAMP(bucket, 11);   // combine weights
      emit(0, tid, Acc, M, Ls);
    }
  } else {
    // Each wavefront's weight in the combined state, once per head: lane
    // 16 (h % 4) + w of wavefront h / 4 (one 16-lane row per head).  Then every
    // output channel sums the weighted wavefront states (independent LDS reads);
    // the same arithmetic as the fused kernel's, so both give equal outputs.
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
    DS_STAMP(bucket, 11);   // combine weights
    for (int i = tid; i < HC * kHeadDim; i += kNT) {
      const int h = i / kHeadDim, c = i % kHeadDim;
      float Acc = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) Acc = fmaf(sm.u.a.wacc[w][h][c], sm.wf[h][w], Acc);
      emit(h, c, Acc, sm.hm[h], sm.hl[h]);
    }
  }
  DS_STAMP(bucket, 12);   // output or split state stored
  if (n_split == 1) {
    DS_STAMP_END(bucket);
    return;
  }

  // The row's last workgroup merges the splits (ordering: see the file header).
  __builtin_amdgcn_s_waitcnt(0);   // this wavefront's state stores have completed
  DS_STAMP(bucket, 13);   // the stores completed
  __syncthreads();
  unsigned* ticket = tickets_ + rc;
  if (tid == 0) sm.ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  DS_STAMP(bucket, 14);   // ticket
  if (sm.ticket != unsigned(n_split - 1)) {
    DS_STAMP_END(bucket);
    return;
  }
  constexpr int kBatch = 8;   // splits whose states are requested together
  for (int i = tid; i < HC * kHeadDim; i += kNT) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    const int64_t bh = bh0 + h;
    const float* ml = part_ml_ + bh * n_split * 2;
    const float* pa_ = part_acc_ + bh * n_split * kHeadDim + c;
    float M = -INFINITY, Ls = 0.f, Acc = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += kBatch) {
      float mb[kBatch], lb[kBatch], ab[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {   // unconditional loads (index clamped), then masked
        const bool in = s0 + u < n_split;
        const int sp = in ? s0 + u : 0;
        mb[u] = __hip_atomic_load(&ml[2 * sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lb[u] = __hip_atomic_load(&ml[2 * sp + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ab[u] = __hip_atomic_load(&pa_[int64_t(sp) * kHeadDim], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!in) {
          mb[u] = -INFINITY;
          lb[u] = 0.f;
          ab[u] = 0.f;
        }
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, mb[u]);
      if (Mb == -INFINITY) continue;    // only empty splits so far
      const float f = __expf(M - Mb);   // M = -inf gives 0
      Ls *= f;
      Acc *= f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float e = __expf(mb[u] - Mb);   // a padding slot has m = -inf: 0
        Ls = fmaf(lb[u], e, Ls);
        Acc = fmaf(ab[u], e, Acc);
      }
      M = Mb;
    }
    out_[bh * kHeadDim + c] = Acc / Ls;
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  DS_STAMP(bucket, 15);   // splits merged
  DS_STAMP_END(bucket);
}

template <typename TE, int HC>
hipError_t launch_t(const void* q, const void* K, const void* V, const uint32_t* slist, const uint16_t* tprefix, int Hq, int Hkv, int64_t T_cap, int64_t k_units, float scale,
                    const DecodePlan& pl, int32_t* indices, float* part_acc, float* part_ml, float* out,
                    unsigned* tickets, hipStream_t s) {
  const unsigned n_rc = unsigned(pl.rows * pl.sp.head_chunks);
  const bool grouped = pl.rows % kXcds == 0 && n_rc / kXcds <= 65535u;
  const dim3 grid = grouped ? dim3(unsigned(kXcds), unsigned(pl.sp.n_split), n_rc / kXcds)
                            : dim3(n_rc, unsigned(pl.sp.n_split), 1u);
  const auto kern = pl.tiles <= 8 ? bucket_attn_kernel<TE, HC, 8> : bucket_attn_kernel<TE, HC, kMaxTiles>;
  hipLaunchKernelGGL(kern, grid, dim3(kNT), 0, s, q, tprefix, int32_t(pl.tiles),
                     int32_t(grouped ? 1 : 0), int32_t(pl.sp.head_chunks), int32_t(Hq / Hkv), int32_t(pl.n_units),
                     int32_t(k_units), int32_t(pl.sp.n_split), int32_t(pl.sp.chunk), slist, pl.score_ld, K, V,
                     T_cap, scale, indices, part_acc, part_ml, out, tickets);
  return hipGetLastError();
}

template <typename TE>
hipError_t dispatch(const void* q, const void* K, const void* V, const uint32_t* slist, const uint16_t* tprefix, int Hq, int Hkv, int64_t T_cap, int64_t k_units, float scale,
                    const DecodePlan& pl, int32_t* indices, float* part_acc, float* part_ml, float* out,
                    unsigned* tickets, hipStream_t s) {
  switch (pl.sp.head_chunk) {
    case 4:
      return launch_t<TE, 4>(q, K, V, slist, tprefix, Hq, Hkv, T_cap, k_units, scale, pl, indices, part_acc,
                             part_ml, out, tickets, s);
    case 2:
      return launch_t<TE, 2>(q, K, V, slist, tprefix, Hq, Hkv, T_cap, k_units, scale, pl, indices, part_acc,
                             part_ml, out, tickets, s);
    default:
      return launch_t<TE, 1>(q, K, V, slist, tprefix, Hq, Hkv, T_cap, k_units, scale, pl, indices, part_acc,
                             part_ml, out, tickets, s);
  }
}

}  // namespace

hipError_t launch_bucket_attention(const void* q, const void* K, const void* V, int is_bf16, const uint32_t* slist,
                                   const uint16_t* tprefix, int Hq, int Hkv, int64_t T_cap,
                                   int64_t k_units, float scale, const DecodePlan& pl, int32_t* indices,
                                   float* part_acc, float* part_ml, float* out, unsigned* tickets, hipStream_t s) {
  if (is_bf16)
    return dispatch<uint16_t>(q, K, V, slist, tprefix, Hq, Hkv, T_cap, k_units, scale, pl, indices, part_acc,
                              part_ml, out, tickets, s);
  return dispatch<float>(q, K, V, slist, tprefix, Hq, Hkv, T_cap, k_units, scale, pl, indices, part_acc,
                         part_ml, out, tickets, s);
}

}  // namespace ds
