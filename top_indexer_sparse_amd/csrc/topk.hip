// topk.hip -- per-query Top-K select on gfx950, no full sort.
//
// Selection rule ("Sparse Attention 数学学习笔记" §9; "MLA 与稀疏注意力" DSA
// section, the selected-position helper ordering by (-score, position)):
// exactly min(k, #candidates) candidates; larger scores first; equal scores
// to the lower position.  Candidates are the positions s < lim (kv_len and
// the causal bound q_pos) whose score is neither NaN nor -inf.
//
// Method (one 1024-thread work-group per row):
//  1. Each score becomes an order-preserving 32-bit key (-0 folded onto +0;
//     NaN and -inf become key 0, "not a candidate").  Wave w holds positions
//     [2048 w, 2048 w + 2048) in registers, loaded as 16-byte vectors: lane l,
//     round i, element e is position 2048 w + 4 (l + 64 i) + e.
//  2. tau = the k-th largest key.  Keys are binned by a digit fitted to the
//     row, d = (key - min key) >> sh, with sh chosen so that the key range
//     spans at most 2048 bins (index scores share sign and exponent, so fixed
//     high-bit digits would pile the keys onto a few LDS words).
//     a. A histogram of 1024 sampled keys brackets the rank-k bin with a
//        margin of four standard deviations of the sample rank.
//     b. One pass over all keys counts, without atomics, the keys above and
//        inside the bracket.  If rank k falls outside it, a histogram of all
//        keys names the exact bin instead.
//     c. The bracket's keys are compacted into LDS (block scan) and radix
//        passes of up to 11 bits over them find tau and the number of keys
//        equal to tau that are taken.
//  3. Per-round (greater-than-tau, equal-to-tau) counts, prefix-summed over
//     the block in position order with ballots, give every selected key its
//     output slot and its rank among the ties: keys > tau and the first
//     k - count(> tau) keys == tau are placed in ascending position order in
//     LDS, then written out with coalesced stores.
// Rows longer than 32768 positions are cut into 32768-position chunks; each
// chunk keeps its own top-k (a superset of its share of the row's top-k under
// the same rule), and a second launch selects from the chunks' candidates,
// which are laid out in ascending position order, so the tie rule carries over.
// Launches with few rows of 8192 or more positions (decode) take the split
// path further down instead: 4096-position chunk work-groups around a
// sampled key bracket, then one select work-group per row.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace sa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkSeg = 32;                   // keys per thread
constexpr int kTkRounds = kTkSeg / 4;        // 16-byte loads per thread
constexpr int kTkRow = kTkThreads * kTkSeg;  // 32768 positions per work-group
constexpr int kTkWaveSpan = kTkRow / kTkWaves;
constexpr int kTkBins = 2048;
constexpr int kTkAux = 5120;  // bracket candidates held in LDS (>= kTopkMaxK)

// Inclusive block scan (sum) of one int per thread; `red` holds kTkWaves ints.
// Returns the inclusive prefix; `total` receives the block sum.
__device__ __forceinline__ int block_scan_incl(int x, int* red, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  x = wave_scan_incl(x);
  __syncthreads();  // red may still be read by a previous scan
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int v = red[w];
    before += w < wave ? v : 0;
    total += v;
  }
  return x + before;
}

// Block sum: every thread receives the total.
__device__ __forceinline__ int block_sum(int x, int* red) {
  const int t = wave_total(x);
  __syncthreads();  // red may still be read by a previous reduction
  if (lane_id() == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) total += red[w];
  return total;
}

// Bins of `hist` (2048 bins) holding ranks r0 <= r1 counted from the top.
// Thread t owns bins 2047-2t and 2046-2t.  found[0..1] = (bin of r0, keys in
// higher bins), found[2] = bin of r1, where ranks(total, r0, r1) sets the
// ranks from the histogram's total; a rank outside [1, total] gives bin -1.
// Starts with a barrier (the histogram is complete) and ends with one (found
// is visible).
template <class Ranks>
__device__ __forceinline__ void find_rank_bins(const int* hist, Ranks ranks, int* red,
                                               int* found) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid == 0) {  // a rank beyond the total leaves these: bin -1, above 0
    found[0] = found[2] = -1;
    found[1] = 0;
  }
  const int bhi = kTkBins - 1 - 2 * tid, blo = bhi - 1;
  const int hhi = hist[bhi], hlo = hist[blo];
  int total;
  const int incl = block_scan_incl(hhi + hlo, red, total);
  const int above = incl - hhi - hlo;
  int r0, r1;
  ranks(total, r0, r1);
  if (above < r0 && r0 <= above + hhi) {
    found[0] = bhi;
    found[1] = above;
  } else if (above + hhi < r0 && r0 <= above + hhi + hlo) {
    found[0] = blo;
    found[1] = above + hhi;
  }
  if (above < r1 && r1 <= above + hhi) {
    found[2] = bhi;
  } else if (above + hhi < r1 && r1 <= above + hhi + hlo) {
    found[2] = blo;
  }
  __syncthreads();
}

// hist[d] += 1 for every lane with `valid`.  When all valid lanes of the wave
// share one bin, one lane adds the whole count instead of 64 lanes hitting
// the same LDS word.
__device__ __forceinline__ void hist_add(int* hist, uint32_t d, bool valid) {
  const uint64_t m = __ballot(valid);
  if (m == 0) return;
  const int lead = __ffsll((unsigned long long)m) - 1;
  const uint32_t d0 = __builtin_amdgcn_readlane(d, lead);
  if (__ballot(valid && d == d0) == m) {
    if (lane_id() == lead) atomicAdd(&hist[d0], __popcll(m));
  } else if (valid) {
    atomicAdd(&hist[d], 1);
  }
}

struct TopkRowArgs {
  const float* scores;   // direct rows: scores[bt * L + s]
  const int32_t* q_pos;
  const int32_t* kv_len;
  int T, L, k;
  int nchunks;           // chunks per row of the first launch
  // first launch with nchunks > 1: candidates per (row, chunk)
  float* cand_score;     // [rows][nchunks][k]
  int32_t* cand_pos;
  // final output
  int32_t* idx;          // [rows][k]
  int32_t* count;        // [rows] or null
};

// MERGE = false: virtual row = positions [chunk*kTkRow, ...) of a score row.
// MERGE = true : virtual row = the nchunks*k candidates of a row.
//
// Code size matters here: a work-group runs its row once, usually on a CU
// whose instruction cache is cold, so every 64 bytes of straight-line code
// cost a fetch from L2.  The keys therefore live in LDS, arrive there by
// global->LDS DMA (no registers, no unrolling), and every phase is a short
// loop; all histogram rounds share one rank search.
template <bool MERGE>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkRowArgs a) {
  __shared__ uint4 keys4[kTkRow / 4];  // the row's keys by position
  __shared__ uint32_t aux[kTkAux];     // bracket candidates, then output positions
  __shared__ int hist[kTkBins];
  __shared__ int red[kTkWaves];
  __shared__ uint32_t rmin[kTkWaves], rmax[kTkWaves];
  __shared__ int found[4];
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(keys4);

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bt = blockIdx.y;
  const int chunk = blockIdx.x;
  const int k = a.k;

  // ---- the virtual row ----
  const float* src;
  const int32_t* vpos = nullptr;
  int pos_base = 0, n;
  int32_t* out_idx;
  float* out_score = nullptr;
  int32_t* out_count = nullptr;
  if (!MERGE) {
    const int b = (int)(bt / a.T);
    const int lim = candidate_limit(a.q_pos, a.kv_len, b, bt, a.L);
    pos_base = chunk * kTkRow;
    n = min(max(lim - pos_base, 0), kTkRow);
    src = a.scores + bt * a.L + pos_base;
    if (a.nchunks == 1) {
      out_idx = a.idx + bt * k;
      out_count = a.count ? a.count + bt : nullptr;
    } else {
      const int64_t o = (bt * a.nchunks + chunk) * k;
      out_idx = a.cand_pos + o;
      out_score = a.cand_score + o;
    }
  } else {
    n = a.nchunks * k;
    src = a.cand_score + bt * n;
    vpos = a.cand_pos + bt * n;
    out_idx = a.idx + bt * k;
    out_count = a.count ? a.count + bt : nullptr;
  }

  // ---- scores into LDS by DMA; wave w fills positions [2048 w, 2048 w + 2048)
  const int wbase4 = wave * (kTkWaveSpan / 4);  // in 16-byte units
  const uint32_t lds_keys = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&keys4[0];
  const uint8_t* gsrc = reinterpret_cast<const uint8_t*>(src);
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    for (int i = 0; i < kTkRounds; ++i) {  // 16 bytes per lane, 1 KB per wave
      const int u = wbase4 + 64 * i;
      if (4 * (u + lane) + 3 < n) dma16(gsrc, 16u * (uint32_t)(u + lane), lds_keys + 16u * (uint32_t)u);
    }
    const int n4 = n & ~3;  // the ragged end: up to 3 scores, one dword each
    if (wave == 0 && lane < n - n4) dma4(gsrc, 4u * (uint32_t)(n4 + lane), lds_keys + 4u * (uint32_t)n4);
  } else {
    for (int i = 0; i < 4 * kTkRounds; ++i) {  // 4 bytes per lane
      const int p = 4 * wbase4 + 64 * i;
      if (p + lane < n) dma4(gsrc, 4u * (uint32_t)(p + lane), lds_keys + 4u * (uint32_t)p);
    }
  }
  wait_vmcnt<0>();
  lds_barrier();

  // ---- scores -> keys in place (positions >= n -> 0); count, min, max ----
  int n_valid;
  uint32_t kmin, kmax;
  {
    uint32_t mn = 0xffffffffu, mx = 0u;
    int nv = 0;
#pragma unroll 2
    for (int i = 0; i < kTkRounds; ++i) {
      const int u = wbase4 + lane + 64 * i;
      uint4 q = keys4[u];
      uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[e] = 4 * u + e < n ? score_key(__builtin_bit_cast(float, kk[e])) : 0u;
        nv += kk[e] != 0u;
        mn = kk[e] ? min(mn, kk[e]) : mn;
        mx = max(mx, kk[e]);
      }
      keys4[u] = make_uint4(kk[0], kk[1], kk[2], kk[3]);
    }
    nv = wave_total(nv);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      red[wave] = nv;
      rmin[wave] = mn;
      rmax[wave] = mx;
    }
    __syncthreads();  // also publishes the keys
    n_valid = 0;
    kmin = 0xffffffffu;
    kmax = 0u;
    for (int w = 0; w < kTkWaves; ++w) {
      n_valid += red[w];
      kmin = min(kmin, rmin[w]);
      kmax = max(kmax, rmax[w]);
    }
  }

  // ---- tau = the k-th largest key ----
  uint32_t tau = 0u;   // keys > tau are all selected
  int need_eq = 0;     // how many keys == tau to take (lowest positions)
  if (n_valid > k) {
    const uint32_t range = kmax - kmin;
    const int sh = max(0, 32 - __clz(range) - 11);  // (range >> sh) < 2048
    const float p_sel = (float)k / (float)n_valid;
    enum { kSample, kAll, kCand, kFilter };
    int mode = kSample;
    int krem = k, ncand = 0, top = -1, in_me = 0;
    uint32_t lo_key = 0u, hi_key = 0u, prefix = 0u, pmask = 0u;  // bracket [lo_key, hi_key]
    for (;;) {
      __syncthreads();  // the previous round's bins have been read
      for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0;
      __syncthreads();
      int s2 = 0;
      uint32_t dmask = 0u;
      if (mode == kSample) {
        // one key per lane, spread over the wave's eight rounds
        const uint32_t key = keys[4 * (wbase4 + lane + 64 * (lane & 7)) + ((lane >> 3) & 3)];
        hist_add(hist, (key - kmin) >> sh, key != 0u);
      } else if (mode == kAll) {
        #pragma unroll 1
        for (int i = 0; i < kTkRounds; ++i) {
          const uint4 q = keys4[wbase4 + lane + 64 * i];
          const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) hist_add(hist, (kk[e] - kmin) >> sh, kk[e] != 0u);
        }
      } else {
        const int width = min(11, top + 1);
        s2 = top + 1 - width;
        dmask = (1u << width) - 1u;
        if (mode == kCand) {
    #pragma unroll 1
      for (int j0 = 0; j0 < ncand; j0 += kTkThreads) {
            const int j = j0 + tid;
            const uint32_t c = j < ncand ? aux[j] : 0u;
            hist_add(hist, (c >> s2) & dmask, j < ncand && (c & pmask) == prefix);
          }
        } else {  // kFilter: the bracket outgrew aux; filter the whole row
          #pragma unroll 1
          for (int i = 0; i < kTkRounds; ++i) {
            const uint4 q = keys4[wbase4 + lane + 64 * i];
            const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t c = kk[e] - lo_key;
              const bool in = kk[e] != 0u && kk[e] >= lo_key && kk[e] <= hi_key &&
                              (c & pmask) == prefix;
              hist_add(hist, (c >> s2) & dmask, in);
            }
          }
        }
      }
      find_rank_bins(
          hist,
          [&](int m, int& r0, int& r1) {
            if (mode == kSample) {  // four standard deviations of the sample rank
              const float mean = p_sel * (float)m;
              const float margin = 4.f * sqrtf(mean * (1.f - p_sel)) + 2.f;
              r0 = max(1, (int)floorf(mean - margin));
              r1 = min(m, (int)ceilf(mean + margin));
            } else {
              r0 = r1 = krem;
            }
          },
          red, found);

      if (mode == kSample || mode == kAll) {
        // bins as unsigned: an empty sample gives 0xffffffff, so that nothing
        // is above or inside and the check below falls back to kAll
        uint32_t b_hi = (uint32_t)found[0], b_lo = (uint32_t)found[2];
        int above, inside;
        if (mode == kSample) {
          int ab = 0, in = 0;
          #pragma unroll 1
          for (int i = 0; i < kTkRounds; ++i) {
            const uint4 q = keys4[wbase4 + lane + 64 * i];
            const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t d = (kk[e] - kmin) >> sh;
              ab += kk[e] != 0u && d > b_hi;
              in += kk[e] != 0u && d >= b_lo && d <= b_hi;
            }
          }
          // packed: above < 32768 (bin b_hi holds a sampled key), inside <= 32768
          const int both = block_sum((ab << 16) | in, red);
          above = both >> 16;
          inside = both & 0xffff;
          in_me = in;
          if (!(above < k && k <= above + inside)) {
            mode = kAll;
            continue;
          }
        } else {
          b_hi = b_lo = (uint32_t)found[0];
          above = found[1];
          inside = hist[b_hi];  // the bins are only cleared after a barrier
          in_me = -1;           // not counted per thread
        }
        krem = k - above;
        lo_key = kmin + (b_lo << sh);
        const uint64_t crange = ((uint64_t)(b_hi - b_lo + 1) << sh) - 1u;  // largest offset
        hi_key = (uint32_t)min((uint64_t)0xffffffffu, (uint64_t)lo_key + crange);
        top = crange ? 63 - __clzll((long long)crange) : -1;
        if (top < 0) break;  // the bracket is a single key value
        if (inside > kTkAux) {
          mode = kFilter;
          continue;
        }
        // the bracket's keys, as offsets from lo_key, into aux
        if (in_me < 0) {
          in_me = 0;
          #pragma unroll 1
          for (int i = 0; i < kTkRounds; ++i) {
            const uint4 q = keys4[wbase4 + lane + 64 * i];
            in_me += (q.x != 0u && q.x >= lo_key && q.x <= hi_key) +
                     (q.y != 0u && q.y >= lo_key && q.y <= hi_key) +
                     (q.z != 0u && q.z >= lo_key && q.z <= hi_key) +
                     (q.w != 0u && q.w >= lo_key && q.w <= hi_key);
          }
        }
        int slot = block_scan_incl(in_me, red, ncand) - in_me;
        #pragma unroll 1
        for (int i = 0; i < kTkRounds && in_me > 0; ++i) {
          const uint4 q = keys4[wbase4 + lane + 64 * i];
          const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kk[e] != 0u && kk[e] >= lo_key && kk[e] <= hi_key) aux[slot++] = kk[e] - lo_key;
        }
        mode = kCand;
        continue;  // the loop head's barrier publishes aux
      }
      // a radix pass over the bracket
      prefix |= (uint32_t)found[0] << s2;
      pmask |= dmask << s2;
      krem -= found[1];
      top = s2 - 1;
      if (top < 0) break;
    }
    tau = lo_key + prefix;
    need_eq = krem;
  }
  const int n_sel = min(k, n_valid);

  // ---- slots in position order ----
  // Per round, lane counts packed as (gt << 16) | eq (each at most 4 per lane,
  // 256 per wave); a DPP scan gives the lanes below and the wave's total.
  int wtot = 0;
  #pragma unroll 1
  for (int i = 0; i < kTkRounds; ++i) {
    const uint4 q = keys4[wbase4 + lane + 64 * i];
    const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += ((kk[e] > tau) << 16) | ((kk[e] == tau) & (kk[e] != 0u));
    wtot += wave_total(c);
  }
  __syncthreads();  // every thread has read red; aux (candidates) is free
  if (lane == 0) red[wave] = wtot;  // gt <= 4096 and eq <= 32768 per row
  __syncthreads();
  int run = 0;  // packed counts of the waves before this one
  for (int w = 0; w < wave; ++w) run += red[w];
  #pragma unroll 1
  for (int i = 0; i < kTkRounds; ++i) {
    const int u = wbase4 + lane + 64 * i;
    const uint4 q = keys4[u];
    const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += ((kk[e] > tau) << 16) | ((kk[e] == tau) & (kk[e] != 0u));
    const int incl = wave_scan_incl(c);
    const int before = run + incl - c;
    run += __builtin_amdgcn_readlane(incl, 63);
    if (c) {
      int gtb = before >> 16, eqb = before & 0xffff;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool g = kk[e] > tau, eq = (kk[e] == tau) & (kk[e] != 0u);
        if (g || (eq && eqb < need_eq)) aux[gtb + min(eqb, need_eq)] = (uint32_t)(4 * u + e);
        gtb += g;
        eqb += eq;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += kTkThreads) {
    if (i < n_sel) {
      const int v = min((int)aux[i], n - 1);  // (a slot is always < n)
      out_idx[i] = vpos ? vpos[v] : pos_base + v;
      if (out_score) out_score[i] = key_score(keys[v]);
    } else {
      out_idx[i] = -1;
      if (out_score) out_score[i] = -INFINITY;
    }
  }
  if (out_count && tid == 0) *out_count = n_sel;
}

// ---------------------------------------------------------------------------
// Split path: few long rows (decode).  One work-group per row leaves most of
// the GPU idle and runs every pass over the row on one CU, so a row is cut
// into 4096-position chunks, one work-group each, in two launches:
//  A. Every chunk's work-group draws the same deterministic sample of its row
//     (128 evenly spaced runs of 16 positions) and from it the same key
//     bracket [lo, hi] around the expected rank of the k-th key (four
//     standard deviations of the sample rank).  It keeps the keys >= lo of
//     its chunk, with their positions, compacted in position order, and
//     counts those above hi, those inside, and the candidates at all.
//  B. One work-group per row checks the bracket against the chunks' counts
//     (above < k <= above + inside).  Radix passes over the inside keys give
//     tau, the k-th largest key; one block scan over the kept keys in
//     position order then places every selected position (keys > tau, and
//     keys == tau up to k, lowest positions first) at its ascending slot.
//     When the bracket misses, the kept keys overflow, or the row has at most
//     k candidates, the same work-group selects straight from the row's
//     scores instead (radix passes over the whole row), so correctness never
//     rests on the sample.
// ---------------------------------------------------------------------------
constexpr int kSpChunk = 4096;
constexpr int kSpThreads = 512;
constexpr int kSpWaves = kSpThreads / 64;
constexpr int kSpPer = kSpChunk / kSpThreads;  // consecutive positions per thread
constexpr int kSpRuns = 128, kSpRun = 16;      // the row sample: 2048 keys
constexpr int kSpSamplePer = kSpRuns * kSpRun / kSpThreads;
constexpr int kSpRunThreads = kSpThreads / kSpRuns;  // threads per sample run
static_assert(kSpRunThreads * kSpSamplePer == kSpRun, "a run is split evenly over threads");
constexpr int kSpBins = 2048;
constexpr int kSpMaxRows = 128;    // rows of a launch taking the split path
constexpr int kSpMinL = 8192;      // shortest row length taking it
constexpr int kSpMaxChunks = 256;  // rows up to 1M positions
constexpr int kSpKeep = 16384;     // kept keys the second launch holds in LDS
constexpr int kSpSelThreads = 512; // threads of a select work-group (one per row)

struct TopkSplitArgs {
  const float* scores;
  const int32_t* q_pos;
  const int32_t* kv_len;
  int T, L, k, nchunk;
  int vec4;            // scores rows are 16-byte aligned (float4 loads)
  int32_t* cnt;        // [rows][nchunk][4]: above, inside, candidates, -
  uint32_t* bracket;   // [rows][nchunk][2]: lo, hi (equal in every chunk)
  uint32_t* keepk;     // [rows][nchunk][kSpChunk]: kept keys (>= lo), position order
  int32_t* keepp;      // [rows][nchunk][kSpChunk]: their positions
  int32_t* idx;        // [rows][k]
  int32_t* count;      // [rows] or null
};

// Exclusive block scan over the NT threads of a split work-group.
template <int NT = kSpThreads>
__device__ __forceinline__ int sp_scan_excl(int x, int* red, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int v = red[w];
    before += w < wave ? v : 0;
    total += v;
  }
  return incl - x + before;
}

// Bins of `hist` (2048 bins) holding ranks r0 <= r1 counted from the top:
// found[0] = bin of r0, found[1] = entries in higher bins, found[2] = bin of
// r1; a rank outside [1, total] gives bin -1.  Thread t owns the BPT =
// 2048 / NT bins 2047 - BPT t downwards.  Starts with a barrier (the
// histogram is complete); `found` is visible when it returns.
template <int NT = kSpThreads>
__device__ __forceinline__ void sp_rank_bins(const int* hist, int r0, int r1, int* red,
                                             int* found) {
  constexpr int BPT = kSpBins / NT;
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid == 0) {
    found[0] = found[2] = -1;
    found[1] = 0;
  }
  int h[BPT], own = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    h[e] = hist[kSpBins - 1 - BPT * tid - e];
    own += h[e];
  }
  int total;
  int above = sp_scan_excl<NT>(own, red, total);
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    if (above < r0 && r0 <= above + h[e]) {
      found[0] = kSpBins - 1 - BPT * tid - e;
      found[1] = above;
    }
    if (above < r1 && r1 <= above + h[e]) found[2] = kSpBins - 1 - BPT * tid - e;
    above += h[e];
  }
  __syncthreads();
}
template <int NT = kSpThreads>
__device__ __forceinline__ void sp_rank_bin(const int* hist, int r, int* red, int* found) {
  sp_rank_bins<NT>(hist, r, r, red, found);
}

template <int NT = kSpThreads>
__device__ __forceinline__ int sp_block_sum(int x, int* red) {
  const int t = wave_total(x);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += red[w];
  return total;
}

// Launch A: one work-group per (chunk, row).
__global__ __launch_bounds__(kSpThreads) void topk_split_scan_kernel(TopkSplitArgs a) {
  __shared__ int hist[kSpBins];
  __shared__ int red[kSpWaves];
  __shared__ uint32_t rmin[kSpWaves], rmax[kSpWaves];
  __shared__ int found[3];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int b = (int)(row / a.T);
  const int lim = candidate_limit(a.q_pos, a.kv_len, b, row, a.L);
  const float* srow = a.scores + row * a.L;
  const int c0 = chunk * kSpChunk;
  const int64_t unit = row * a.nchunk + chunk;
  int32_t* cnt = a.cnt + unit * 4;
  if (c0 >= lim) {  // nothing of the row here
    if (tid == 0) cnt[0] = cnt[1] = cnt[2] = cnt[3] = 0;
    return;
  }
  // this thread's 16 consecutive positions and its 8 sample positions, all
  // loads issued before any is used
  const int p0 = c0 + kSpPer * tid;
  float cs[kSpPer];
  if (a.vec4 && p0 + kSpPer <= lim) {
#pragma unroll
    for (int i = 0; i < kSpPer / 4; ++i) {
      const float4 v = *(const float4*)(srow + p0 + 4 * i);
      cs[4 * i] = v.x;
      cs[4 * i + 1] = v.y;
      cs[4 * i + 2] = v.z;
      cs[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSpPer; ++i) cs[i] = p0 + i < lim ? srow[p0 + i] : -INFINITY;
  }
  // sample: run r = tid / kSpRunThreads starts at r * lim / 128 (every position when the
  // row is shorter than the sample)
  const int sbase = lim >= kSpRuns * kSpRun
                        ? (int)((int64_t)(tid / kSpRunThreads) * lim / kSpRuns) +
                              kSpSamplePer * (tid % kSpRunThreads)
                        : kSpSamplePer * tid;
  float ss[kSpSamplePer];
#pragma unroll
  for (int m = 0; m < kSpSamplePer; ++m) ss[m] = sbase + m < lim ? srow[sbase + m] : -INFINITY;
  const int S = min(lim, kSpRuns * kSpRun);

  // ---- the row's bracket from the sample (identical in every chunk) ----
  uint32_t sk[kSpSamplePer];
  int nv = 0;
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int m = 0; m < kSpSamplePer; ++m) {
    sk[m] = score_key(ss[m]);
    nv += sk[m] != 0u;
    mn = sk[m] ? min(mn, sk[m]) : mn;
    mx = max(mx, sk[m]);
  }
  nv = wave_total(nv);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  for (int i = tid; i < kSpBins; i += kSpThreads) hist[i] = 0;
  if (lane == 0) {
    red[wave] = nv;
    rmin[wave] = mn;
    rmax[wave] = mx;
  }
  __syncthreads();
  int ns = 0;
  uint32_t smin = 0xffffffffu, smax = 0u;
#pragma unroll
  for (int w = 0; w < kSpWaves; ++w) {
    ns += red[w];
    smin = min(smin, rmin[w]);
    smax = max(smax, rmax[w]);
  }
  uint32_t lo = 1u, hi = 0xffffffffu;  // no usable sample: every candidate is inside
  if (ns > 0) {
    const int sh = max(0, 32 - __clz(smax - smin) - 11);  // (range >> sh) < 2048
#pragma unroll
    for (int m = 0; m < kSpSamplePer; ++m) hist_add(hist, (sk[m] - smin) >> sh, sk[m] != 0u);
    // sample ranks, counted from the top, that bracket the row's k-th key
    const float p = fminf(1.f, (float)a.k / (float)lim);
    const float mean = p * (float)S;
    const float margin = 4.f * sqrtf(mean * (1.f - p)) + 2.f;
    const int r0 = min(max(1, (int)floorf(mean - margin)), ns);
    const int r1u = (int)ceilf(mean + margin);
    const int r1 = min(max(r1u, r0), ns);
    sp_rank_bins(hist, r0, r1, red, found);
    const int bhi = found[0], blo = found[2];
    hi = (uint32_t)min((uint64_t)0xffffffffu, (uint64_t)smin + ((uint64_t)(bhi + 1) << sh) - 1u);
    lo = r1u > ns ? 1u : smin + ((uint32_t)blo << sh);
  }

  // ---- this chunk: the keys >= lo, compacted in position order ----
  uint32_t ck[kSpPer];
  int na = 0, nk = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kSpPer; ++i) {
    ck[i] = score_key(cs[i]);
    nc += ck[i] != 0u;
    na += ck[i] > hi;
    nk += ck[i] != 0u && ck[i] >= lo;
  }
  int tot_packed;
  int o = sp_scan_excl((na << 16) | nk, red, tot_packed) & 0xffff;
  const int64_t base = unit * (int64_t)kSpChunk;
#pragma unroll
  for (int i = 0; i < kSpPer; ++i) {
    if (ck[i] != 0u && ck[i] >= lo) {
      a.keepk[base + o] = ck[i];
      a.keepp[base + o] = p0 + i;
      ++o;
    }
  }
  const int nct = sp_block_sum(nc, red);
  if (tid == 0) {
    cnt[0] = tot_packed >> 16;                            // above hi
    cnt[1] = (tot_packed & 0xffff) - (tot_packed >> 16);  // inside [lo, hi]
    cnt[2] = nct;                                         // candidates
    cnt[3] = 0;
    a.bracket[2 * unit] = lo;
    a.bracket[2 * unit + 1] = hi;
  }
}

// Launch B: one NT-thread work-group per row.
template <int NT>
__global__ __launch_bounds__(NT) void topk_split_select_kernel(TopkSplitArgs a) {
  constexpr int kSelWaves = NT / 64;
  __shared__ uint32_t kk[kSpKeep];
  __shared__ int32_t kp[kSpKeep];
  __shared__ int hist[kSpBins];
  __shared__ int red[kSelWaves];
  __shared__ int found[3];
  __shared__ int preK[kSpMaxChunks + 1];
  __shared__ int tot[4];
  __shared__ uint32_t small[66];
  __shared__ int nsmall;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int k = a.k;
  const int b = (int)(row / a.T);
  const int lim = candidate_limit(a.q_pos, a.kv_len, b, row, a.L);
  const int nch = min(a.nchunk, (lim + kSpChunk - 1) / kSpChunk);
  int32_t* out = a.idx + row * k;

  // ---- the chunks' counts -> offsets of their kept keys ----
  {
    const int32_t* cnt = a.cnt + row * a.nchunk * 4;
    int ca = 0, ci = 0, cc = 0;
    if (tid < nch) {
      const int4 c4 = *(const int4*)(cnt + 4 * tid);
      ca = c4.x;
      ci = c4.y;
      cc = c4.z;
    }
    int tK;
    const int ek = sp_scan_excl<NT>(ca + ci, red, tK);
    const int tA = sp_block_sum<NT>(ca, red);
    const int tC = sp_block_sum<NT>(cc, red);
    if (tid < nch) preK[tid] = ek;
    if (tid == 0) {
      preK[nch] = tK;
      tot[0] = tA;
      tot[1] = tK - tA;
      tot[2] = tC;
    }
    __syncthreads();
  }
  const int A = tot[0], I = tot[1], V = tot[2], K = A + I;
  const int n_sel = min(k, V);
  const bool fast = V > k && A < k && K >= k && K <= kSpKeep;

  if (fast) {
    const uint32_t lo = a.bracket[2 * row * a.nchunk], hi = a.bracket[2 * row * a.nchunk + 1];
    // ---- kept keys into LDS (chunk order = position order): 256 / nch
    //      threads per chunk, 16 loads in flight per thread and batch ----
    {
      const int tpc = NT / nch;  // >= 1
      const int c = tid / tpc, r = tid % tpc;
      if (c < nch) {
        const int n_c = preK[c + 1] - preK[c];
        const int d0 = preK[c];
        const int64_t src0 = (row * a.nchunk + c) * (int64_t)kSpChunk;
        for (int i0 = r; i0 < n_c; i0 += 16 * tpc) {
          uint32_t vk[16];
          int32_t vp[16];
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const int i = min(i0 + tpc * m, n_c - 1);
            vk[m] = a.keepk[src0 + i];
            vp[m] = a.keepp[src0 + i];
          }
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const int i = i0 + tpc * m;
            if (i < n_c) {
              kk[d0 + i] = vk[m];
              kp[d0 + i] = vp[m];
            }
          }
        }
      }
    }
    // ---- tau: the (k - A)-th largest inside key, by radix passes over the
    //      offsets key - lo (11 bits at a time, from the top) ----
    int krem = k - A;
    uint32_t prefix = 0u, pmask = 0u;
    const uint32_t span = hi - lo;
    int top = span ? 31 - __clz(span) : -1;
    uint32_t tau = 0u;
    int need_eq = 0;
    bool done = false;
#pragma unroll 1
    while (top >= 0) {
      const int width = min(11, top + 1);
      const int s2 = top + 1 - width;
      const uint32_t dmask = (1u << width) - 1u;
      __syncthreads();  // kept keys stored / previous bins read
      for (int i = tid; i < kSpBins; i += NT) hist[i] = 0;
      if (tid == 0) nsmall = 0;
      __syncthreads();
#pragma unroll 1
      for (int j0 = 0; j0 < K; j0 += NT) {
        const int j = j0 + tid;
        const uint32_t key = j < K ? kk[j] : 0u;
        const uint32_t c = key - lo;
        hist_add(hist, (c >> s2) & dmask, j < K && key <= hi && (c & pmask) == prefix);
      }
      sp_rank_bin<NT>(hist, krem, red, found);
      prefix |= (uint32_t)found[0] << s2;
      pmask |= dmask << s2;
      krem -= found[1];
      top = s2 - 1;
      if (top >= 0 && hist[found[0]] <= 64) {
        // few keys left in the bin: one wave ranks them directly
#pragma unroll 1
        for (int j0 = 0; j0 < K; j0 += NT) {
          const int j = j0 + tid;
          const uint32_t key = j < K ? kk[j] : 0u;
          if (j < K && key <= hi && ((key - lo) & pmask) == prefix) small[atomicAdd(&nsmall, 1)] = key;
        }
        __syncthreads();
        if (tid < 64) {
          const int n = nsmall;
          const uint32_t x = tid < n ? small[tid] : 0u;  // kept keys are >= lo >= 1
          int gt = 0, eq = 0;
          for (int i = 0; i < n; ++i) {
            const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, i);
            gt += y > x;
            eq += y == x;
          }
          const uint64_t hit = __ballot(tid < n && gt < krem && krem <= gt + eq);
          const int lead = __ffsll((unsigned long long)hit) - 1;
          if (tid == lead) {
            small[64] = x;
            small[65] = (uint32_t)(krem - gt);
          }
        }
        __syncthreads();
        tau = small[64];
        need_eq = (int)small[65];
        done = true;
        break;
      }
    }
    if (!done) {
      tau = lo + prefix;
      need_eq = krem;
    }
    // ---- ascending output: thread t scans its run of the kept keys ----
    __syncthreads();
    const int s = (K + NT - 1) / NT;  // <= 64
    const int j0 = tid * s, j1 = min(K, j0 + s);
    int c = 0;
    for (int j = j0; j < j1; ++j) c += ((kk[j] > tau) << 16) | (kk[j] == tau);
    int total;
    const int before = sp_scan_excl<NT>(c, red, total);  // gt, eq <= 16384 each
    int gtb = before >> 16, eqb = before & 0xffff;
    for (int j = j0; j < j1; ++j) {
      const bool g = kk[j] > tau, eq = kk[j] == tau;
      if (g || (eq && eqb < need_eq)) out[gtb + min(eqb, need_eq)] = kp[j];
      gtb += g;
      eqb += eq;
    }
  } else {
    // ---- straight from the row: radix passes over all its keys ----
    const float* srow = a.scores + row * a.L;
    uint32_t tau = 0u;  // V <= k: every candidate (key > 0) is taken
    int need_eq = 0;
    if (V > k) {
      int krem = k;
      uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
      for (int pass = 0; pass < 3; ++pass) {
        const int s2 = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
        __syncthreads();
        for (int i = tid; i < kSpBins; i += NT) hist[i] = 0;
        __syncthreads();
#pragma unroll 1
        for (int q0 = 0; q0 < lim; q0 += NT) {
          const int q = q0 + tid;
          const uint32_t c = q < lim ? score_key(srow[q]) : 0u;
          hist_add(hist, (c >> s2) & dmask, c != 0u && (c & pmask) == prefix);
        }
        sp_rank_bin<NT>(hist, krem, red, found);
        prefix |= (uint32_t)found[0] << s2;
        pmask |= dmask << s2;
        krem -= found[1];
      }
      tau = prefix;
      need_eq = krem;
    }
    // emission in position order, 256 positions per round
    int run_gt = 0, run_eq = 0;
#pragma unroll 1
    for (int q0 = 0; q0 < lim; q0 += NT) {
      const int q = q0 + tid;
      const uint32_t c = q < lim ? score_key(srow[q]) : 0u;
      const int g = c != 0u && c > tau, eq = c != 0u && c == tau;
      int total;
      const int before = sp_scan_excl<NT>((g << 16) | eq, red, total);
      const int gtb = run_gt + (before >> 16), eqb = run_eq + (before & 0xffff);
      if (g || (eq && eqb < need_eq)) out[gtb + min(eqb, need_eq)] = q;
      run_gt += total >> 16;
      run_eq += total & 0xffff;
    }
  }
  __syncthreads();
  for (int i = n_sel + tid; i < k; i += NT) out[i] = -1;
  if (a.count && tid == 0) a.count[row] = n_sel;
}

static bool topk_split(int64_t rows, int L) { return rows <= kSpMaxRows && L >= kSpMinL &&
                                                     (L + kSpChunk - 1) / kSpChunk <= kSpMaxChunks; }

static int topk_chunks(int L) { return (L + kTkRow - 1) / kTkRow; }

bool topk_supported(int L, int k) {
  if (k < 1 || k > kTopkMaxK) return false;
  const int nch = topk_chunks(L);
  // the merge launch holds ceil(L / 32768) * k candidates in one work-group
  return nch == 1 || (int64_t)nch * k <= kTkRow;
}

static size_t split_bytes(int64_t rows, int L) {
  const int64_t units = rows * ((L + kSpChunk - 1) / kSpChunk);
  return (size_t)units * (4 * sizeof(int32_t) + 2 * sizeof(uint32_t) +
                          (size_t)kSpChunk * 2 * sizeof(int32_t));
}

size_t topk_workspace_bytes(int B, int T, int L, int k) {
  const int64_t rows = (int64_t)B * T;
  if (topk_split(rows, L)) return split_bytes(rows, L);
  const int nch = topk_chunks(L);
  if (nch <= 1) return 0;
  return (size_t)rows * nch * k * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.T;
  if (rows == 0) return hipSuccess;
  if (topk_split(rows, a.L)) {
    TopkSplitArgs sp{};
    sp.scores = a.scores;
    sp.q_pos = a.q_pos;
    sp.kv_len = a.kv_len;
    sp.T = a.T;
    sp.L = a.L;
    sp.k = a.k;
    sp.nchunk = (a.L + kSpChunk - 1) / kSpChunk;
    sp.vec4 = (a.L % 4 == 0) && ((uintptr_t)a.scores % 16 == 0);
    const int64_t units = rows * sp.nchunk;
    sp.cnt = (int32_t*)a.ws;
    sp.bracket = (uint32_t*)(sp.cnt + units * 4);
    sp.keepk = sp.bracket + units * 2;
    sp.keepp = (int32_t*)(sp.keepk + units * kSpChunk);
    sp.idx = a.idx;
    sp.count = a.count;
    topk_split_scan_kernel<<<dim3(sp.nchunk, (unsigned)rows), kSpThreads, 0, st>>>(sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    topk_split_select_kernel<kSpSelThreads><<<(unsigned)rows, kSpSelThreads, 0, st>>>(sp);
    return hipGetLastError();
  }
  TopkRowArgs r{};
  r.scores = a.scores;
  r.q_pos = a.q_pos;
  r.kv_len = a.kv_len;
  r.T = a.T;
  r.L = a.L;
  r.k = a.k;
  r.nchunks = topk_chunks(a.L);
  r.idx = a.idx;
  r.count = a.count;
  if (r.nchunks > 1) {
    r.cand_score = (float*)a.ws;
    r.cand_pos = (int32_t*)((char*)a.ws + sizeof(float) * rows * r.nchunks * a.k);
  }
  topk_kernel<false><<<dim3(r.nchunks, (unsigned)rows), kTkThreads, 0, st>>>(r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || r.nchunks == 1) return e;
  topk_kernel<true><<<dim3(1, (unsigned)rows), kTkThreads, 0, st>>>(r);
  return hipGetLastError();
}

}  // namespace sa
