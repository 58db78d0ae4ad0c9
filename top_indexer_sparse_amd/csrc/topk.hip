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
//  2. tau = the k-th largest key.  The first histogram digit is fitted to the
//     row: d = (key - min key) >> sh with sh chosen so that the key range
//     spans at most 2048 bins.  Index scores share their sign and exponent,
//     so fixed high-bit digits would pile most keys onto a handful of LDS
//     addresses and serialise the atomics.  A block scan from the top finds
//     the bin holding rank k; only that bin's keys (block-scan compacted into
//     LDS) take part in the passes over the remaining sh bits.
//  3. Packed (greater-than-tau, equal-to-tau) counts, scanned over the block
//     in position order, give every selected key its output slot and its
//     rank among the ties: keys > tau and the first k - count(> tau) keys
//     == tau are placed in ascending position order in LDS, then written out
//     with coalesced stores.
// Rows longer than 32768 positions are cut into 32768-position chunks; each
// chunk keeps its own top-k (a superset of its share of the row's top-k under
// the same rule), and a second launch selects from the chunks' candidates,
// which are laid out in ascending position order, so the tie rule carries over.
#include "common.hpp"
#include "launch.hpp"

namespace sa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkSeg = 32;
constexpr int kTkRow = kTkThreads * kTkSeg;  // 32768 positions per work-group
constexpr int kTkBins = 2048;

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;                    // -0 == +0
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0xff800000u) return 0u;                 // -inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __builtin_bit_cast(float, u);
}

// Inclusive block scan (sum) of one int per thread; `red` holds kTkWaves ints.
// Returns the inclusive prefix; `total` receives the block sum.
__device__ __forceinline__ int block_scan_incl(int x, int* red, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();  // red may still be read by a previous scan
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    int v = red[w];
    if (w < wave) before += v;
    total += v;
  }
  return x + before;
}

__device__ __forceinline__ int block_sum(int x, int* red) {
  int total;
  block_scan_incl(x, red, total);
  return total;
}

// The bin of `hist` (2048 bins) holding rank krem counted from the top;
// writes (bin, keys in higher bins) to found[0..1].  1024 threads, thread t
// owning bins 2047-2t and 2046-2t.  Starts with a barrier (the histogram is
// complete) and ends with one (found is visible).
__device__ __forceinline__ void find_rank_bin(const int* hist, int krem, int* red, int* found) {
  __syncthreads();
  const int tid = threadIdx.x;
  const int bhi = kTkBins - 1 - 2 * tid, blo = bhi - 1;
  const int hhi = hist[bhi], hlo = hist[blo];
  int total;
  const int incl = block_scan_incl(hhi + hlo, red, total);
  const int above = incl - hhi - hlo;
  if (above < krem && krem <= above + hhi) {
    found[0] = bhi;
    found[1] = above;
  } else if (above + hhi < krem && krem <= above + hhi + hlo) {
    found[0] = blo;
    found[1] = above + hhi;
  }
  __syncthreads();
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

// MERGE = false: virtual row = positions [chunk*kTkRow, ...) of a score row.
// MERGE = true : virtual row = the nchunks*k candidates of a row.
template <bool MERGE>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkRowArgs a) {
  __shared__ uint32_t cand[kTkRow];  // rank-k bin candidates, then the output
  __shared__ int hist[kTkBins];
  __shared__ int red[kTkWaves];
  __shared__ uint32_t rmin[kTkWaves], rmax[kTkWaves];
  __shared__ int found[2];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
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

  // ---- keys to registers: kr[4 i + e] is position wbase + 4 (lane + 64 i) + e
  const int wbase = wave * (kTkRow / kTkWaves);
  uint32_t kr[kTkSeg];
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    float4 f[kTkSeg / 4];
#pragma unroll
    for (int i = 0; i < kTkSeg / 4; ++i) {
      const int p = wbase + 4 * (lane + 64 * i);
      f[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p + 3 < n) f[i] = *reinterpret_cast<const float4*>(src + p);
    }
#pragma unroll
    for (int i = 0; i < kTkSeg / 4; ++i) {
      const int p = wbase + 4 * (lane + 64 * i);
      float v[4] = {f[i].x, f[i].y, f[i].z, f[i].w};
      if (p < n && p + 3 >= n) {  // the row's ragged end
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p + e < n ? src[p + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) kr[4 * i + e] = p + e < n ? score_key(v[e]) : 0u;
    }
  } else {
    float f[kTkSeg];
#pragma unroll
    for (int i = 0; i < kTkSeg / 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = wbase + 4 * (lane + 64 * i) + e;
        f[4 * i + e] = p < n ? src[p] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < kTkSeg / 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = wbase + 4 * (lane + 64 * i) + e;
        kr[4 * i + e] = p < n ? score_key(f[4 * i + e]) : 0u;
      }
    }
  }

  // ---- count, min and max of the valid keys ----
  int n_valid;
  uint32_t kmin, kmax;
  {
    uint32_t mn = 0xffffffffu, mx = 0u;
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kTkSeg; ++j) {
      nv += kr[j] != 0u;
      mn = kr[j] ? min(mn, kr[j]) : mn;
      mx = max(mx, kr[j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      nv += __shfl_xor(nv, o);
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if (lane == 0) {
      red[wave] = nv;
      rmin[wave] = mn;
      rmax[wave] = mx;
    }
    __syncthreads();
    n_valid = 0;
    kmin = 0xffffffffu;
    kmax = 0u;
#pragma unroll
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
    for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTkSeg; ++j) hist_add(hist, (kr[j] - kmin) >> sh, kr[j] != 0u);
    find_rank_bin(hist, k, red, found);
    const uint32_t bin = (uint32_t)found[0];
    int krem = k - found[1];
    const uint32_t lo = kmin + (bin << sh);
    uint32_t prefix = 0u, pmask = 0u;  // over key - lo, bits below sh
    if (sh > 0) {
      // the bin's keys (as offsets from lo) into LDS, block-scan compacted
      int mc = 0;
#pragma unroll
      for (int j = 0; j < kTkSeg; ++j) mc += kr[j] != 0u && ((kr[j] - kmin) >> sh) == bin;
      int ncand;
      int slot = block_scan_incl(mc, red, ncand) - mc;
      if (mc) {
#pragma unroll
        for (int j = 0; j < kTkSeg; ++j)
          if (kr[j] != 0u && ((kr[j] - kmin) >> sh) == bin) cand[slot++] = kr[j] - lo;
      }
      for (int top = sh - 1; top >= 0;) {
        const int width = min(11, top + 1), s2 = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        __syncthreads();  // candidates written / previous pass's bins read
        for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0;
        __syncthreads();
        const int nit = (ncand + kTkThreads - 1) / kTkThreads;
        for (int it = 0; it < nit; ++it) {
          const int j = tid + it * kTkThreads;
          const uint32_t c = j < ncand ? cand[j] : 0u;
          hist_add(hist, (c >> s2) & dmask, j < ncand && (c & pmask) == prefix);
        }
        find_rank_bin(hist, krem, red, found);
        prefix |= (uint32_t)found[0] << s2;
        pmask |= dmask << s2;
        krem -= found[1];
        top = s2 - 1;
      }
    }
    tau = lo + prefix;
    need_eq = krem;
    __syncthreads();  // cand is reused for the output below
  }
  const int n_sel = min(k, n_valid);

  // ---- slots in position order: scan of packed (gt, eq) counts ----
  int c4[kTkSeg / 4];
  int wtot = 0;
#pragma unroll
  for (int i = 0; i < kTkSeg / 4; ++i) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = kr[4 * i + e];
      gt += key > tau;
      eq += (key == tau) & (key != 0u);
    }
    c4[i] = (gt << 16) | eq;  // gt <= k <= 4096 and eq <= 32768 per row
    wtot += c4[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wtot += __shfl_xor(wtot, o);
  __syncthreads();  // every thread has read red (counts above)
  if (lane == 0) red[wave] = wtot;
  __syncthreads();
  int run = 0;  // packed counts of the waves before this one
  for (int w = 0; w < wave; ++w) run += red[w];
  uint32_t* opos = cand;             // [k] virtual positions, in order
  uint32_t* okey = cand + kTopkMaxK;  // [k] their keys (chunk launches)
#pragma unroll
  for (int i = 0; i < kTkSeg / 4; ++i) {
    int x = c4[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int before = run + x - c4[i];
    run += __shfl(x, 63);
    if (c4[i]) {
      int gtb = before >> 16, eqb = before & 0xffff;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kr[4 * i + e];
        const bool g = key > tau, q = (key == tau) & (key != 0u);
        if (g || (q && eqb < need_eq)) {
          const int slot = gtb + min(eqb, need_eq);
          opos[slot] = (uint32_t)(wbase + 4 * (lane + 64 * i) + e);
          if (out_score) okey[slot] = key;
        }
        gtb += g;
        eqb += q;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += kTkThreads) {
    if (i < n_sel) {
      const int v = (int)opos[i];
      out_idx[i] = vpos ? vpos[v] : pos_base + v;
      if (out_score) out_score[i] = key_score(okey[i]);
    } else {
      out_idx[i] = -1;
      if (out_score) out_score[i] = -INFINITY;
    }
  }
  if (out_count && tid == 0) *out_count = n_sel;
}

static int topk_chunks(int L) { return (L + kTkRow - 1) / kTkRow; }

bool topk_supported(int L, int k) {
  if (k < 1 || k > kTopkMaxK) return false;
  const int nch = topk_chunks(L);
  // many rows take the one-work-group-per-row kernel, whose merge of long
  // rows holds ceil(L/32768) * k candidates
  return nch == 1 || (int64_t)nch * k <= kTkRow;
}

size_t topk_workspace_bytes(int B, int T, int L, int k) {
  const int64_t rows = (int64_t)B * T;
  const int nch = topk_chunks(L);
  if (nch <= 1) return 0;
  return (size_t)rows * nch * k * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.T;
  if (rows == 0) return hipSuccess;
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
