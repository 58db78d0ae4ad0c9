// split_select.hpp -- the second phase of the split Top-K (few long rows):
// from the chunk work-groups' counts and kept keys, the row's k selected
// positions in ascending order.  Its pieces (the radix search for tau over
// kept keys, the straight row select) also serve the select over the decode
// indexer's candidate lists, and the histogram helpers the indexer's own
// floor search, so every path finds tau by the same code.
//
// Selection rule ("Sparse Attention 数学学习笔记" §9; "MLA 与稀疏注意力" DSA
// section, the selected-position helper ordering by (-score, position)):
// exactly min(k, #candidates) candidates; larger scores first; equal scores
// to the lower position.
//
// The first phase (topk_split_scan_kernel) cuts a row into 4096-position
// chunks; every chunk keeps its keys >= lo, compacted in position order, and
// counts those above hi and inside [lo, hi], around a key bracket [lo, hi]
// drawn from a row sample.  Here:
//  1. the chunks' counts give the offsets of their kept keys;
//  2. if the bracket holds the k-th key (above < k <= above + inside) and
//     the kept keys fit in LDS, radix passes over the inside keys find tau,
//     the k-th largest key, and need_eq, how many keys equal to tau are
//     taken; one block scan over the kept keys in position order then gives
//     every selected key its ascending output slot;
//  3. otherwise the row's scores are read directly: radix passes over all
//     its keys, then emission in position order, NT positions per round.
#pragma once
#include "common.hpp"
#include "select_core.hpp"

namespace sa {

constexpr int kSpChunk = 4096;
constexpr int kSpBins = 2048;
constexpr int kSpMaxChunks = 256;  // rows up to 1M positions

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

// Exclusive block scan over the NT threads of a work-group.
template <int NT>
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
template <int NT>
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
template <int NT>
__device__ __forceinline__ void sp_rank_bin(const int* hist, int r, int* red, int* found) {
  sp_rank_bins<NT>(hist, r, r, red, found);
}

template <int NT>
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

// The bin of `hist` (kSpBins bins, 16-byte aligned) holding rank r counted
// from the top (1 <= r <= total) and the entries in higher bins, found by one
// wave on its own: every wave that calls it gets the same answer, with no
// barrier.  Lane l sums the 32 bins below 2048 - 32 l (its 16-byte reads
// rotated by lane against bank conflicts); the wave then reads the 32 bins of
// the lane holding rank r, one per lane from the top, and a prefix scan over
// them names the bin.  total = all entries; bin = -1 when r > total.
__device__ __forceinline__ void wave_rank_bin(const int* hist, int r, int& bin, int& above,
                                              int& total) {
  const int lane = lane_id();
  const int base = kSpBins - 32 * (lane + 1);
  int own = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int4 v = *(const int4*)(hist + base + 4 * ((q + lane) & 7));
    own += v.x + v.y + v.z + v.w;
  }
  const int incl = wave_scan_incl(own);
  total = __builtin_amdgcn_readlane(incl, 63);
  const int ab = incl - own;  // entries in the bins above this lane's
  const uint64_t m = __ballot(ab < r && r <= incl);
  bin = -1;
  above = 0;
  if (m == 0) return;
  const int src = __ffsll((unsigned long long)m) - 1;
  const int sbase = __builtin_amdgcn_readlane(base, src);
  const int sab = __builtin_amdgcn_readlane(ab, src);
  const int h = lane < 32 ? hist[sbase + 31 - lane] : 0;  // lane i: i-th bin from the top
  const int hi = wave_scan_incl(h);
  const uint64_t mm = __ballot(lane < 32 && sab + hi - h < r && r <= sab + hi);
  const int f = __ffsll((unsigned long long)mm) - 1;
  bin = sbase + 31 - f;
  above = sab + __builtin_amdgcn_readlane(hi - h, f);
}

// What the first phase left in the workspace, per (row, chunk).
struct SplitView {
  const float* scores;      // [rows][L] (the fallback reads the row itself)
  int L, nchunk;
  const int32_t* cnt;       // [rows][nchunk][4]: above, inside, candidates, -
  const uint32_t* bracket;  // [rows][nchunk][2]: lo, hi (equal in every chunk)
  const uint32_t* keepk;    // [rows][nchunk][kSpChunk]: kept keys (>= lo), position order
  const int32_t* keepp;     // [rows][nchunk][kSpChunk]: their positions
};

// LDS the select works in: KEEP kept keys and positions, the histogram and
// a few scalars.
struct SplitSmem {
  uint32_t* kk;    // [KEEP]
  int32_t* kp;     // [KEEP]
  int* hist;       // [kSpBins]
  int* red;        // [NT / 64]
  int* found;      // [3]
  int* preK;       // [kSpMaxChunks + 1]
  int* tot;        // [4]
  uint32_t* small; // [68], 16-byte aligned
  int* nsmall;     // [1]
};

// tau, the krem-th largest of the kept keys that lie in [lo, hi] (ranks
// counted from the top), and need_eq, how many of the keys equal to tau are
// taken: radix passes over the offsets key - lo, 11 bits at a time from the
// top, until at most 64 keys share the current bin; one wave then ranks those
// directly.  Thread t holds its kept keys in rk[0, s) (0: none; kept keys are
// >= lo >= 1).  Run by all NT threads; 1 <= krem <= the keys in [lo, hi].
template <int NT, int RUN>
__device__ __forceinline__ void kept_tau(const uint32_t (&rk)[RUN], int s, uint32_t lo,
                                         uint32_t hi, int krem, const SplitSmem& sm,
                                         uint32_t& tau_out, int& need_out) {
  const int tid = threadIdx.x;
  int* const red = sm.red;
  int* const found = sm.found;
  uint32_t prefix = 0u, pmask = 0u;
  const uint32_t span = hi - lo;
  int top = span ? 31 - __clz(span) : -1;
#pragma unroll 1
  while (top >= 0) {
    const int width = min(11, top + 1);
    const int s2 = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    __syncthreads();  // previous bins read
    for (int i = tid; i < kSpBins; i += NT) sm.hist[i] = 0;
    if (tid == 0) *sm.nsmall = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < RUN; ++e) {  // key 0 (none) is below lo >= 1
      if (e >= s) break;              // uniform
      const uint32_t c = rk[e] - lo;
      hist_add(sm.hist, (c >> s2) & dmask, rk[e] >= lo && rk[e] <= hi && (c & pmask) == prefix);
    }
    sp_rank_bin<NT>(sm.hist, krem, red, found);
    prefix |= (uint32_t)found[0] << s2;
    pmask |= dmask << s2;
    krem -= found[1];
    top = s2 - 1;
    if (top >= 0 && sm.hist[found[0]] <= 64) {
      // few keys left in the bin: one wave ranks them directly
#pragma unroll
      for (int e = 0; e < RUN; ++e) {
        if (e >= s) break;  // uniform
        if (rk[e] >= lo && rk[e] <= hi && ((rk[e] - lo) & pmask) == prefix)
          sm.small[atomicAdd(sm.nsmall, 1)] = rk[e];
      }
      __syncthreads();
      if (tid < 64) {
        const int n = *sm.nsmall;
        const uint32_t x = tid < n ? sm.small[tid] : 0u;  // kept keys are >= lo >= 1
        // each lane compares its key with all n keys, four per (broadcast) read
        int gt = 0, eq = 0;
        for (int i0 = 0; i0 < n; i0 += 4) {
          const uint4 y = *(const uint4*)(sm.small + i0);
          gt += (y.x > x) + (i0 + 1 < n && y.y > x) + (i0 + 2 < n && y.z > x) +
                (i0 + 3 < n && y.w > x);
          eq += (y.x == x) + (i0 + 1 < n && y.y == x) + (i0 + 2 < n && y.z == x) +
                (i0 + 3 < n && y.w == x);
        }
        const uint64_t hit = __ballot(tid < n && gt < krem && krem <= gt + eq);
        const int lead = __ffsll((unsigned long long)hit) - 1;
        if (tid == lead) {
          sm.small[64] = x;
          sm.small[65] = (uint32_t)(krem - gt);
        }
      }
      __syncthreads();
      tau_out = sm.small[64];
      need_out = (int)sm.small[65];
      return;
    }
  }
  tau_out = lo + prefix;
  need_out = krem;
}

// The row's selected positions straight from its scores (candidates: the V
// positions < lim with a key): radix passes over all its keys find tau when
// V > k, then the emission walks the row in position order.  Both take the
// row in rounds of kRsU * NT positions, each thread's kRsU loads in flight
// together (position q0 + u NT + thread in round q0); the emission's slots
// come from one scan per round over the (u, wave) totals, in that order.
// Passes emit(slot, position).  Run by all NT threads.
constexpr int kRsU = 8;
template <int NT, class Emit>
__device__ __forceinline__ void row_select(const float* srow, int k, int lim, int V,
                                           const SplitSmem& sm, Emit&& emit) {
  constexpr int NWV = NT / 64, NTAB = kRsU * NWV;
  static_assert(NTAB <= 64, "one wave scans the round's (u, wave) totals in sm.small");
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  int* const red = sm.red;
  int* const found = sm.found;
  int* const tab = (int*)sm.small;  // [NTAB] (u, wave) prefixes, [64] the round's total
  auto load = [&](int q0, uint32_t (&c)[kRsU]) {
    float f[kRsU];
#pragma unroll
    for (int u = 0; u < kRsU; ++u) f[u] = srow[min(q0 + u * NT + tid, lim - 1)];
#pragma unroll
    for (int u = 0; u < kRsU; ++u) c[u] = q0 + u * NT + tid < lim ? score_key(f[u]) : 0u;
  };
  // ---- straight from the row: radix passes over all its keys ----
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
      for (int i = tid; i < kSpBins; i += NT) sm.hist[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int q0 = 0; q0 < lim; q0 += kRsU * NT) {
        uint32_t c[kRsU];
        load(q0, c);
#pragma unroll
        for (int u = 0; u < kRsU; ++u)
          hist_add(sm.hist, (c[u] >> s2) & dmask, c[u] != 0u && (c[u] & pmask) == prefix);
      }
      sp_rank_bin<NT>(sm.hist, krem, red, found);
      prefix |= (uint32_t)found[0] << s2;
      pmask |= dmask << s2;
      krem -= found[1];
    }
    tau = prefix;
    need_eq = krem;
  }
  // ---- emission in position order ----
  int run_gt = 0, run_eq = 0;
#pragma unroll 1
  for (int q0 = 0; q0 < lim; q0 += kRsU * NT) {
    uint32_t c[kRsU];
    load(q0, c);
    int cu[kRsU], wi[kRsU];  // (keys > tau) << 16 | ties: at most kRsU * NT each
#pragma unroll
    for (int u = 0; u < kRsU; ++u) {
      cu[u] = ((c[u] != 0u && c[u] > tau) << 16) | (c[u] != 0u && c[u] == tau);
      wi[u] = wave_scan_incl(cu[u]);
    }
    __syncthreads();  // the previous round's table is read
    if (lane == 63) {
#pragma unroll
      for (int u = 0; u < kRsU; ++u) tab[u * NWV + wave] = wi[u];
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefixes in (u, wave) order: position order
      const int v = lane < NTAB ? tab[lane] : 0;
      const int inc = wave_scan_incl(v);
      if (lane < NTAB) tab[lane] = inc - v;
      if (lane == 63) tab[64] = inc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRsU; ++u) {
      const int before = tab[u * NWV + wave] + wi[u] - cu[u];
      const int gtb = run_gt + (before >> 16), eqb = run_eq + (before & 0xffff);
      const bool g = (cu[u] >> 16) != 0, eq = (cu[u] & 1) != 0;
      if (g || (eq && eqb < need_eq)) emit(gtb + min(eqb, need_eq), q0 + u * NT + tid);
    }
    const int total = tab[64];
    run_gt += total >> 16;
    run_eq += total & 0xffff;
  }
}

// The selected positions of row `row` (candidates: positions < lim with a
// key), each passed to emit(slot, position) with its ascending output slot
// slot < min(k, #candidates), which is returned.  loaded() runs once the
// function has issued its last global load of the fast path (a caller can
// start other memory traffic there without delaying the select's own
// loads).  Run by all NT threads of a work-group; ends with a barrier
// (emit's LDS writes are visible).
template <int NT, int KEEP, class Emit, class Loaded>
__device__ __forceinline__ int split_select(const SplitView& v, int64_t row, int k, int lim,
                                            const SplitSmem& sm, Emit&& emit, Loaded&& loaded) {
  constexpr int kRun = (KEEP + NT - 1) / NT;  // kept keys per thread in the emission
  static_assert(kSpMaxChunks <= NT && KEEP <= 65535, "chunk counts per thread; packed counts");
  const int tid = threadIdx.x;
  const int nch = min(v.nchunk, (lim + kSpChunk - 1) / kSpChunk);
  int* const red = sm.red;

  // ---- the chunks' counts -> offsets of their kept keys ----
  {
    const int32_t* cnt = v.cnt + row * v.nchunk * 4;
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
    if (tid < nch) sm.preK[tid] = ek;
    if (tid == 0) {
      sm.preK[nch] = tK;
      sm.tot[0] = tA;
      sm.tot[1] = tK - tA;
      sm.tot[2] = tC;
    }
    __syncthreads();
  }
  const int A = sm.tot[0], I = sm.tot[1], V = sm.tot[2], K = A + I;
  (void)I;
  const int n_sel = min(k, V);
  const bool fast = V > k && A < k && K >= k && K <= KEEP;

  if (fast) {
    const uint32_t lo = v.bracket[2 * row * v.nchunk], hi = v.bracket[2 * row * v.nchunk + 1];
    // ---- kept keys into LDS (chunk order = position order): NT / nch
    //      threads per chunk, 16 loads in flight per thread and batch ----
    {
      const int tpc = NT / nch;  // >= 1
      const int c = tid / tpc, r = tid % tpc;
      if (c < nch) {
        const int n_c = sm.preK[c + 1] - sm.preK[c];
        const int d0 = sm.preK[c];
        const int64_t src0 = (row * v.nchunk + c) * (int64_t)kSpChunk;
        for (int i0 = r; i0 < n_c; i0 += 16 * tpc) {
          uint32_t vk[16];
          int32_t vp[16];
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const int i = min(i0 + tpc * m, n_c - 1);
            vk[m] = v.keepk[src0 + i];
            vp[m] = v.keepp[src0 + i];
          }
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const int i = i0 + tpc * m;
            if (i < n_c) {
              sm.kk[d0 + i] = vk[m];
              sm.kp[d0 + i] = vp[m];
            }
          }
        }
      }
    }
    loaded();
    // Thread t owns the run of kept keys [s t, s t + s), held in registers
    // from here on: the radix passes, the small-bin ranking and the emission
    // read them there instead of waiting out an LDS read per key.
    __syncthreads();  // kept keys stored
    const int s = (K + NT - 1) / NT;  // <= kRun
    const int j0 = tid * s;
    uint32_t rk[kRun];
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (e >= s) break;  // uniform
      rk[e] = j0 + e < K ? sm.kk[j0 + e] : 0u;  // 0: none
    }
    // ---- tau: the (k - A)-th largest inside key ----
    uint32_t tau;
    int need_eq;
    kept_tau<NT>(rk, s, lo, hi, k - A, sm, tau, need_eq);
    // ---- ascending output: thread t counts its run's selected keys, a
    //      block scan gives their slots ----
    int c = 0;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (e >= s) break;  // uniform
      c += ((rk[e] > tau) << 16) | (rk[e] == tau);
    }
    int total;
    const int before = sp_scan_excl<NT>(c, red, total);  // gt, eq < 65536 each
    int gtb = before >> 16, eqb = before & 0xffff;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (e >= s) break;  // uniform
      const bool g = rk[e] > tau, eq = rk[e] == tau;
      if (g || (eq && eqb < need_eq)) emit(gtb + min(eqb, need_eq), sm.kp[j0 + e]);
      gtb += g;
      eqb += eq;
    }
  } else {
    loaded();
    row_select<NT>(v.scores + row * v.L, k, lim, V, sm, emit);
  }
  __syncthreads();
  return n_sel;
}

}  // namespace sa
