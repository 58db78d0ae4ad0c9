// prefill.hip -- fused prefill select: the lightning-indexer scores of a query
// row and its Top-K in one kernel, with the row's scores held in LDS.
//
// "MLA 与稀疏注意力", DSA section: the indexer score I_{t,s} and the Top-K
// over the causal candidates s <= t ("Sparse Attention 数学学习笔记" §9 for the
// score).  The selection rule is the one of the top-k kernels: exactly
// min(k, #candidates) positions, larger scores first, equal scores to the
// lower position, NaN and -inf never selected; the output lists the selected
// positions in ascending order, -1 padded, with their number in count.
//
// One work-group of four waves per query row (b, t):
//  1. Scores.  Wave w takes the w-th quarter of the candidate range [0, lim)
//     and streams its keys from global memory through a register ring of
//     16-position chunks, exactly as the decode score kernel does (the same
//     QueryRegs::score, so the scores carry the same bits as the score
//     kernels').  They land in the row buffer in LDS, 4 bytes per position:
//     no score is written to global memory.
//  2. Select.  The row turns into order-preserving keys in place.  tau, the
//     k-th largest key, comes from a radix select on a digit fitted to the
//     row's key range: 2048 bins per pass, at most three passes, each pass
//     narrowing to the bin that holds the wanted rank.  The last pass also
//     gives `take`, the number of keys equal to tau that are selected.
//  3. Emit.  Each wave walks its quarter again in position order: keys above
//     tau, and the first `take` keys equal to tau of the whole row, go to
//     consecutive output slots, so the list comes out ascending.
// The row buffer bounds L (at most 32768 positions, 128 KB); at L <= 16384 two
// work-groups share a CU, so one row's select overlaps another's scores.
#include "common.hpp"
#include "index_core.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace sa {

constexpr int kPfsThreads = 256;
constexpr int kPfsBins = 2048;
constexpr int kPfsBinBits = 11;

// Exclusive scan over the work-group's four waves of one int per thread.
__device__ __forceinline__ int pfs_block_excl(int x, int* red, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  __syncthreads();  // red may still be read by a previous scan
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kPfsThreads / 64; ++i) {
    const int v = red[i];
    before += i < wave ? v : 0;
    total += v;
  }
  return incl - x + before;
}

template <int HT, int DI, bool FP8>
__global__ __launch_bounds__(kPfsThreads) void pf_select_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, int topk, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  constexpr int HI = 16 * HT;
  constexpr int ROWB = FP8 ? DI : 2 * DI;
  constexpr int R = 16 * HT * DI >= 16384 ? 4 : 8;  // ring depth (as the decode scores)
  extern __shared__ uintx4 row_v[];                  // round_up(L, 64) + 64 words
  uint32_t* row = (uint32_t*)row_v;
  __shared__ uint32_t hist[kPfsBins];
  __shared__ float spill[4][16];  // scores of ring chunks past a wave's range
  __shared__ int red[4], red2[4], red3[4], red4[4];
  __shared__ uint32_t ured[8];
  __shared__ int found[2];

  const int t = T - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int64_t bt = (int64_t)b * T + t;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int lim = candidate_limit(q_pos, kv_len, b, bt, L);
  // wave quarters: multiples of 16 positions
  const int span = ((lim + 3) / 4 + 15) & ~15;
  const int s_begin = wave * span;
  const int v_end = min(s_begin + span, lim);

  // ---- 1. scores into the LDS row ----
  if (s_begin < v_end) {  // wave-uniform
    const uint8_t* kb = k + (int64_t)b * L * ROWB;
    const int nch = (v_end - s_begin + 15) / 16;
    auto row_of = [&](int c) {
      return kb + (int64_t)min(s_begin + 16 * c + n, v_end - 1) * ROWB;
    };
    QueryRegs<HT, DI, FP8> qr;
    qr.load(q + bt * HI * DI, w + bt * HI, lane);
    // the query has landed before the ring starts, so that the ring's waits
    // count only its own loads
    wait_vmcnt<0>();
    KeyChunk<DI, FP8> ring[R];
    float* rowf = (float*)row + s_begin;
    for (int c0 = -R; c0 < nch; c0 += R) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = c0 + i;
        if (c0 >= 0) {  // uniform; chunks past nch are computed and dropped
          const float sc = qr.score(ring[i]);
          float* dst = c < nch ? rowf + 16 * c : spill[wave];
          dst[n] = sc;  // the four lane groups write the same value
        }
        ring[i].load(row_of(c + R), g);
      }
    }
  }
  __syncthreads();

  // ---- 2a. keys in place; candidates, smallest and largest key ----
  const float* scb = FP8 ? kscale + (int64_t)b * L : nullptr;
  int nv = 0;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int s4 = 4 * tid; s4 < lim; s4 += 4 * kPfsThreads) {
    uintx4 v = *(const uintx4*)&row[s4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = s4 + e;
      // through a scalar: a bit_cast taken straight from a vector element
      // was compiled to a load of element 0 only
      const uint32_t raw = v[e];
      float f = __builtin_bit_cast(float, raw);
      if constexpr (FP8) f *= scb[min(s, lim - 1)];
      const uint32_t key = s < lim ? score_key(f) : 0u;
      v[e] = key;
      nv += key != 0u;
      if (key != 0u) mn = min(mn, key);
      mx = max(mx, key);
    }
    *(uintx4*)&row[s4] = v;
  }
  {
    const int wnv = wave_total(nv);
    const uint32_t wmn = wave_min_u32(mn), wmx = wave_max_u32(mx);
    if (lane == 0) {
      red[wave] = wnv;
      ured[wave] = wmn;
      ured[4 + wave] = wmx;
    }
  }
  __syncthreads();
  int nv_all = 0;
  uint32_t mn_all = 0xffffffffu, mx_all = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nv_all += red[i];
    mn_all = min(mn_all, ured[i]);
    mx_all = max(mx_all, ured[4 + i]);
  }

  // ---- 2b. tau and take ----
  uint32_t tau = 0u;  // select keys > tau, and the first `take` keys == tau
  int take = 0;
  if (nv_all > topk) {
    uint32_t lo = mn_all;
    const uint32_t range = mx_all - mn_all;
    const int bits = range ? 32 - __builtin_clz(range) : 0;
    int sh = max(0, bits - kPfsBinBits);
    uint32_t nb = kPfsBins;  // bins of this pass: the range is [lo, lo + (nb << sh))
    int r = topk;            // wanted rank, counted from the top inside the range
    for (;;) {
      for (int i = tid; i < kPfsBins; i += kPfsThreads) hist[i] = 0u;
      __syncthreads();
      for (int s4 = 4 * tid; s4 < lim; s4 += 4 * kPfsThreads) {
        const uintx4 v = *(const uintx4*)&row[s4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = v[e];
          if (s4 + e < lim && key >= lo) {
            const uint32_t d = (key - lo) >> sh;
            if (d < nb) atomicAdd(&hist[d], 1u);
          }
        }
      }
      __syncthreads();
      // thread i owns bins 2047 - 8 i down to 2040 - 8 i (top first)
      const int top = kPfsBins - 1 - 8 * tid;
      int c = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) c += (int)hist[top - j];
      int total;
      int acc = pfs_block_excl(c, red2, total);  // keys in higher bins
      if (acc < r && r <= acc + c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int hb = (int)hist[top - j];
          if (acc < r && r <= acc + hb) {
            found[0] = top - j;
            found[1] = acc;
          }
          acc += hb;
        }
      }
      __syncthreads();
      const int bin = found[0], above = found[1];
      r -= above;
      lo += (uint32_t)bin << sh;
      if (sh == 0) {
        tau = lo;
        take = r;
        break;
      }
      // the next pass splits this bin, 2^sh keys wide, into at most 2048 bins
      const int sh_next = max(0, sh - kPfsBinBits);
      nb = 1u << (sh - sh_next);
      sh = sh_next;
    }
  }
  const int cnt = min(nv_all, topk);

  // ---- 3. emit in position order ----
  int gt = 0, eq = 0;
  for (int s4 = s_begin + 4 * lane; s4 < v_end; s4 += 256) {
    const uintx4 v = *(const uintx4*)&row[s4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = s4 + e < v_end;
      gt += in && v[e] > tau;
      eq += in && v[e] == tau && tau != 0u;
    }
  }
  {
    const int wgt = wave_total(gt), weq = wave_total(eq);
    if (lane == 0) {
      red3[wave] = wgt;
      red4[wave] = weq;
    }
  }
  __syncthreads();
  int base = 0, eq_before = 0;
  for (int i = 0; i < wave; ++i) {
    const int ti = min(max(take - eq_before, 0), red4[i]);  // ties wave i takes
    base += red3[i] + ti;
    eq_before += red4[i];
  }
  int32_t* out = idx + bt * topk;
  int run_sel = 0, run_eq = 0;
  for (int s0 = s_begin; s0 < v_end; s0 += 256) {  // uniform rounds of 64 x 4
    const int s4 = s0 + 4 * lane;
    uintx4 v = {0u, 0u, 0u, 0u};
    if (s4 < v_end) v = *(const uintx4*)&row[s4];
    int leq = 0;
    bool isgt[4], iseq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = s4 + e < v_end;
      isgt[e] = in && v[e] > tau;
      iseq[e] = in && v[e] == tau && tau != 0u;
      leq += iseq[e];
    }
    const int eq_incl = wave_scan_incl(leq);
    int eq_rank = eq_before + run_eq + eq_incl - leq;  // ties before this lane's first
    bool sel[4];
    int lsel = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = isgt[e] || (iseq[e] && eq_rank < take);
      eq_rank += iseq[e];
      lsel += sel[e];
    }
    const int sel_incl = wave_scan_incl(lsel);
    int slot = base + run_sel + sel_incl - lsel;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e]) {
        if (slot < topk) out[slot] = s4 + e;  // always true; keeps every store in the row
        ++slot;
      }
    run_sel += __builtin_amdgcn_readlane(sel_incl, 63);
    run_eq += __builtin_amdgcn_readlane(eq_incl, 63);
  }
  for (int j = cnt + tid; j < topk; j += kPfsThreads) out[j] = -1;
  if (tid == 0 && count) count[bt] = cnt;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
size_t prefill_select_lds_bytes(int L) { return ((size_t)((L + 63) / 64) * 64 + 64) * 4; }

bool prefill_select_supported(const IndexerArgs& a, int topk) {
  if (!indexer_uses_mfma(a)) return false;
  if (a.dI != 64 && a.dI != 128) return false;
  if (a.L > kPrefillSelectMaxL || topk < 1) return false;
  return true;
}

template <int HT, int DI, bool FP8>
static hipError_t launch_pfs(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                             hipStream_t st) {
  const size_t lds = prefill_select_lds_bytes(a.L);
  static bool attr_set = false;  // the opt-in is per kernel and process-wide
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)pf_select_kernel<HT, DI, FP8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)prefill_select_lds_bytes(kPrefillSelectMaxL));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)a.T, (unsigned)a.B);
  pf_select_kernel<HT, DI, FP8><<<grid, kPfsThreads, lds, st>>>(
      (const uint16_t*)a.q, a.w, (const uint8_t*)a.k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L, topk,
      idx, count);
  return hipGetLastError();
}

template <int DI, bool FP8>
static hipError_t pfs_dispatch_ht(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                                  hipStream_t st) {
  switch (a.HI / 16) {
    case 1: return launch_pfs<1, DI, FP8>(a, topk, idx, count, st);
    case 2: return launch_pfs<2, DI, FP8>(a, topk, idx, count, st);
    case 4: return launch_pfs<4, DI, FP8>(a, topk, idx, count, st);
    case 8: return launch_pfs<8, DI, FP8>(a, topk, idx, count, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_select(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                                 hipStream_t st) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  const bool fp8 = a.k_dtype == SA_FP8_E4M3;
  if (a.dI == 128)
    return fp8 ? pfs_dispatch_ht<128, true>(a, topk, idx, count, st)
               : pfs_dispatch_ht<128, false>(a, topk, idx, count, st);
  return fp8 ? pfs_dispatch_ht<64, true>(a, topk, idx, count, st)
             : pfs_dispatch_ht<64, false>(a, topk, idx, count, st);
}

}  // namespace sa
