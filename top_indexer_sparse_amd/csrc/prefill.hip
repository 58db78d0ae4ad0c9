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

constexpr int kPfsBins = 2048;
constexpr int kPfsBinBits = 11;

// Exclusive scan over the work-group's NW waves of one int per thread.
template <int NW>
__device__ __forceinline__ int pfs_block_excl(int x, int* red, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  __syncthreads();  // red may still be read by a previous scan
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = red[i];
    before += i < wave ? v : 0;
    total += v;
  }
  return incl - x + before;
}

template <int NW>
struct PfsShared {
  uint32_t hist[kPfsBins];
  float spill[NW][16];  // scores of ring chunks past a wave's range
  int red[NW], red2[NW], red3[NW], red4[NW];
  uint32_t ured[2 * NW];
  int found[2];
};

// Steps 2 and 3 for one row of scores held in LDS, run by the whole
// work-group (NW waves).  Wave w emits positions [w span, (w+1) span) of the
// row's candidate range [0, lim).
template <int NW, bool FP8>
__device__ void pfs_select_row(uint32_t* row, int lim, int span, const float* scb, int topk,
                               int32_t* out, int32_t* count_out, PfsShared<NW>& sh) {
  constexpr int NT = 64 * NW;
  constexpr int BPT = kPfsBins / NT;  // histogram bins per thread
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;

  // ---- 2a. keys in place; candidates, smallest and largest key ----
  int nv = 0;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int s4 = 4 * tid; s4 < lim; s4 += 4 * NT) {
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
      sh.red[wave] = wnv;
      sh.ured[wave] = wmn;
      sh.ured[NW + wave] = wmx;
    }
  }
  __syncthreads();
  int nv_all = 0;
  uint32_t mn_all = 0xffffffffu, mx_all = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    nv_all += sh.red[i];
    mn_all = min(mn_all, sh.ured[i]);
    mx_all = max(mx_all, sh.ured[NW + i]);
  }

  // ---- 2b. tau and take ----
  uint32_t tau = 0u;  // select keys > tau, and the first `take` keys == tau
  int take = 0;
  if (nv_all > topk) {
    uint32_t lo = mn_all;
    const uint32_t range = mx_all - mn_all;
    const int bits = range ? 32 - __builtin_clz(range) : 0;
    int sh_bits = max(0, bits - kPfsBinBits);
    uint32_t nb = kPfsBins;  // bins of this pass: the range is [lo, lo + (nb << sh_bits))
    int r = topk;            // wanted rank, counted from the top inside the range
    for (;;) {
      for (int i = tid; i < kPfsBins; i += NT) sh.hist[i] = 0u;
      __syncthreads();
      for (int s4 = 4 * tid; s4 < lim; s4 += 4 * NT) {
        const uintx4 v = *(const uintx4*)&row[s4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = v[e];
          if (s4 + e < lim && key >= lo) {
            const uint32_t d = (key - lo) >> sh_bits;
            if (d < nb) atomicAdd(&sh.hist[d], 1u);
          }
        }
      }
      __syncthreads();
      // thread i owns bins 2047 - BPT i down to 2048 - BPT (i + 1) (top first)
      const int top = kPfsBins - 1 - BPT * tid;
      int c = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) c += (int)sh.hist[top - j];
      int total;
      int acc = pfs_block_excl<NW>(c, sh.red2, total);  // keys in higher bins
      if (acc < r && r <= acc + c) {
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          const int hb = (int)sh.hist[top - j];
          if (acc < r && r <= acc + hb) {
            sh.found[0] = top - j;
            sh.found[1] = acc;
          }
          acc += hb;
        }
      }
      __syncthreads();
      const int bin = sh.found[0], above = sh.found[1];
      r -= above;
      lo += (uint32_t)bin << sh_bits;
      if (sh_bits == 0) {
        tau = lo;
        take = r;
        break;
      }
      // the next pass splits this bin, 2^sh_bits keys wide, into at most 2048 bins
      const int sh_next = max(0, sh_bits - kPfsBinBits);
      nb = 1u << (sh_bits - sh_next);
      sh_bits = sh_next;
    }
  }
  const int cnt = min(nv_all, topk);

  // ---- 3. emit in position order ----
  const int s_begin = wave * span;
  const int v_end = min(s_begin + span, lim);
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
      sh.red3[wave] = wgt;
      sh.red4[wave] = weq;
    }
  }
  __syncthreads();
  int base = 0, eq_before = 0;
  for (int i = 0; i < wave; ++i) {
    const int ti = min(max(take - eq_before, 0), sh.red4[i]);  // ties wave i takes
    base += sh.red3[i] + ti;
    eq_before += sh.red4[i];
  }
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
  for (int j = cnt + tid; j < topk; j += NT) out[j] = -1;
  if (tid == 0 && count_out) *count_out = cnt;
}

// QPW query rows per work-group of 4 QPW waves.  With QPW = 2 (two adjacent
// queries) every key chunk a wave loads feeds both queries' products, which
// halves the key traffic into the CU; the two rows then take 2 x 4 bytes per
// position of LDS, so QPW = 2 serves L <= 16384 and HI <= 64.
template <int HT, int DI, bool FP8, int QPW>
__global__ __launch_bounds__(256 * QPW) void pf_select_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, int rowwords, int topk, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  constexpr int NW = 4 * QPW;
  constexpr int HI = 16 * HT;
  constexpr int ROWB = FP8 ? DI : 2 * DI;
  // ring depth: as the decode scores for one query; two queries' operands
  // leave room for four chunks
  constexpr int R = QPW == 2 ? 4 : (16 * HT * DI >= 16384 ? 4 : 8);
  extern __shared__ uintx4 row_v[];  // QPW rows of rowwords words
  uint32_t* rows = (uint32_t*)row_v;
  __shared__ PfsShared<NW> sh;

  const int npair = (T + QPW - 1) / QPW;
  const int t0 = QPW * (npair - 1 - (int)blockIdx.x);  // longest rows first
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int lim[QPW];
  int64_t bt[QPW];
  int lim_max = 0;
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int t = min(t0 + i, T - 1);  // a missing second query repeats the first
    bt[i] = (int64_t)b * T + t;
    lim[i] = candidate_limit(q_pos, kv_len, b, bt[i], L);
    lim_max = max(lim_max, lim[i]);
  }
  // wave parts: multiples of 16 positions
  const int span = ((lim_max + NW - 1) / NW + 15) & ~15;
  const int s_begin = wave * span;
  const int v_end = min(s_begin + span, lim_max);

  // ---- 1. scores into the LDS rows ----
  if (s_begin < v_end) {  // wave-uniform
    const uint8_t* kb = k + (int64_t)b * L * ROWB;
    const int nch = (v_end - s_begin + 15) / 16;
    auto row_of = [&](int c) {
      return kb + (int64_t)min(s_begin + 16 * c + n, v_end - 1) * ROWB;
    };
    QueryRegs<HT, DI, FP8> qr[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) qr[i].load(q + bt[i] * HI * DI, w + bt[i] * HI, lane);
    // the queries have landed before the ring starts, so that the ring's
    // waits count only its own loads
    wait_vmcnt<0>();
    KeyChunk<DI, FP8> ring[R];
    for (int c0 = -R; c0 < nch; c0 += R) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = c0 + i;
        if (c0 >= 0) {  // uniform; chunks past nch are computed and dropped
          float sc[QPW];
          if constexpr (QPW == 2)
            score_pair(qr[0], qr[1], ring[i], sc[0], sc[1]);
          else
            sc[0] = qr[0].score(ring[i]);
#pragma unroll
          for (int qi = 0; qi < QPW; ++qi) {
            float* dst = c < nch ? (float*)rows + qi * rowwords + s_begin + 16 * c
                                 : sh.spill[wave];
            dst[n] = sc[qi];  // the four lane groups write the same value
          }
        }
        ring[i].load(row_of(c + R), g);
      }
    }
  }
  __syncthreads();

  // ---- 2, 3. one row after the other, by the whole work-group ----
  const float* scb = FP8 ? kscale + (int64_t)b * L : nullptr;
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    if (t0 + qi >= T) break;  // uniform
    if (qi > 0) __syncthreads();
    pfs_select_row<NW, FP8>(rows + qi * rowwords, lim[qi], span, scb, topk,
                            idx + bt[qi] * topk, count ? count + bt[qi] : nullptr, sh);
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static int pfs_rowwords(int L) { return (L + 63) / 64 * 64 + 64; }

bool prefill_select_supported(const IndexerArgs& a, int topk) {
  if (!indexer_uses_mfma(a)) return false;
  if (a.dI != 64 && a.dI != 128) return false;
  if (a.L > kPrefillSelectMaxL || topk < 1) return false;
  return true;
}

template <int HT, int DI, bool FP8, int QPW>
static hipError_t launch_pfs(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                             hipStream_t st) {
  const int rowwords = pfs_rowwords(a.L);
  const size_t lds = (size_t)QPW * rowwords * 4;
  // the opt-in to more than 64 KB of dynamic LDS, set on every launch (a host
  // call; it keeps no per-device or per-thread state here)
  const int most = QPW * pfs_rowwords(QPW == 2 ? kPrefillSelectPairMaxL : kPrefillSelectMaxL) * 4;
  hipError_t e = hipFuncSetAttribute((const void*)pf_select_kernel<HT, DI, FP8, QPW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, most);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.T + QPW - 1) / QPW), (unsigned)a.B);
  pf_select_kernel<HT, DI, FP8, QPW><<<grid, 256 * QPW, lds, st>>>(
      (const uint16_t*)a.q, a.w, (const uint8_t*)a.k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L,
      rowwords, topk, idx, count);
  return hipGetLastError();
}

// two queries per work-group where both rows fit and the two query blocks fit
// the registers (HI <= 64); one otherwise
template <int HT, int DI, bool FP8>
static hipError_t launch_pfs_q(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                               hipStream_t st) {
  if constexpr (HT <= 4)
    if (a.L <= kPrefillSelectPairMaxL && a.T >= 2)
      return launch_pfs<HT, DI, FP8, 2>(a, topk, idx, count, st);
  return launch_pfs<HT, DI, FP8, 1>(a, topk, idx, count, st);
}

template <int DI, bool FP8>
static hipError_t pfs_dispatch_ht(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                                  hipStream_t st) {
  switch (a.HI / 16) {
    case 1: return launch_pfs_q<1, DI, FP8>(a, topk, idx, count, st);
    case 2: return launch_pfs_q<2, DI, FP8>(a, topk, idx, count, st);
    case 4: return launch_pfs_q<4, DI, FP8>(a, topk, idx, count, st);
    case 8: return launch_pfs_q<8, DI, FP8>(a, topk, idx, count, st);
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
