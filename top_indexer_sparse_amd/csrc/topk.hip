// topk.hip -- per-query Top-K select on gfx950, no full sort.
//
// Selection rule ("Sparse Attention 数学学习笔记" §9; "MLA 与稀疏注意力" DSA
// section, the selected-position helper ordering by (-score, position)):
// exactly min(k, #candidates) candidates; larger scores first; equal scores
// to the lower position.  Candidates are the positions s < lim (kv_len and
// the causal bound q_pos) whose score is neither NaN nor -inf.
//
// Method (one 1024-thread work-group per row, row staged in LDS):
//  1. Each score becomes an order-preserving 32-bit key (-0 folded onto +0;
//     NaN and -inf become key 0, "not a candidate").  Thread i owns the 32
//     consecutive positions [32 i, 32 i + 32) (LDS padded by one word per 32,
//     so the segment reads are bank-conflict free) and keeps them in registers.
//  2. tau = the k-th largest key: a sign pre-pass (block count of positive
//     keys), then three radix passes over key bits 30..20, 19..9 and 8..0, each
//     a 2048-bin LDS histogram of the keys that still match the prefix, and a
//     block scan from the top bin down to the bin that holds rank k.
//  3. One block scan of packed (greater-than-tau, equal-to-tau) counts gives
//     every thread its output slot and its rank among the ties, so keys > tau
//     and the first k - count(> tau) keys == tau are written in ascending
//     position order.
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
template <bool MERGE>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkRowArgs a) {
  __shared__ uint32_t keys[kTkRow + kTkRow / kTkSeg];
  __shared__ int hist[kTkBins];
  __shared__ int red[kTkWaves];
  __shared__ int found[2];

  const int tid = threadIdx.x, lane = lane_id();
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

  // ---- stage keys: coalesced loads, padded LDS, then own segment to regs ----
  // all 32 loads of a thread are issued before the first store (the loop is
  // unrolled over a compile-time bound), so their latencies overlap
  const int nround = (n + kTkSeg - 1) / kTkSeg * kTkSeg;
  {
    float sv[kTkSeg];
#pragma unroll
    for (int i = 0; i < kTkSeg; ++i) {
      const int v = tid + kTkThreads * i;
      sv[i] = v < n ? src[v] : __builtin_nanf("");
    }
#pragma unroll
    for (int i = 0; i < kTkSeg; ++i) {
      const int v = tid + kTkThreads * i;
      if (v < nround) keys[v + v / kTkSeg] = score_key(sv[i]);
    }
  }
  __syncthreads();
  uint32_t kr[kTkSeg];
  const bool has_seg = tid * kTkSeg < n;
#pragma unroll
  for (int j = 0; j < kTkSeg; ++j) kr[j] = has_seg ? keys[tid * (kTkSeg + 1) + j] : 0u;

  // ---- counts: valid, positive ----
  int nv = 0, np = 0;
#pragma unroll
  for (int j = 0; j < kTkSeg; ++j) {
    nv += kr[j] != 0u;
    np += kr[j] >= 0x80000000u;
  }
  const int n_valid = block_sum(nv, red);
  const int n_pos = block_sum(np, red);

  // ---- tau = k-th largest key ----
  uint32_t tau = 0u;   // keys > tau are all selected
  int need_eq = 0;     // how many keys == tau to take (lowest positions)
  if (n_valid > k) {
    uint32_t prefix, pmask = 0x80000000u;
    int krem;
    if (n_pos >= k) {
      prefix = 0x80000000u;
      krem = k;
    } else {
      prefix = 0u;
      krem = k - n_pos;
    }
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
      const int sh = p == 0 ? 20 : (p == 1 ? 9 : 0);  // bits 30..20, 19..9, 8..0
      const uint32_t dmask = p == 2 ? 0x1ffu : 0x7ffu;
      for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kTkSeg; ++j) {
        const uint32_t key = kr[j];
        const bool match = key != 0u && (key & pmask) == prefix;
        const int digit = (int)((key >> sh) & dmask);
        const uint64_t m = __ballot(match);
        if (m == 0) continue;
        // all matching lanes share one digit (ties, narrow ranges): one atomic
        const int lead = __ffsll((unsigned long long)m) - 1;
        const int d0 = __shfl(digit, lead);
        const uint64_t same = __ballot(match && digit == d0);
        if (same == m) {
          if (lane == lead) atomicAdd(&hist[d0], __popcll(m));
        } else if (match) {
          atomicAdd(&hist[digit], 1);
        }
      }
      __syncthreads();
      // thread t covers bins hi = 2047 - 2t and lo = 2046 - 2t (top first)
      const int bhi = kTkBins - 1 - 2 * tid, blo = bhi - 1;
      const int hhi = hist[bhi], hlo = hist[blo];
      int total;
      const int incl = block_scan_incl(hhi + hlo, red, total);
      const int above = incl - hhi - hlo;  // matching keys in higher bins
      if (above < krem && krem <= above + hhi) {
        found[0] = bhi;
        found[1] = above;
      } else if (above + hhi < krem && krem <= above + hhi + hlo) {
        found[0] = blo;
        found[1] = above + hhi;
      }
      __syncthreads();
      prefix |= (uint32_t)found[0] << sh;
      pmask |= dmask << sh;
      krem -= found[1];
      __syncthreads();  // found[] is rewritten by the next pass
    }
    tau = prefix;
    need_eq = krem;
  }
  const int n_sel = min(k, n_valid);

  // ---- compaction in position order ----
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kTkSeg; ++j) {
    gt += kr[j] > tau;
    eq += (kr[j] == tau) & (kr[j] != 0u);
  }
  int tot;
  const int incl = block_scan_incl((gt << 16) | eq, red, tot);
  const int excl = incl - ((gt << 16) | eq);
  const int gt_before = excl >> 16, eq_before = excl & 0xffff;
  int slot = gt_before + min(eq_before, need_eq);
  int eq_rank = eq_before;
  if (gt | eq) {
#pragma unroll
    for (int j = 0; j < kTkSeg; ++j) {
      const uint32_t key = kr[j];
      bool take = key > tau;
      if (key == tau && key != 0u) {
        take = eq_rank < need_eq;
        ++eq_rank;
      }
      if (take) {
        const int v = tid * kTkSeg + j;
        out_idx[slot] = vpos ? vpos[v] : pos_base + v;
        if (out_score) out_score[slot] = key_score(key);
        ++slot;
      }
    }
  }
  for (int i = n_sel + tid; i < k; i += kTkThreads) {
    out_idx[i] = -1;
    if (out_score) out_score[i] = -INFINITY;
  }
  if (out_count && tid == 0) *out_count = n_sel;
}

static int topk_chunks(int L) { return (L + kTkRow - 1) / kTkRow; }

bool topk_supported(int L, int k) {
  if (k < 1 || k > kTopkMaxK) return false;
  const int nch = topk_chunks(L);
  return nch == 1 || (int64_t)nch * k <= kTkRow;
}

size_t topk_workspace_bytes(int B, int T, int L, int k) {
  const int nch = topk_chunks(L);
  if (nch <= 1) return 0;
  return (size_t)B * T * nch * k * (sizeof(float) + sizeof(int32_t));
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
