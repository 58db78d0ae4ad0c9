// block_sparse.hip -- GQA block-sparse decode on gfx950.
//
// The block-selection variant ("第 11 章 稀疏注意力" §12.5-§12.6: attend to
// whole contiguous blocks, chosen by the inner product of the query with a
// block representative, the mean of the block's keys; sink tokens and a
// sliding window are always kept, "Sparse Attention 数学学习笔记" §4):
//   krep[b,n,g,:] = mean_{j < blk} k[b, n blk + j, g, :]      (complete blocks)
//   per query head h (KV head g = h / (Hq / Hkv)):
//     block score n = q[b,h,:] . krep[b,n,g,:]
//     S_h = the nsel best blocks (ties to the lower block), as token ranges,
//           union [0, n_sink), union [L - n_win, L)
//     out[b,h,:] = softmax_{s in S_h}(sm_scale q . k_s) weighted sum of v_s
//
// Three kernels:
//  * block_pool_kernel: one work-group per (block, sequence); 8-byte bf16
//    loads, fp32 sums, the mean stored as bf16 (round to nearest even), the
//    keys' own type.  A cache-maintenance step (the pooled keys of a block
//    change only when the block fills), not part of a decode step.
//  * block_score_kernel: one work-group per (64 blocks, KV head, sequence).
//    Each pooled-key row (256 bytes) is read once, coalesced, by half a wave
//    (8 bytes per lane, widened to fp32) and scored against every query head of the KV group
//    (or, with a shared choice, their sum); the per-lane partial dot products
//    are summed over the half wave.  Scores go to the workspace, [B, Hq, nblk].
//  * block_attn_kernel: one work-group per (query head, sequence).  It first
//    chooses the head's blocks from its scores: (score key, inverted block
//    index) keys, so that one maximum search orders by score with ties to the
//    lower block; the nsel largest by repeated wave maxima (per wave, then
//    over the four waves' survivors), in ascending block order.  The visible
//    ranges (sinks, chosen blocks, window) are merged into disjoint ascending
//    ranges; the four waves take 64-token chunks in turn.  Sixteen lanes share
//    each key and value row (16 bytes each, four rows per load instruction),
//    with an online softmax per wave and a final merge.
#include "common.hpp"
#include "launch.hpp"

namespace sa {

constexpr int kBlkD = 128;            // head dim of the compiled set
constexpr int kBlkMaxBlocks = 8192;   // L / blk
constexpr int kBlkMaxSel = 64;        // nsel
constexpr int kBlkMaxGroup = 8;       // Hq / Hkv
constexpr int kBlkMaxRanges = kBlkMaxSel + 2;

bool block_supported(const BlockArgs& a) {
  const int G = a.Hq / a.Hkv;
  return a.d == kBlkD && (a.blk == 32 || a.blk == 64 || a.blk == 128) &&
         (G == 1 || G == 2 || G == 4 || G == kBlkMaxGroup) && a.nsel >= 1 && a.nsel <= kBlkMaxSel &&
         a.L / a.blk <= kBlkMaxBlocks;
}

// workspace: block scores [B, Hq, L / blk] fp32
size_t block_workspace_bytes(int B, int Hq, int L, int nsel, int Hkv, int d, int blk) {
  (void)Hkv;
  (void)d;
  if (blk < 1 || B < 0 || Hq < 1 || nsel < 1 || L < 0) return 0;
  return (size_t)B * Hq * (L / blk) * sizeof(float);
}

// ---------------------------------------------------------------------------
// pooled block keys
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_pool_kernel(const uint16_t* __restrict__ k, int L,
                                                         int E, int blk,
                                                         uint16_t* __restrict__ krep) {
  const int n = blockIdx.x, b = blockIdx.y;
  const int nblk = L / blk;
  const uint16_t* src = k + ((int64_t)b * L + (int64_t)n * blk) * E;
  uint16_t* dst = krep + ((int64_t)b * nblk + n) * E;
  const float inv = 1.f / (float)blk;
  for (int e = 4 * threadIdx.x; e < E; e += 4 * 256) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
    for (int j = 0; j < blk; ++j) {
      const uint2 u = *(const uint2*)(src + (int64_t)j * E + e);
      a0 += bf16_lo(u.x);
      a1 += bf16_hi(u.x);
      a2 += bf16_lo(u.y);
      a3 += bf16_hi(u.y);
    }
    // the fp32 mean, rounded to nearest even bf16
    *(uint2*)(dst + e) = make_uint2(pack_bf16x2_rne(a0 * inv, a1 * inv), pack_bf16x2_rne(a2 * inv, a3 * inv));
  }
}

// ---------------------------------------------------------------------------
// block scores and choice
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t blk_score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;                    // -0 == +0
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct BlockScoreArgs {
  const uint16_t* q;    // [B, Hq, d]
  const uint16_t* krep;  // [B, nblk, Hkv, d] bf16
  int Hq, Hkv, nblk;
  int shared;           // score with the sum of the KV group's queries
  float* scores;        // [B, Hq, nblk] (workspace)
};

constexpr int kScoreBlocks = 64;  // blocks per scoring work-group (16 per wave)

// DPP lane moves (no LDS round trip): quad permutations and the row mirrors.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
// Sum over the 32 lanes of each half wave, in every lane: quad swaps, the
// half-row and row mirrors (sum of 16), then rows 0 and 1 (2 and 3) swapped
// by v_permlane16_swap.  Needs all 64 lanes active.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_f32<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// G query heads per KV head.  Lane l of half-wave e holds dims 4 (l % 32) ..
// +3 of each query; wave w scores blocks n0 + 16 w + 2 i + e, i < 8, all its
// 16-byte loads issued before the first product.
template <int G>
__global__ __launch_bounds__(256) void block_score_kernel(BlockScoreArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int e = lane >> 5, l = lane & 31;
  const int nblk = a.nblk;
  float qv[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint2 u = *(const uint2*)(a.q + ((int64_t)b * a.Hq + g * G + hh) * kBlkD + 4 * l);
    qv[hh][0] = bf16_lo(u.x);
    qv[hh][1] = bf16_hi(u.x);
    qv[hh][2] = bf16_lo(u.y);
    qv[hh][3] = bf16_hi(u.y);
  }
  if (a.shared) {  // the group's summed query, heads in order
#pragma unroll
    for (int hh = 1; hh < G; ++hh)
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[0][c] += qv[hh][c];
  }
  const int n0 = blockIdx.x * kScoreBlocks + 16 * wave + e;
  uint2 kv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = min(n0 + 2 * i, nblk - 1);
    kv[i] = *(const uint2*)(a.krep + (((int64_t)b * nblk + n) * a.Hkv + g) * kBlkD + 4 * l);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = n0 + 2 * i;
    float p[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      p[hh] = 0.f;
      if (a.shared && hh > 0) continue;  // uniform: one summed query
      float acc = bf16_lo(kv[i].x) * qv[hh][0];
      acc = fmaf(bf16_hi(kv[i].x), qv[hh][1], acc);
      acc = fmaf(bf16_lo(kv[i].y), qv[hh][2], acc);
      acc = fmaf(bf16_hi(kv[i].y), qv[hh][3], acc);
      p[hh] = half_wave_sum(acc);
    }
    if (n < nblk && l < G) {  // lane l of the half wave writes head g G + l
      float v = p[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh)
        if (!a.shared && l == hh) v = p[hh];
      a.scores[((int64_t)b * a.Hq + g * G + l) * nblk + n] = v;
    }
  }
}

struct BlockSelArgs {
  const float* scores;  // [B, Hq, nblk]
  int Hq, nblk, nsel;
  int32_t* blocks_out;  // [B, Hq, nsel] or null
};

// Largest 64-bit key over the wave, in every lane: quad swaps and row
// mirrors give each row of 16 its maximum (DPP, both halves with the same
// control), then gfx950's permlane16 / permlane32 swaps exchange rows (each
// swap hands a lane the pair {v[l], v[l ^ 16]}, then {v[l], v[l ^ 32]}, the
// two 32-bit halves taken from the same lanes).  Needs all 64 lanes active.
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xb1>(v));
  v = max_u64(v, dpp_u64<0x4e>(v));
  v = max_u64(v, dpp_u64<0x141>(v));
  v = max_u64(v, dpp_u64<0x140>(v));
  {
    const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    v = max_u64(((uint64_t)(uint32_t)h[0] << 32) | (uint32_t)l[0],
                ((uint64_t)(uint32_t)h[1] << 32) | (uint32_t)l[1]);
  }
  {
    const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    v = max_u64(((uint64_t)(uint32_t)h[0] << 32) | (uint32_t)l[0],
                ((uint64_t)(uint32_t)h[1] << 32) | (uint32_t)l[1]);
  }
  return v;
}

constexpr int kSelMaxPerLane = kBlkMaxBlocks / 256;  // blocks per thread, at most

// The nsel highest blocks of (sequence b, query head h), run by a 256-thread
// work-group at the start of the attention.  Keys (score key << 32 | ~block)
// order blocks by score, ties to the lower block, so the selection is a
// plain maximum search: each wave takes the nsel largest keys of its share
// (nsel rounds of a wave maximum, the winner's lane retiring it), one wave
// then takes the nsel largest of the 4 nsel survivors the same way.  The
// chosen blocks land in chs[0, nsel) in ascending order, -1 padded (and in
// blocks_out when given); the function ends with a barrier.
template <int KPL>  // keys per thread: blocks n = tid + 256 r, r < KPL
__device__ __forceinline__ void block_choose(const BlockSelArgs& a, int b, int h, int* chs,
                                             uint64_t (*cand)[kBlkMaxSel], int* pick) {
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int nblk = a.nblk;
  const float* srow = a.scores + ((int64_t)b * a.Hq + h) * nblk;
  // All loads are issued before any is used (clamped addresses, masked keys).
  float sv[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) sv[r] = nblk > 0 ? srow[min(tid + 256 * r, nblk - 1)] : 0.f;
  uint64_t key[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int n = tid + 256 * r;
    key[r] = n < nblk ? ((uint64_t)blk_score_key(sv[r]) << 32) | (uint32_t)~(uint32_t)n : 0ull;
  }
  // this wave's nsel largest keys
  const int m = min(nblk, a.nsel);
  for (int i = 0; i < m; ++i) {
    uint64_t best = 0ull;
#pragma unroll
    for (int r = 0; r < KPL; ++r) best = key[r] > best ? key[r] : best;
    const uint64_t w = wave_max_u64(best);
    if (lane == 0) cand[wave][i] = w;
    // the owner retires the winning key (keys are distinct; a zero winner
    // leaves only zero keys, which stay zero)
#pragma unroll
    for (int r = 0; r < KPL; ++r) key[r] = key[r] == w ? 0ull : key[r];
  }
  __syncthreads();
  if (wave == 0) {
    // the nsel largest of the 4 m survivors: lane l holds candidates l, l+64..
    uint64_t c4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = lane + 64 * r;  // candidate j = (wave j / m, rank j % m)
      c4[r] = j < 4 * m ? cand[j / m][j % m] : 0ull;
    }
    for (int i = 0; i < m; ++i) {
      uint64_t best = 0ull;
#pragma unroll
      for (int r = 0; r < 4; ++r) best = c4[r] > best ? c4[r] : best;
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) pick[i] = (int)~(uint32_t)w;
#pragma unroll
      for (int r = 0; r < 4; ++r) c4[r] = c4[r] == w ? 0ull : c4[r];
    }
  }
  __syncthreads();
  // ascending order: rank of each chosen block among the chosen (m <= 64)
  int32_t* bo = a.blocks_out ? a.blocks_out + ((int64_t)b * a.Hq + h) * a.nsel : nullptr;
  if (tid < a.nsel) {
    int val = -1, rank = tid;
    if (tid < m) {
      const int mine = pick[tid];
      rank = 0;
      for (int i = 0; i < m; ++i) rank += pick[i] < mine;
      val = mine;
    }
    chs[rank] = val;
    if (bo) bo[rank] = val;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// attention over the visible set
// ---------------------------------------------------------------------------
struct BlockAttnArgs {
  const uint16_t* q;  // [B, Hq, d]
  const uint16_t* k;  // [B, L, Hkv, d]
  const uint16_t* v;
  BlockSelArgs sel;   // the block scores, and where the choice is reported
  int B, L, Hq, Hkv, blk, nsel, n_sink, n_win;
  float scale_log2;
  float* out;  // [B, Hq, d]
};

// Sum over the 16 lanes of each row (quad swaps and the row mirrors), in
// every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xb1>(v);
  v += dpp_f32<0x4e>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

template <int KPL>
__global__ __launch_bounds__(256) void block_attn_kernel(BlockAttnArgs a) {
  __shared__ uint64_t cand[4][kBlkMaxSel];
  __shared__ int pick[kBlkMaxSel];
  __shared__ int rs[kBlkMaxRanges], re[kBlkMaxRanges], rcum[kBlkMaxRanges + 1];
  __shared__ int st[kBlkMaxRanges], en[kBlkMaxRanges];  // unsorted ranges
  __shared__ int s_nr;
  __shared__ int chs[kBlkMaxSel];
  __shared__ int tb[4][64];
  __shared__ float wm[4], wl[4];
  __shared__ float wo[4][kBlkD];
  // Work-groups go to the eight XCDs in turn (linear id mod 8).  Item
  // w = (sequence, head) is placed so that each XCD takes a contiguous run
  // of items: a KV group's query heads then share one L2, where the keys and
  // values they have in common (sinks, window, blocks chosen alike) are read
  // from HBM once.
  const int n_items = a.Hq * a.B, id = blockIdx.x;
  const int w_item = n_items % 8 == 0 ? (id % 8) * (n_items / 8) + id / 8 : id;
  const int h = w_item % a.Hq, b = w_item / a.Hq, tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int g = h / (a.Hq / a.Hkv);
  const int L = a.L;

  // ---- the chosen blocks, then the visible ranges: sinks, chosen blocks,
  // window -> disjoint, ascending
  block_choose<KPL>(a.sel, b, h, chs, cand, pick);
  if (tid == 0) {
    int n = 0;
    if (a.n_sink > 0) {
      st[n] = 0;
      en[n++] = min(a.n_sink, L);
    }
    for (int i = 0; i < a.nsel; ++i) {
      const int c = chs[i];
      if (c < 0) break;
      st[n] = c * a.blk;
      en[n++] = c * a.blk + a.blk;
    }
    if (a.n_win > 0) {
      st[n] = max(0, L - a.n_win);
      en[n++] = L;
    }
    for (int i = 1; i < n; ++i) {  // insertion sort by start (n <= 66)
      const int s0 = st[i], e0 = en[i];
      int j = i - 1;
      while (j >= 0 && st[j] > s0) {
        st[j + 1] = st[j];
        en[j + 1] = en[j];
        --j;
      }
      st[j + 1] = s0;
      en[j + 1] = e0;
    }
    int nr = 0, cum = 0;
    for (int i = 0; i < n; ++i) {
      if (nr > 0 && st[i] <= re[nr - 1]) {
        if (en[i] > re[nr - 1]) {
          cum += en[i] - re[nr - 1];
          re[nr - 1] = en[i];
        }
      } else {
        rs[nr] = st[i];
        re[nr] = en[i];
        rcum[nr] = cum;
        cum += en[i] - st[i];
        ++nr;
      }
    }
    rcum[nr] = cum;
    s_nr = nr;
  }
  // Lane (r, j) = (lane / 16, lane % 16) takes dims 8 j .. 8 j + 7 of slot
  // 4 i + r, i < 16, of each 64-slot chunk: every key or value row (256
  // bytes) is read by 16 lanes with one 16-byte load each, four rows per
  // instruction.  A score is summed over its 16 lanes by DPP moves, so the
  // row's lanes all hold it; the softmax state and the value sums stay in
  // registers, and the four rows' partial sums are added at the end.
  const int r4 = lane >> 4, j16 = lane & 15;
  float qd[8];
  {
    const uint4 u = *(const uint4*)(a.q + ((int64_t)b * a.Hq + h) * kBlkD + 8 * j16);
    qd[0] = bf16_lo(u.x);
    qd[1] = bf16_hi(u.x);
    qd[2] = bf16_lo(u.y);
    qd[3] = bf16_hi(u.y);
    qd[4] = bf16_lo(u.z);
    qd[5] = bf16_hi(u.z);
    qd[6] = bf16_lo(u.w);
    qd[7] = bf16_hi(u.w);
  }
  __syncthreads();
  const int nr = s_nr, ntok = rcum[nr];
  const int64_t row_stride = (int64_t)a.Hkv * kBlkD;  // elements between tokens
  const uint16_t* kb = a.k + (int64_t)b * L * row_stride + (int64_t)g * kBlkD + 8 * j16;
  const uint16_t* vb = a.v + (int64_t)b * L * row_stride + (int64_t)g * kBlkD + 8 * j16;

  float m_w = -INFINITY, l_w = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // dims 8 j .. + 7, this row's slots
  for (int c = wave; 64 * c < ntok; c += 4) {
    {  // token of slot 64 c + lane (binary search over the ranges' offsets)
      const int t = 64 * c + lane;
      int tok = 0;
      if (t < ntok) {
        int lo = 0, hi = nr - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (rcum[mid] <= t) lo = mid;
          else hi = mid - 1;
        }
        tok = rs[lo] + (t - rcum[lo]);
      }
      tb[wave][lane] = tok;  // past the end: token 0 (read, then masked)
    }
    __builtin_amdgcn_wave_barrier();
    int tokr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) tokr[i] = tb[wave][4 * i + r4];
    uint4 kr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kr[i] = *(const uint4*)(kb + (int64_t)tokr[i] * row_stride);
    float sc[16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = qd[0] * bf16_lo(kr[i].x);
      acc = fmaf(qd[1], bf16_hi(kr[i].x), acc);
      acc = fmaf(qd[2], bf16_lo(kr[i].y), acc);
      acc = fmaf(qd[3], bf16_hi(kr[i].y), acc);
      acc = fmaf(qd[4], bf16_lo(kr[i].z), acc);
      acc = fmaf(qd[5], bf16_hi(kr[i].z), acc);
      acc = fmaf(qd[6], bf16_lo(kr[i].w), acc);
      acc = fmaf(qd[7], bf16_hi(kr[i].w), acc);
      acc = row16_sum(acc);
      sc[i] = 64 * c + 4 * i + r4 < ntok ? acc * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    uint4 vr[16];  // value rows, loaded while the softmax runs
#pragma unroll
    for (int i = 0; i < 16; ++i) vr[i] = *(const uint4*)(vb + (int64_t)tokr[i] * row_stride);
    const float cmax = max_over_lane_groups_vx(mx);  // finite: the chunk has a valid slot
    const float m_new = fmaxf(m_w, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m_w - m_new);  // 0 at the first chunk
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);  // 0 for masked slots
      psum += p;
      o[0] = fmaf(p, bf16_lo(vr[i].x), o[0]);
      o[1] = fmaf(p, bf16_hi(vr[i].x), o[1]);
      o[2] = fmaf(p, bf16_lo(vr[i].y), o[2]);
      o[3] = fmaf(p, bf16_hi(vr[i].y), o[3]);
      o[4] = fmaf(p, bf16_lo(vr[i].z), o[4]);
      o[5] = fmaf(p, bf16_hi(vr[i].z), o[5]);
      o[6] = fmaf(p, bf16_lo(vr[i].w), o[6]);
      o[7] = fmaf(p, bf16_hi(vr[i].w), o[7]);
    }
    l_w = l_w * alpha + sum_over_lane_groups_vx(psum);
    m_w = m_new;
    __builtin_amdgcn_wave_barrier();  // tb is rewritten by the next chunk
  }
  // ---- the four rows' partial value sums, then merge the four waves' (m, l, o)
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = sum_over_lane_groups_vx(o[e]);
  if (lane == 0) {
    wm[wave] = m_w;
    wl[wave] = l_w;
  }
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wo[wave][8 * lane + e] = o[e];
  }
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w]);
    float den = 0.f, n0 = 0.f, n1 = 0.f;
    for (int w = 0; w < 4; ++w) {
      if (wm[w] == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(wm[w] - M);
      den += e * wl[w];
      n0 += e * wo[w][2 * lane];
      n1 += e * wo[w][2 * lane + 1];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    float* out = a.out + ((int64_t)b * a.Hq + h) * kBlkD;
    out[2 * lane] = n0 * inv;
    out[2 * lane + 1] = n1 * inv;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_block_pool(const void* k, int B, int L, int Hkv, int d, int blk, void* krep,
                             hipStream_t st) {
  const int nblk = L / blk;
  if (B == 0 || nblk == 0) return hipSuccess;
  block_pool_kernel<<<dim3(nblk, B), 256, 0, st>>>((const uint16_t*)k, L, Hkv * d, blk,
                                                   (uint16_t*)krep);
  return hipGetLastError();
}

hipError_t launch_block_decode(const BlockArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int nblk = a.L / a.blk;
  float* scores = (float*)a.ws;
  if (nblk > 0) {
    BlockScoreArgs c{};
    c.q = (const uint16_t*)a.q;
    c.krep = (const uint16_t*)a.krep;
    c.Hq = a.Hq;
    c.Hkv = a.Hkv;
    c.nblk = nblk;
    c.shared = a.shared_choice;
    c.scores = scores;
    const dim3 grid((unsigned)((nblk + kScoreBlocks - 1) / kScoreBlocks), (unsigned)a.Hkv,
                    (unsigned)a.B);
    switch (a.Hq / a.Hkv) {
      case 1: block_score_kernel<1><<<grid, 256, 0, st>>>(c); break;
      case 2: block_score_kernel<2><<<grid, 256, 0, st>>>(c); break;
      case 4: block_score_kernel<4><<<grid, 256, 0, st>>>(c); break;
      default: block_score_kernel<8><<<grid, 256, 0, st>>>(c); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BlockAttnArgs t{};
  t.sel.scores = scores;
  t.sel.Hq = a.Hq;
  t.sel.nblk = nblk;
  t.sel.nsel = a.nsel;
  t.sel.blocks_out = a.blocks_out;
  t.q = (const uint16_t*)a.q;
  t.k = (const uint16_t*)a.k;
  t.v = (const uint16_t*)a.v;
  t.B = a.B;
  t.L = a.L;
  t.Hq = a.Hq;
  t.Hkv = a.Hkv;
  t.blk = a.blk;
  t.nsel = a.nsel;
  t.n_sink = a.n_sink;
  t.n_win = a.n_win;
  t.scale_log2 = a.sm_scale * kLog2e;
  t.out = a.out;
  const dim3 grid((unsigned)(a.Hq * a.B));
  if (nblk <= 256 * 4)
    block_attn_kernel<4><<<grid, 256, 0, st>>>(t);
  else if (nblk <= 256 * 8)
    block_attn_kernel<8><<<grid, 256, 0, st>>>(t);
  else if (nblk <= 256 * 16)
    block_attn_kernel<16><<<grid, 256, 0, st>>>(t);
  else
    block_attn_kernel<kSelMaxPerLane><<<grid, 256, 0, st>>>(t);
  return hipGetLastError();
}

}  // namespace sa
