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
//    loads, fp32 sums.  A cache-maintenance step (the pooled keys of a block
//    change only when the block fills), not part of a decode step.
//  * block_score_kernel: one work-group per (64 blocks, KV head, sequence).
//    Each pooled-key row (512 bytes) is read once, coalesced, by half a wave
//    (16 bytes per lane) and scored against every query head of the KV group
//    (or, with a shared choice, their sum); the per-lane partial dot products
//    are summed over the half wave.  Scores go to the workspace, [B, Hq, nblk].
//  * block_select_kernel: one work-group per (query head, sequence).  Block
//    scores as (score key, inverted block index) keys, so that one maximum
//    search orders by score with ties to the lower block; the nsel largest by
//    repeated wave maxima (per wave, then over the four waves' survivors),
//    written in ascending block order.
//  * block_attn_kernel: one work-group per (query head, sequence).  The
//    visible ranges (sinks, chosen blocks, window) are merged into disjoint
//    ascending ranges; the four waves take 64-token chunks in turn: lane =
//    token for q . k (the key row is one lane's 256 contiguous bytes), lane =
//    dimension pair for the value sum (the value row is one coalesced 256-byte
//    load per token), with an online softmax per wave and a final merge.
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
         (G == 1 || G == 2 || G == 4 || G == 8) && a.nsel >= 1 && a.nsel <= kBlkMaxSel &&
         a.L / a.blk <= kBlkMaxBlocks;
}

// workspace: chosen blocks [B, Hq, nsel] int32 | block scores [B, Hq, L / blk] fp32
static size_t block_chosen_bytes(int B, int Hq, int nsel) {
  return ((size_t)B * Hq * nsel * sizeof(int32_t) + 255) & ~(size_t)255;
}
size_t block_workspace_bytes(int B, int Hq, int L, int nsel, int Hkv, int d, int blk) {
  (void)Hkv;
  (void)d;
  if (blk < 1 || B < 0 || Hq < 1 || nsel < 1 || L < 0) return 0;
  return block_chosen_bytes(B, Hq, nsel) + (size_t)B * Hq * (L / blk) * sizeof(float);
}

// ---------------------------------------------------------------------------
// pooled block keys
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_pool_kernel(const uint16_t* __restrict__ k, int L,
                                                         int E, int blk,
                                                         float* __restrict__ krep) {
  const int n = blockIdx.x, b = blockIdx.y;
  const int nblk = L / blk;
  const uint16_t* src = k + ((int64_t)b * L + (int64_t)n * blk) * E;
  float* dst = krep + ((int64_t)b * nblk + n) * E;
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
    *(float4*)(dst + e) = make_float4(a0 * inv, a1 * inv, a2 * inv, a3 * inv);
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
  const float* krep;    // [B, nblk, Hkv, d]
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
  float4 kv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = min(n0 + 2 * i, nblk - 1);
    kv[i] = *(const float4*)(a.krep + (((int64_t)b * nblk + n) * a.Hkv + g) * kBlkD + 4 * l);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = n0 + 2 * i;
    float p[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      p[hh] = 0.f;
      if (a.shared && hh > 0) continue;  // uniform: one summed query
      float acc = kv[i].x * qv[hh][0];
      acc = fmaf(kv[i].y, qv[hh][1], acc);
      acc = fmaf(kv[i].z, qv[hh][2], acc);
      acc = fmaf(kv[i].w, qv[hh][3], acc);
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
  int32_t* chosen;      // [B, Hq, nsel] (workspace)
  int32_t* blocks_out;  // [B, Hq, nsel] or null
};

// Largest 64-bit key over the wave (every lane gets it): quad swaps and row
// mirrors give each row of 16 its maximum (DPP, both halves with the same
// control), then the four row maxima through scalar registers.
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
  uint64_t m = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t x = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    m = max_u64(m, x);
  }
  return m;
}

constexpr int kSelMaxPerLane = kBlkMaxBlocks / 256;  // blocks per thread, at most

// One work-group per (query head, sequence).  Keys (score key << 32 | ~block)
// order blocks by score, ties to the lower block, so the selection is a
// plain maximum search: each wave takes the nsel largest keys of its share
// (nsel rounds of a wave maximum, the winner's lane retiring it), one wave
// then takes the nsel largest of the 4 nsel survivors the same way.
template <int KPL>  // keys per thread: blocks n = tid + 256 r, r < KPL
__global__ __launch_bounds__(256) void block_select_kernel(BlockSelArgs a) {
  __shared__ uint64_t cand[4][kBlkMaxSel];
  __shared__ int pick[kBlkMaxSel];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int nblk = a.nblk;
  const float* srow = a.scores + ((int64_t)b * a.Hq + h) * nblk;
  // block n = tid + 256 r
  uint64_t key[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int n = tid + 256 * r;
    key[r] = 0ull;
    if (256 * r >= nblk) continue;  // uniform: nothing left for any thread
    if (n < nblk) key[r] = ((uint64_t)blk_score_key(srow[n]) << 32) | (uint32_t)~(uint32_t)n;
  }
  // this wave's nsel largest keys
  const int m = min(nblk, a.nsel);
  for (int i = 0; i < m; ++i) {
    uint64_t best = 0ull;
#pragma unroll
    for (int r = 0; r < KPL; ++r) best = key[r] > best ? key[r] : best;
    const uint64_t w = wave_max_u64(best);
    if (lane == 0) cand[wave][i] = w;
    if (w != 0ull) {  // the owner retires the winning key (keys are distinct)
#pragma unroll
      for (int r = 0; r < KPL; ++r) key[r] = key[r] == w ? 0ull : key[r];
    }
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
  int32_t* ch = a.chosen + ((int64_t)b * a.Hq + h) * a.nsel;
  int32_t* bo = a.blocks_out ? a.blocks_out + ((int64_t)b * a.Hq + h) * a.nsel : nullptr;
  if (tid < a.nsel) {
    int val = -1, rank = tid;
    if (tid < m) {
      const int mine = pick[tid];
      rank = 0;
      for (int i = 0; i < m; ++i) rank += pick[i] < mine;
      val = mine;
    }
    ch[rank] = val;
    if (bo) bo[rank] = val;
  }
}

// ---------------------------------------------------------------------------
// attention over the visible set
// ---------------------------------------------------------------------------
struct BlockAttnArgs {
  const uint16_t* q;  // [B, Hq, d]
  const uint16_t* k;  // [B, L, Hkv, d]
  const uint16_t* v;
  const int32_t* chosen;  // [B, Hq, nsel], ascending, -1 padded
  int L, Hq, Hkv, blk, nsel, n_sink, n_win;
  float scale_log2;
  float* out;  // [B, Hq, d]
};

__device__ __forceinline__ float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void block_attn_kernel(BlockAttnArgs a) {
  __shared__ int rs[kBlkMaxRanges], re[kBlkMaxRanges], rcum[kBlkMaxRanges + 1];
  __shared__ int st[kBlkMaxRanges], en[kBlkMaxRanges];  // unsorted ranges
  __shared__ int s_nr;
  __shared__ float pb[4][64];
  __shared__ int tb[4][64];
  __shared__ float wm[4], wl[4];
  __shared__ float wo[4][kBlkD];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int g = h / (a.Hq / a.Hkv);
  const int L = a.L;

  // ---- visible ranges: sinks, chosen blocks, window -> disjoint, ascending
  if (tid == 0) {
    int n = 0;
    if (a.n_sink > 0) {
      st[n] = 0;
      en[n++] = min(a.n_sink, L);
    }
    const int32_t* ch = a.chosen + ((int64_t)b * a.Hq + h) * a.nsel;
    for (int i = 0; i < a.nsel; ++i) {
      const int c = ch[i];
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
  // query in registers, fp32 (every lane holds the whole row)
  float qf[kBlkD];
  {
    const uint4* qp = (const uint4*)(a.q + ((int64_t)b * a.Hq + h) * kBlkD);
#pragma unroll
    for (int i = 0; i < kBlkD / 8; ++i) {
      const uint4 u = qp[i];
      qf[8 * i + 0] = bf16_lo(u.x);
      qf[8 * i + 1] = bf16_hi(u.x);
      qf[8 * i + 2] = bf16_lo(u.y);
      qf[8 * i + 3] = bf16_hi(u.y);
      qf[8 * i + 4] = bf16_lo(u.z);
      qf[8 * i + 5] = bf16_hi(u.z);
      qf[8 * i + 6] = bf16_lo(u.w);
      qf[8 * i + 7] = bf16_hi(u.w);
    }
  }
  __syncthreads();
  const int nr = s_nr, ntok = rcum[nr];
  const int64_t row_stride = (int64_t)a.Hkv * kBlkD;  // elements between tokens
  const uint16_t* kb = a.k + (int64_t)b * L * row_stride + (int64_t)g * kBlkD;
  const uint16_t* vb = a.v + (int64_t)b * L * row_stride + (int64_t)g * kBlkD;

  float m_w = -INFINITY, l_w = 0.f, o0 = 0.f, o1 = 0.f;  // dims 2 lane, 2 lane + 1
  for (int c = wave; 64 * c < ntok; c += 4) {
    const int t = 64 * c + lane;
    const bool valid = t < ntok;
    int tok = 0;
    if (valid) {  // range holding flattened index t (binary search over rcum)
      int lo = 0, hi = nr - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rcum[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      tok = rs[lo] + (t - rcum[lo]);
    }
    float s = -INFINITY;
    if (valid) {
      const uint4* kp = (const uint4*)(kb + (int64_t)tok * row_stride);
      uint4 kr[kBlkD / 8];
#pragma unroll
      for (int i = 0; i < kBlkD / 8; ++i) kr[i] = kp[i];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kBlkD / 8; ++i) {
        acc = fmaf(qf[8 * i + 0], bf16_lo(kr[i].x), acc);
        acc = fmaf(qf[8 * i + 1], bf16_hi(kr[i].x), acc);
        acc = fmaf(qf[8 * i + 2], bf16_lo(kr[i].y), acc);
        acc = fmaf(qf[8 * i + 3], bf16_hi(kr[i].y), acc);
        acc = fmaf(qf[8 * i + 4], bf16_lo(kr[i].z), acc);
        acc = fmaf(qf[8 * i + 5], bf16_hi(kr[i].z), acc);
        acc = fmaf(qf[8 * i + 6], bf16_lo(kr[i].w), acc);
        acc = fmaf(qf[8 * i + 7], bf16_hi(kr[i].w), acc);
      }
      s = acc * a.scale_log2;
    }
    const float cmax = wave_max_f(s);  // finite: the chunk has a valid token
    const float m_new = fmaxf(m_w, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m_w - m_new);  // 0 at the first chunk
    const float p = valid ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
    l_w = l_w * alpha + wave_sum_f(p);
    o0 *= alpha;
    o1 *= alpha;
    m_w = m_new;
    pb[wave][lane] = p;
    tb[wave][lane] = tok;
    __builtin_amdgcn_wave_barrier();
    // value rows: 32 coalesced 256-byte loads in flight at a time
#pragma unroll
    for (int t0 = 0; t0 < 64; t0 += 32) {
      uint32_t vv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        vv[i] = *(const uint32_t*)(vb + (int64_t)tb[wave][t0 + i] * row_stride + 2 * lane);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float pp = pb[wave][t0 + i];
        o0 = fmaf(pp, bf16_lo(vv[i]), o0);
        o1 = fmaf(pp, bf16_hi(vv[i]), o1);
      }
    }
    __builtin_amdgcn_wave_barrier();  // pb / tb are rewritten by the next chunk
  }
  // ---- merge the four waves' (m, l, o)
  if (lane == 0) {
    wm[wave] = m_w;
    wl[wave] = l_w;
  }
  wo[wave][2 * lane] = o0;
  wo[wave][2 * lane + 1] = o1;
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
    float* o = a.out + ((int64_t)b * a.Hq + h) * kBlkD;
    o[2 * lane] = n0 * inv;
    o[2 * lane + 1] = n1 * inv;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_block_pool(const void* k, int B, int L, int Hkv, int d, int blk, float* krep,
                             hipStream_t st) {
  const int nblk = L / blk;
  if (B == 0 || nblk == 0) return hipSuccess;
  block_pool_kernel<<<dim3(nblk, B), 256, 0, st>>>((const uint16_t*)k, L, Hkv * d, blk, krep);
  return hipGetLastError();
}

hipError_t launch_block_decode(const BlockArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int nblk = a.L / a.blk;
  float* scores = (float*)((char*)a.ws + block_chosen_bytes(a.B, a.Hq, a.nsel));
  if (nblk > 0) {
    BlockScoreArgs c{};
    c.q = (const uint16_t*)a.q;
    c.krep = a.krep;
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
  BlockSelArgs s{};
  s.scores = scores;
  s.Hq = a.Hq;
  s.nblk = nblk;
  s.nsel = a.nsel;
  s.chosen = (int32_t*)a.ws;
  s.blocks_out = a.blocks_out;
  const dim3 sgrid((unsigned)a.Hq, (unsigned)a.B);
  if (nblk <= 256 * 4)
    block_select_kernel<4><<<sgrid, 256, 0, st>>>(s);
  else if (nblk <= 256 * 8)
    block_select_kernel<8><<<sgrid, 256, 0, st>>>(s);
  else if (nblk <= 256 * 16)
    block_select_kernel<16><<<sgrid, 256, 0, st>>>(s);
  else
    block_select_kernel<kSelMaxPerLane><<<sgrid, 256, 0, st>>>(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BlockAttnArgs t{};
  t.q = (const uint16_t*)a.q;
  t.k = (const uint16_t*)a.k;
  t.v = (const uint16_t*)a.v;
  t.chosen = s.chosen;
  t.L = a.L;
  t.Hq = a.Hq;
  t.Hkv = a.Hkv;
  t.blk = a.blk;
  t.nsel = a.nsel;
  t.n_sink = a.n_sink;
  t.n_win = a.n_win;
  t.scale_log2 = a.sm_scale * kLog2e;
  t.out = a.out;
  block_attn_kernel<<<dim3(a.Hq, a.B), 256, 0, st>>>(t);
  return hipGetLastError();
}

}  // namespace sa
