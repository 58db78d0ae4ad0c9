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

// chosen blocks [B, Hq, nsel] int32
size_t block_workspace_bytes(int B, int Hq, int L, int nsel, int Hkv, int d, int blk) {
  (void)Hkv;
  (void)d;
  (void)L;
  if (blk < 1 || B < 0 || Hq < 1 || nsel < 1) return 0;
  return (size_t)B * Hq * nsel * sizeof(int32_t);
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

struct BlockSelArgs {
  const uint16_t* q;    // [B, Hq, d]
  const float* krep;    // [B, nblk, Hkv, d]
  int Hq, Hkv, nblk, nsel;
  int shared;           // score with the sum of the KV group's queries
  int32_t* chosen;      // [B, Hq, nsel] (workspace)
  int32_t* blocks_out;  // [B, Hq, nsel] or null
};

// Largest 64-bit key over the wave (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = ((uint64_t)(uint32_t)__shfl_xor((int)(v >> 32), o) << 32) |
                       (uint32_t)__shfl_xor((int)(uint32_t)v, o);
    v = w > v ? w : v;
  }
  return v;
}

constexpr int kSelPerLane = kBlkMaxBlocks / 256;  // blocks per thread

// One work-group per (query head, sequence).  Keys (score key << 32 | ~block)
// order blocks by score, ties to the lower block, so the selection is a
// plain maximum search: each wave takes the nsel largest keys of its share
// (nsel rounds of a wave maximum, the winner's lane retiring it), one wave
// then takes the nsel largest of the 4 nsel survivors the same way.
__global__ __launch_bounds__(256) void block_select_kernel(BlockSelArgs a) {
  __shared__ uint64_t cand[4][kBlkMaxSel];
  __shared__ int pick[kBlkMaxSel];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int G = a.Hq / a.Hkv, g = h / G, nblk = a.nblk;
  // the head's query, or with a shared choice the sum of the group's queries
  // (the sum of the heads' block scores is the group-sum query's score, so
  // the group's work-groups all reach the same choice), staged in LDS
  __shared__ float qs[kBlkD];
  if (tid < kBlkD) {
    const int h0 = a.shared ? g * G : h, h1 = a.shared ? h0 + G : h + 1;
    float acc = 0.f;
    for (int hh = h0; hh < h1; ++hh)
      acc += bf16_bits_to_float(a.q[((int64_t)b * a.Hq + hh) * kBlkD + tid]);
    qs[tid] = acc;
  }
  __syncthreads();
  float qf[kBlkD];
#pragma unroll
  for (int i = 0; i < kBlkD / 4; ++i) {
    const float4 v = *(const float4*)&qs[4 * i];
    qf[4 * i] = v.x;
    qf[4 * i + 1] = v.y;
    qf[4 * i + 2] = v.z;
    qf[4 * i + 3] = v.w;
  }
  // block n = tid + 256 r: one pooled-key row (512 bytes) per lane
  uint64_t key[kSelPerLane];
#pragma unroll
  for (int r = 0; r < kSelPerLane; ++r) {
    const int n = tid + 256 * r;
    key[r] = 0ull;
    if (256 * r >= nblk) continue;  // uniform: nothing left for any thread
    if (n < nblk) {
      const float4* kr = (const float4*)(a.krep + (((int64_t)b * nblk + n) * a.Hkv + g) * kBlkD);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // 8 x 16 bytes in flight
        float4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = kr[8 * c + i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d0 = 32 * c + 4 * i;
          acc = fmaf(v[i].x, qf[d0], acc);
          acc = fmaf(v[i].y, qf[d0 + 1], acc);
          acc = fmaf(v[i].z, qf[d0 + 2], acc);
          acc = fmaf(v[i].w, qf[d0 + 3], acc);
        }
      }
      key[r] = ((uint64_t)blk_score_key(acc) << 32) | (uint32_t)~(uint32_t)n;
    }
  }
  // this wave's nsel largest keys
  const int m = min(nblk, a.nsel);
  for (int i = 0; i < m; ++i) {
    uint64_t best = 0ull;
#pragma unroll
    for (int r = 0; r < kSelPerLane; ++r) best = key[r] > best ? key[r] : best;
    const uint64_t w = wave_max_u64(best);
    if (lane == 0) cand[wave][i] = w;
    if (w != 0ull) {  // the owner retires the winning key (keys are distinct)
#pragma unroll
      for (int r = 0; r < kSelPerLane; ++r) key[r] = key[r] == w ? 0ull : key[r];
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
  BlockSelArgs s{};
  s.q = (const uint16_t*)a.q;
  s.krep = a.krep;
  s.Hq = a.Hq;
  s.Hkv = a.Hkv;
  s.nblk = nblk;
  s.nsel = a.nsel;
  s.shared = a.shared_choice;
  s.chosen = (int32_t*)a.ws;
  s.blocks_out = a.blocks_out;
  block_select_kernel<<<dim3(a.Hq, a.B), 256, 0, st>>>(s);
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
