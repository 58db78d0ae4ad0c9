// mla.hip -- sparse MLA over a gathered set of latent rows, on gfx950.
//
// For each query (b,t) and head h, over the slots j of idx[b,t,:] that hold a
// position in [0, L):
//   s[h,j] = (q_lat[h,:] . c_kv[j,:] + q_rope[h,:] . k_rope[j,:]) * sm_scale
//   out[h,:] = sum_j softmax_j(s[h,:]) c_kv[j,:],  lse[h] = log sum_j exp(s[h,j])
// ("MLA 与稀疏注意力" full-score and absorption sections; "Sparse Attention
// 数学学习笔记" §2, §8, §9).  All heads of a query read the same rows.
//
// mla_mfma_kernel (bf16, dc = 512, dR = 64): a work-group is four waves of 16
// heads each and walks a range of the query's slots 32 rows at a time.  The
// 32 gathered rows (1152 bytes each: 1024 of c_kv, 128 of k_rope) are staged
// in LDS, double buffered.  Per wave and tile:
//   S^T[32 rows x 16 heads] = K[32 x 576] Q^T            (36 MFMA 16x16x32)
//   online softmax per head (each lane owns one head: a lane's S^T values all
//   belong to head l%16, so the max, the rescale and the row sums stay in the
//   lane, with one max across the four lane groups)
//   O^T[512 x 16 heads] += V^T[512 x 32] P^T[32 x 16]    (2 x 32 MFMA 16x16x32)
// P^T is already in the B-operand layout: the contraction order over the 32
// rows is chosen so that lane group g's eight k-slots are rows 4g..4g+3 and
// 16+4g..16+4g+3, exactly the rows its S^T registers hold.  V^T comes from LDS
// through ds_read_b64_tr_b16, which hands each lane four consecutive rows of
// one column.  P enters the product as two bf16 terms, P_hi = bf16(P) and
// P_lo = bf16(P - P_hi) (two MFMAs on the same V^T operand, so no extra LDS
// traffic); a single bf16 P would perturb each weight by up to 2^-9, which
// breaks a 2e-3 max-abs bound when few rows carry the mass.
// Long index sets are split over work-groups (KV split); a combine kernel
// merges the partial (m, l, o) by log-sum-exp.
//
// mla_vector_kernel: fp32 vector ALU, any dc <= 512, dR <= 64, for fp32
// inputs (and bf16 outside the MFMA shape); one work-group per query.
#include "common.hpp"
#include "launch.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// bf16 MFMA path
// ---------------------------------------------------------------------------
constexpr int kMlaDc = 512, kMlaDr = 64, kMlaD = kMlaDc + kMlaDr;
constexpr int kMlaRowB = kMlaD * 2;           // 1152 bytes per gathered row
constexpr int kMlaLRow = kMlaRowB + 16;       // padded LDS row (bank spread)
constexpr int kMlaTile = 32;                  // rows per tile
constexpr int kMlaWaves = 4;                  // 16 heads per wave
constexpr int kMlaHeadsWg = 16 * kMlaWaves;
constexpr int kMlaChunksRow = kMlaRowB / 16;  // 72 x 16 bytes
constexpr int kMlaStage = (kMlaTile * kMlaChunksRow + 64 * kMlaWaves - 1) / (64 * kMlaWaves);

struct MlaKernelArgs {
  const uint16_t* q_lat;   // [BT, H, 512]
  const uint16_t* q_rope;  // [BT, H, 64]
  const uint8_t* c_kv;     // row (b,s) at + (b*L+s)*c_stride_b
  const uint8_t* k_rope;   // row (b,s) at + (b*L+s)*r_stride_b
  int64_t c_stride_b, r_stride_b;  // bytes
  const int32_t* idx;      // [BT, k]
  int k, T, L, H;
  int nsplit, slots_per_split;
  float scale_log2;        // sm_scale * log2(e)
  float* out;              // [BT, H, 512]
  float* lse;              // [BT, H] or null
  float* part_o;           // [BT, H, nsplit, 512] when nsplit > 1
  float* part_ml;          // [BT, H, nsplit, 2]
};

constexpr int kMlaMaxSplitSlots = 2048;  // index slice of one work-group, kept in LDS

__global__ __launch_bounds__(64 * kMlaWaves, 1) void mla_mfma_kernel(MlaKernelArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kMlaTile * kMlaLRow];
  __shared__ int spos[kMlaMaxSplitSlots];  // positions of this split, -1 = skip

  // block -> (bt, head group, split); blocks that share (bt, split) are placed
  // on the same XCD (blocks are dealt to the 8 XCDs round-robin) so the head
  // groups' re-reads of the gathered rows hit that XCD's L2.
  const int hgroups = a.H / kMlaHeadsWg;
  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int hg = lin % hgroups;
  const int split = (lin / hgroups) % a.nsplit;
  const int64_t bt = lin / (hgroups * a.nsplit);
  const int b = (int)(bt / a.T);

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int h = hg * kMlaHeadsWg + wave * 16 + n;  // this lane's head

  const int j_begin = split * a.slots_per_split;
  const int j_end = min(a.k, j_begin + a.slots_per_split);
  const int ntiles = (j_end - j_begin + kMlaTile - 1) / kMlaTile;
  const int32_t* idxr = a.idx + bt * a.k;
  // the split's index slice goes to LDS first: row addresses then never wait
  // on a global load
  for (int j = tid; j < ntiles * kMlaTile; j += 64 * kMlaWaves) {
    const int s = j_begin + j < j_end ? idxr[j_begin + j] : -1;
    spos[j] = (s >= 0 && s < a.L) ? s : -1;
  }
  __syncthreads();

  // Q^T operand: qb[ks] = q[h][32 ks + 8 g .. +8], ks < 16 from q_lat, 16..17 q_rope
  bf16x8 qb[18];
  {
    const uint16_t* ql = a.q_lat + (bt * a.H + h) * (int64_t)kMlaDc;
    const uint16_t* qr = a.q_rope + (bt * a.H + h) * (int64_t)kMlaDr;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[ks] = as_bf16x8(*(const uintx4*)(ql + 32 * ks + 8 * g));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qb[16 + ks] = as_bf16x8(*(const uintx4*)(qr + 32 * ks + 8 * g));
  }

  floatx4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- staging: chunk c = tid + 256 i -> row c / 72, 16-byte piece c % 72 ----
  uintx4 stage[kMlaStage];
  auto gload = [&](int tl) {
#pragma unroll
    for (int i = 0; i < kMlaStage; ++i) {
      const int c = tid + 64 * kMlaWaves * i;
      stage[i] = uintx4{0u, 0u, 0u, 0u};
      if (c < kMlaTile * kMlaChunksRow) {
        const int r = c / kMlaChunksRow, p = c % kMlaChunksRow;
        const int s = spos[tl * kMlaTile + r];
        if (s >= 0) {
          const int64_t row = (int64_t)b * a.L + s;
          const uint8_t* src = p < 64 ? a.c_kv + row * a.c_stride_b + 16 * p
                                      : a.k_rope + row * a.r_stride_b + 16 * (p - 64);
          stage[i] = *(const uintx4*)src;
        }
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kMlaStage; ++i) {
      const int c = tid + 64 * kMlaWaves * i;
      if (c < kMlaTile * kMlaChunksRow) {
        const int r = c / kMlaChunksRow, p = c % kMlaChunksRow;
        *(uintx4*)(&tile[buf][r * kMlaLRow + 16 * p]) = stage[i];
      }
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int tl = 0; tl < ntiles; ++tl) {
    const int buf = tl & 1;
    if (tl + 1 < ntiles) gload(tl + 1);
    const uint8_t* tb = tile[buf];

    // S^T[jt]: rows 16 jt + 4 g + r, head n
    floatx4 st[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* rowp = tb + (16 * jt + n) * kMlaLRow + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        acc = mfma16x16x32(as_bf16x8(*(const uintx4*)(rowp + 64 * ks)), qb[ks], acc);
      st[jt] = acc;
    }
    // scale to log2 units, mask skipped slots, tile max per head
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * jt + 4 * g + r;
        const float v = spos[tl * kMlaTile + row] >= 0 ? st[jt][r] * a.scale_log2 : -INFINITY;
        x[4 * jt + r] = v;
        mt = fmaxf(mt, v);
      }
    mt = max_over_lane_groups(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);  // 0 while nothing seen yet
    // P = P_hi + P_lo, both bf16: the pair carries ~16 significant bits, so
    // the product stays at fp32-level accuracy while the MFMAs stay bf16.
    uint32_t pbh[4], pbl[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = exp2f(x[e] - m_use), p1 = exp2f(x[e + 1] - m_use);
      psum += p0 + p1;
      const uint32_t hi = pack_bf16x2_rne(p0, p1);
      pbh[e / 2] = hi;
      pbl[e / 2] = pack_bf16x2_rne(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }
    const bf16x8 pBh = __builtin_bit_cast(bf16x8, uintx4{pbh[0], pbh[1], pbh[2], pbh[3]});
    const bf16x8 pBl = __builtin_bit_cast(bf16x8, uintx4{pbl[0], pbl[1], pbl[2], pbl[3]});
    // V^T operand rows: 4 g + (lane%16)/4 and 16 + 4 g + (lane%16)/4, columns
    // 16 dt + 4 (lane%4) .. +3  (see the transpose-read note in common.hpp)
    const uint8_t* v0 = tb + (4 * g + (n >> 2)) * kMlaLRow + 8 * (n & 3);
    const uint8_t* v1 = v0 + 16 * kMlaLRow;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (shortx4 __attribute__((address_space(3)))*)(v0 + 32 * dt));
      shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (shortx4 __attribute__((address_space(3)))*)(v1 + 32 * dt));
      const bf16x8 vA = __builtin_bit_cast(
          bf16x8, uintx4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))});
      o[dt] = mfma16x16x32(vA, pBh, o[dt]);
      o[dt] = mfma16x16x32(vA, pBl, o[dt]);
    }
    if (tl + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- finish ----
  const float l_tot = sum_over_lane_groups(l_run);
  if (a.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = a.out + (bt * a.H + h) * (int64_t)kMlaDc;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *(floatx4*)(orow + 16 * dt + 4 * g) = o[dt] * inv;
    if (a.lse && g == 0)
      a.lse[bt * a.H + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t u = (bt * a.H + h) * a.nsplit + split;
    float* orow = a.part_o + u * kMlaDc;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(floatx4*)(orow + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      a.part_ml[2 * u] = m_run;
      a.part_ml[2 * u + 1] = l_tot;
    }
  }
}

// Merge nsplit partial (m, l, o) of one (query, head): one 128-thread group,
// four output columns per thread.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int nsplit, int dc,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t u = blockIdx.x;  // (bt, h)
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[2 * (u * nsplit + s)]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float Lsum = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ml = part_ml + 2 * (u * nsplit + s);
    Lsum += exp2f(ml[0] - Mu) * ml[1];
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  for (int d = 4 * threadIdx.x; d < dc; d += 4 * 128) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float wgt = exp2f(part_ml[2 * (u * nsplit + s)] - Mu);
      acc += wgt * *(const floatx4*)(part_o + (u * nsplit + s) * dc + d);
    }
    *(floatx4*)(out + u * dc + d) = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[u] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 vector path
// ---------------------------------------------------------------------------
constexpr int kVecRows = 32;

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}

constexpr int kVecMaxOut = 32;  // outputs per thread: H * dc <= 256 * 32

template <typename T>
__global__ __launch_bounds__(256) void mla_vector_kernel(
    const T* __restrict__ q_lat, const T* __restrict__ q_rope, const T* __restrict__ c_kv,
    const T* __restrict__ k_rope, int64_t c_stride, int64_t r_stride,
    const int32_t* __restrict__ idx, int k, int T_, int L, int H, int dc, int dR,
    float scale_log2, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float lds[];
  const int D = dc + dR, DP = D + 1;  // padded row
  float* qs = lds;                          // [H][D+1]
  float* rows = qs + H * DP;                // [kVecRows][D+1]
  float* sc = rows + kVecRows * DP;         // [H][kVecRows]
  float* mrun = sc + H * kVecRows;          // [H]
  float* lrun = mrun + H;                   // [H]
  float* alph = lrun + H;                   // [H]
  __shared__ int valid[kVecRows];

  const int64_t bt = blockIdx.x;
  const int b = (int)(bt / T_);
  const int tid = threadIdx.x;
  for (int i = tid; i < H * D; i += 256) {
    const int hh = i / D, c = i % D;
    qs[hh * DP + c] = c < dc ? ld(q_lat, (bt * H + hh) * dc + c)
                             : ld(q_rope, (bt * H + hh) * dR + (c - dc));
  }
  for (int i = tid; i < H; i += 256) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
  }
  const int nout = (H * dc + 255) / 256;
  float acc[kVecMaxOut];
#pragma unroll
  for (int i = 0; i < kVecMaxOut; ++i) acc[i] = 0.f;

  const int32_t* idxr = idx + bt * k;
  for (int j0 = 0; j0 < k; j0 += kVecRows) {
    __syncthreads();  // previous tile fully consumed
    if (tid < kVecRows) {
      const int j = j0 + tid;
      const int s = j < k ? idxr[j] : -1;
      valid[tid] = (s >= 0 && s < L) ? s : -1;
    }
    __syncthreads();
    for (int i = tid; i < kVecRows * D; i += 256) {
      const int r = i / D, c = i % D;
      const int s = valid[r];
      float v = 0.f;
      if (s >= 0) {
        const int64_t row = (int64_t)b * L + s;
        v = c < dc ? ld(c_kv, row * c_stride + c) : ld(k_rope, row * r_stride + (c - dc));
      }
      rows[r * DP + c] = v;
    }
    __syncthreads();
    for (int p = tid; p < H * kVecRows; p += 256) {
      const int hh = p / kVecRows, r = p % kVecRows;
      float s = -INFINITY;
      if (valid[r] >= 0) {
        const float* qh = qs + hh * DP;
        const float* rr = rows + r * DP;
        float cont = 0.f, rope = 0.f;
        for (int c = 0; c < dc; ++c) cont = fmaf(qh[c], rr[c], cont);
        for (int c = dc; c < D; ++c) rope = fmaf(qh[c], rr[c], rope);
        s = (cont + rope) * scale_log2;
      }
      sc[hh * kVecRows + r] = s;
    }
    __syncthreads();
    for (int hh = tid; hh < H; hh += 256) {
      float mt = -INFINITY;
      for (int r = 0; r < kVecRows; ++r) mt = fmaxf(mt, sc[hh * kVecRows + r]);
      const float m_new = fmaxf(mrun[hh], mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float al = exp2f(mrun[hh] - m_use);
      float ps = 0.f;
      for (int r = 0; r < kVecRows; ++r) {
        const float p = exp2f(sc[hh * kVecRows + r] - m_use);
        sc[hh * kVecRows + r] = p;
        ps += p;
      }
      lrun[hh] = lrun[hh] * al + ps;
      mrun[hh] = m_new;
      alph[hh] = al;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kVecMaxOut; ++i) {
      if (i >= nout) break;
      const int oi = tid + 256 * i;
      if (oi >= H * dc) break;
      const int hh = oi / dc, d = oi % dc;
      float v = acc[i] * alph[hh];
      const float* p = sc + hh * kVecRows;
      for (int r = 0; r < kVecRows; ++r) v = fmaf(p[r], rows[r * DP + d], v);
      acc[i] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kVecMaxOut; ++i) {
    if (i >= nout) break;
    const int oi = tid + 256 * i;
    if (oi >= H * dc) break;
    const int hh = oi / dc, d = oi % dc;
    const float l = lrun[hh];
    out[(bt * H + hh) * dc + d] = l > 0.f ? acc[i] / l : 0.f;
  }
  if (lse)
    for (int hh = tid; hh < H; hh += 256)
      lse[bt * H + hh] = lrun[hh] > 0.f ? (mrun[hh] + __log2f(lrun[hh])) * kLn2 : -INFINITY;
}

static size_t vector_lds_bytes(int H, int dc, int dR) {
  const size_t D = dc + dR;
  return sizeof(float) * ((size_t)H * (D + 1) + kVecRows * (D + 1) + (size_t)H * kVecRows + 3 * H);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
bool mla_uses_mfma(const MlaArgs& a) {
  return a.dtype == SA_BF16 && a.dc == kMlaDc && a.dR == kMlaDr && a.H % kMlaHeadsWg == 0;
}

bool mla_supported(const MlaArgs& a) {
  if (mla_uses_mfma(a)) return true;
  if (a.dc > 512 || a.dR > 64 || a.dR < 0 || a.dc < 1) return false;
  if ((int64_t)a.H * a.dc > 256 * kVecMaxOut) return false;
  return vector_lds_bytes(a.H, a.dc, a.dR) <= 64 * 1024;
}

// KV-split count for the MFMA path: enough work-groups to cover the CUs.
static int mla_nsplit(int64_t bt, int H, int k) {
  const int64_t groups = bt * (H / kMlaHeadsWg);
  const int max_split = (k + 2 * kMlaTile - 1) / (2 * kMlaTile);  // >= 64 rows per split
  int ns = 1;
  while ((int64_t)ns * kMlaMaxSplitSlots < k) ns *= 2;  // one split's slice fits in LDS
  while (groups * ns < 256 && ns * 2 <= max_split) ns *= 2;
  return ns;
}

size_t mla_workspace_bytes(int dtype, int B, int T, int k, int H, int dc) {
  if (dtype != SA_BF16 || dc != kMlaDc || H % kMlaHeadsWg) return 0;
  const int64_t bt = (int64_t)B * T;
  const int ns = mla_nsplit(bt, H, k);
  if (ns == 1) return 0;
  return (size_t)bt * H * ns * (kMlaDc + 2) * sizeof(float);
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t st) {
  const int64_t bt = (int64_t)a.B * a.T;
  if (bt == 0) return hipSuccess;
  const float scale_log2 = a.sm_scale * kLog2e;
  if (mla_uses_mfma(a)) {
    MlaKernelArgs m{};
    m.q_lat = (const uint16_t*)a.q_lat;
    m.q_rope = (const uint16_t*)a.q_rope;
    m.c_kv = (const uint8_t*)a.c_kv;
    m.k_rope = (const uint8_t*)a.k_rope;
    m.c_stride_b = a.c_stride * 2;
    m.r_stride_b = a.r_stride * 2;
    m.idx = a.idx;
    m.k = a.k;
    m.T = a.T;
    m.L = a.L;
    m.H = a.H;
    m.nsplit = mla_nsplit(bt, a.H, a.k);
    m.slots_per_split = ((a.k + m.nsplit - 1) / m.nsplit + kMlaTile - 1) / kMlaTile * kMlaTile;
    m.scale_log2 = scale_log2;
    m.out = a.out;
    m.lse = a.lse;
    if (m.nsplit > 1) {
      m.part_o = (float*)a.ws;
      m.part_ml = m.part_o + bt * a.H * m.nsplit * kMlaDc;
    }
    const int64_t nblk = bt * (a.H / kMlaHeadsWg) * m.nsplit;
    mla_mfma_kernel<<<(unsigned)nblk, 64 * kMlaWaves, 0, st>>>(m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || m.nsplit == 1) return e;
    mla_combine_kernel<<<(unsigned)(bt * a.H), 128, 0, st>>>(m.part_o, m.part_ml, m.nsplit,
                                                            kMlaDc, a.out, a.lse);
    return hipGetLastError();
  }
  const size_t lds = vector_lds_bytes(a.H, a.dc, a.dR);
  if (a.dtype == SA_F32) {
    mla_vector_kernel<float><<<(unsigned)bt, 256, lds, st>>>(
        (const float*)a.q_lat, (const float*)a.q_rope, (const float*)a.c_kv,
        (const float*)a.k_rope, a.c_stride, a.r_stride, a.idx, a.k, a.T, a.L, a.H, a.dc,
        a.dR, scale_log2, a.out, a.lse);
  } else {
    mla_vector_kernel<uint16_t><<<(unsigned)bt, 256, lds, st>>>(
        (const uint16_t*)a.q_lat, (const uint16_t*)a.q_rope, (const uint16_t*)a.c_kv,
        (const uint16_t*)a.k_rope, a.c_stride, a.r_stride, a.idx, a.k, a.T, a.L, a.H, a.dc,
        a.dR, scale_log2, a.out, a.lse);
  }
  return hipGetLastError();
}

}  // namespace sa
