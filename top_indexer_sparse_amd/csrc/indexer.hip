// indexer.hip -- lightning-indexer scores on gfx950.
//
//   I[b,t,s] = sum_h w[b,t,h] * ReLU(q[b,t,h,:] . k[b,s,:])
// ("Sparse Attention 数学学习笔记" §9; "MLA 与稀疏注意力" DSA section), -inf for
// positions that are not candidates (s >= kv_len, or s > q_pos in prefill).
//
// Three kernels:
//  * idx_vector_kernel -- fp32 vector ALU, any dtype mix, exact for the small
//    integer workload.  One work-group per (query, 32-position tile).
//  * idx_decode_kernel -- bf16 MFMA for few queries (decode).  The query's
//    HI x dI block stays in registers as the A operand (rows = heads); keys
//    stream from HBM straight into B-operand registers (columns = positions),
//    16 positions per step through a 4-deep register ring.  The ReLU * w reduction over
//    heads runs in the epilogue: per lane 4 heads per head tile, then across
//    the four lane groups.
//  * idx_prefill_kernel -- the same contraction for many queries: eight waves
//    hold eight consecutive queries and share 64-position key tiles staged in
//    LDS, so each key byte read from L2 feeds eight queries.
// fp8 keys (OCP e4m3fn) are widened to bf16 in registers (exact) and the
// per-token scale multiplies the finished score: s*ReLU(x) = ReLU(s*x), s >= 0.
#include "common.hpp"
#include "index_core.hpp"
#include "launch.hpp"

namespace sa {

// ---------------------------------------------------------------------------
// fp32 vector path
// ---------------------------------------------------------------------------
template <typename QT>
__device__ __forceinline__ float load_q(const QT* p, int64_t i);
template <>
__device__ __forceinline__ float load_q<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_q<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
template <typename KT>
__device__ __forceinline__ float load_k(const KT* p, int64_t i);
template <>
__device__ __forceinline__ float load_k<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_k<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
template <>
__device__ __forceinline__ float load_k<uint8_t>(const uint8_t* p, int64_t i) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)p[i], false);
  return v[0];
}

constexpr int kVecTile = 32;   // positions per work-group
constexpr int kVecGroups = 8;  // head groups per position (256 threads)

template <typename QT, typename KT>
__global__ __launch_bounds__(256) void idx_vector_kernel(
    const QT* __restrict__ q, const float* __restrict__ w,
    const KT* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, int HI, int dI, float* __restrict__ scores) {
  extern __shared__ float lds[];
  const int stride = dI + 1;  // padded rows: conflict-free column reads
  float* qs = lds;                       // [HI][dI+1]
  float* ks = lds + HI * stride;         // [kVecTile][dI+1]
  float* ws = ks + kVecTile * stride;    // [HI]
  const int64_t bt = blockIdx.y;
  const int b = (int)(bt / T);
  const int s0 = blockIdx.x * kVecTile;
  const int lim = candidate_limit(q_pos, kv_len, b, bt, L);
  const int tid = threadIdx.x;
  const int nrows = min(kVecTile, max(lim - s0, 0));
  if (nrows > 0) {
    for (int i = tid; i < HI * dI; i += 256)
      qs[(i / dI) * stride + i % dI] = load_q(q, bt * HI * dI + i);
    for (int i = tid; i < HI; i += 256) ws[i] = w[bt * HI + i];
    for (int i = tid; i < nrows * dI; i += 256) {
      int r = i / dI, c = i % dI;
      ks[r * stride + c] = load_k(k, ((int64_t)b * L + s0 + r) * dI + c);
    }
  }
  __syncthreads();
  const int j = tid / kVecGroups, hg = tid % kVecGroups;
  float acc = 0.f;
  if (j < nrows) {
    for (int h = hg; h < HI; h += kVecGroups) {
      float dot = 0.f;
      const float* qh = qs + h * stride;
      const float* kj = ks + j * stride;
      for (int c = 0; c < dI; ++c) dot = fmaf(qh[c], kj[c], dot);
      acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  const int s = s0 + j;
  if (hg == 0 && s < L) {
    float v = -INFINITY;
    if (s < lim) v = kscale ? acc * kscale[(int64_t)b * L + s] : acc;
    scores[bt * L + s] = v;
  }
}

// ---------------------------------------------------------------------------
// MFMA paths
// ---------------------------------------------------------------------------
// One query per grid row; waves split the positions of the work-group.  Each
// wave streams a contiguous range through a register ring of R key chunks
// (16 positions each), so R - 1 chunks (28 KB of bf16 keys per wave at R = 8)
// stay in flight while one is consumed; R shrinks to 4 where the query block
// alone takes half the registers (H^I x d^I = 128 x 128).  The loop body is free of conditional memory operations: ring
// loads are always issued (rows past the range are clamped to its last valid
// row and their scores ignored), and scores go to a per-wave LDS buffer, so
// the compiler's vmcnt waits count exactly the older chunk's loads instead of
// draining the ring.  The scores (times the fp8 scale) leave with coalesced
// stores after the loop.
constexpr int kDecMaxRing = 8;
constexpr int kDecMaxSpan = 1024;                    // positions per wave, at most
constexpr int kDecBuf = kDecMaxSpan + 16 * kDecMaxRing;  // + the ring's overrun
template <int HT, int DI>
constexpr int dec_ring() { return 16 * HT * DI >= 16384 ? 4 : kDecMaxRing; }

template <int HT, int DI, bool FP8>
__global__ __launch_bounds__(256) void idx_decode_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, int s_per_wave, float* __restrict__ scores) {
  constexpr int HI = 16 * HT;
  constexpr int ROWB = FP8 ? DI : 2 * DI;  // bytes per key row
  constexpr int NSC = kDecMaxSpan / 64;    // prefetched scales per lane
  constexpr int R = dec_ring<HT, DI>();
  __shared__ float sbuf[4][kDecBuf];
  const int64_t bt = blockIdx.y;
  const int b = (int)(bt / T);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int lim = candidate_limit(q_pos, kv_len, b, bt, L);
  const int s_begin = (blockIdx.x * 4 + wave) * s_per_wave;
  const int s_end = min(s_begin + s_per_wave, L);
  if (s_begin >= s_end) return;
  float* out = scores + bt * L;
  const int v_end = min(s_end, lim);  // positions needing a score
  // positions [max(s_begin, lim), s_end) are not candidates
  for (int s = max(s_begin, lim) + lane; s < s_end; s += 64) out[s] = -INFINITY;
  if (s_begin >= v_end) return;

  const uint8_t* kb = k + (int64_t)b * L * ROWB;
  const int nch = (v_end - s_begin + 15) / 16;
  auto row_of = [&](int c) { return kb + (int64_t)min(s_begin + 16 * c + n, v_end - 1) * ROWB; };

  QueryRegs<HT, DI, FP8> qr;
  qr.load(q + bt * HI * DI, w + bt * HI, lane);
  // The query and weights must have landed before the ring starts: loads
  // still pending at the loop entry would make every iteration's vmcnt wait
  // count the ring's own loads and drain it.
  wait_vmcnt<0>();
  float scr[FP8 ? NSC : 1];  // fp8 per-token scales of this lane's output slots
  if constexpr (FP8) {
    const float* scb = kscale + (int64_t)b * L;
#pragma unroll
    for (int i = 0; i < NSC; ++i)
      scr[i] = scb[min(s_begin + lane + 64 * i, v_end - 1)];
  }
  // The ring is filled by the loop itself (its first pass only loads), so the
  // ring registers are the same on every pass and at the loop entry.
  KeyChunk<DI, FP8> ring[R];
  float* sb = sbuf[wave];
  for (int c0 = -R; c0 < nch; c0 += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = c0 + i;
      if (c0 >= 0) {  // uniform; chunks past nch are computed and dropped
        const float sc = qr.score(ring[i]);
        sb[16 * c + n] = sc;  // the four lane groups write the same value
      }
      ring[i].load(row_of(c + R), g);
    }
  }
  // the wave's own LDS writes are ordered before these reads
  const int span = v_end - s_begin;
#pragma unroll
  for (int i = 0; i < NSC; ++i) {
    const int j = lane + 64 * i;
    if (j < span) {
      float v = sb[j];
      if constexpr (FP8) v *= scr[i];
      out[s_begin + j] = v;
    }
  }
}

// Eight waves = eight consecutive queries of one sequence; 64-position key
// tiles staged in LDS (rows padded by 16 bytes against bank conflicts).
constexpr int kPfWaves = 8;
constexpr int kPfTile = 64;

template <int HT, int DI, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(HT <= 4 ? 4 : 2))) void idx_prefill_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, float* __restrict__ scores) {
  constexpr int HI = 16 * HT;
  constexpr int ROWB = FP8 ? DI : 2 * DI;
  constexpr int LROW = ROWB + 16;                 // padded LDS row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int CPT = kPfTile * CPR;              // chunks per tile
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kPfTile * LROW];
  __shared__ float tscale[2][kPfTile];

  const int ngroups = (T + kPfWaves - 1) / kPfWaves;
  const int grp = ngroups - 1 - (int)blockIdx.x;  // heaviest (latest) queries first
  const int b = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int t = grp * kPfWaves + wave;
  const bool active = t < T;
  const int64_t bt = (int64_t)b * T + (active ? t : T - 1);
  const int lim = active ? candidate_limit(q_pos, kv_len, b, bt, L) : 0;
  // the work-group's tile range covers the largest limit of its queries
  int lim_max = lim;
  {
    __shared__ int wl[kPfWaves];
    if (lane == 0) wl[wave] = lim;
    __syncthreads();
    for (int i = 0; i < kPfWaves; ++i) lim_max = max(lim_max, wl[i]);
  }
  float* out = scores + bt * L;
  if (active)
    for (int s = lim + lane; s < L; s += 64) out[s] = -INFINITY;
  const int ntiles = (lim_max + kPfTile - 1) / kPfTile;
  if (ntiles == 0) return;

  QueryRegs<HT, DI, FP8> qr;
  if (active) qr.load(q + bt * HI * DI, w + bt * HI, lane);
  const uint8_t* kb = k + (int64_t)b * L * ROWB;
  const float* scb = kscale ? kscale + (int64_t)b * L : nullptr;

  // staging: each thread moves chunk ids tid, tid + 512, ... of a tile
  constexpr int PER = (CPT + 511) / 512;
  uintx4 stage[PER];
  auto gload = [&](int tl) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + 512 * i;
      if (c < CPT) {
        const int r = c / CPR, o = c % CPR;
        const int s = min(tl * kPfTile + r, lim_max - 1);
        stage[i] = *(const uintx4*)(kb + (int64_t)s * ROWB + 16 * o);
      }
    }
  };
  auto lstore = [&](int buf, int tl) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + 512 * i;
      if (c < CPT) {
        const int r = c / CPR, o = c % CPR;
        *(uintx4*)(&tile[buf][r * LROW + 16 * o]) = stage[i];
      }
    }
    if (scb && threadIdx.x < kPfTile)
      tscale[buf][threadIdx.x] = scb[min(tl * kPfTile + (int)threadIdx.x, lim_max - 1)];
  };

  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int tl = 0; tl < ntiles; ++tl) {
    const int buf = tl & 1;
    if (tl + 1 < ntiles) gload(tl + 1);
    const int base = tl * kPfTile;
    if (active && base < lim) {
#pragma unroll
      for (int c = 0; c < kPfTile / 16; ++c) {
        const int s0 = base + 16 * c;
        if (s0 >= lim) break;
        KeyChunk<DI, FP8> kc;
        kc.load(&tile[buf][(16 * c + n) * LROW], g);
        float sc = qr.score(kc);
        const int s = s0 + n;
        if (g == 0 && s < lim) {
          if (scb) sc *= tscale[buf][16 * c + n];
          out[s] = sc;
        }
      }
    }
    if (tl + 1 < ntiles) lstore(buf ^ 1, tl + 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int HT, int DI, bool FP8>
static hipError_t launch_mfma(const IndexerArgs& a, hipStream_t st) {
  const auto* q = (const uint16_t*)a.q;
  const auto* k = (const uint8_t*)a.k;
  if (a.q_pos && a.T >= kPfWaves) {
    dim3 grid((a.T + kPfWaves - 1) / kPfWaves, a.B);
    idx_prefill_kernel<HT, DI, FP8><<<grid, 512, 0, st>>>(
        q, a.w, k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L, a.scores);
  } else {
    // long per-wave ranges amortise the query registers; shrink them only
    // until the grid has ~2 waves per SIMD (512 work-groups of 4 waves)
    int s_per_wave = kDecMaxSpan;
    const int64_t rows = (int64_t)a.B * a.T;
    while (s_per_wave > 64 && rows * ((a.L + 4 * s_per_wave - 1) / (4 * s_per_wave)) < 512)
      s_per_wave /= 2;
    dim3 grid((a.L + 4 * s_per_wave - 1) / (4 * s_per_wave), (unsigned)rows);
    idx_decode_kernel<HT, DI, FP8><<<grid, 256, 0, st>>>(
        q, a.w, k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L, s_per_wave, a.scores);
  }
  return hipGetLastError();
}

template <int DI, bool FP8>
static hipError_t dispatch_ht(const IndexerArgs& a, hipStream_t st) {
  switch (a.HI / 16) {
    case 1: return launch_mfma<1, DI, FP8>(a, st);
    case 2: return launch_mfma<2, DI, FP8>(a, st);
    case 4: return launch_mfma<4, DI, FP8>(a, st);
    case 8: return launch_mfma<8, DI, FP8>(a, st);
  }
  return hipErrorInvalidValue;
}

bool indexer_uses_mfma(const IndexerArgs& a) {
  if (a.q_dtype != SA_BF16 || (a.k_dtype != SA_BF16 && a.k_dtype != SA_FP8_E4M3)) return false;
  if (a.HI % 16) return false;
  const int ht = a.HI / 16;
  return ht == 1 || ht == 2 || ht == 4 || ht == 8;
}

template <typename QT, typename KT>
static hipError_t launch_vector(const IndexerArgs& a, hipStream_t st) {
  dim3 grid((a.L + kVecTile - 1) / kVecTile, (unsigned)((int64_t)a.B * a.T));
  size_t lds = sizeof(float) * ((size_t)(a.HI + kVecTile) * (a.dI + 1) + a.HI);
  idx_vector_kernel<QT, KT><<<grid, 256, lds, st>>>(
      (const QT*)a.q, a.w, (const KT*)a.k, a.k_scale, a.q_pos, a.kv_len, a.T,
      a.L, a.HI, a.dI, a.scores);
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st) {
  if (a.B == 0 || a.T == 0 || a.L == 0) return hipSuccess;
  if (indexer_uses_mfma(a)) {
    const bool fp8 = a.k_dtype == SA_FP8_E4M3;
    if (a.dI == 128) return fp8 ? dispatch_ht<128, true>(a, st) : dispatch_ht<128, false>(a, st);
    if (a.dI == 64) return fp8 ? dispatch_ht<64, true>(a, st) : dispatch_ht<64, false>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.q_dtype == SA_F32) {
    if (a.k_dtype == SA_F32) return launch_vector<float, float>(a, st);
    if (a.k_dtype == SA_BF16) return launch_vector<float, uint16_t>(a, st);
    return launch_vector<float, uint8_t>(a, st);
  }
  if (a.k_dtype == SA_F32) return launch_vector<uint16_t, float>(a, st);
  if (a.k_dtype == SA_BF16) return launch_vector<uint16_t, uint16_t>(a, st);
  return launch_vector<uint16_t, uint8_t>(a, st);
}

}  // namespace sa
