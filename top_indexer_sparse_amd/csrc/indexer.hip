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
//    16 positions per step through a register ring of 8 chunks (4 for the
//    largest query blocks); a query's chunks are dealt to its waves in turn.
//    The ReLU * w reduction over
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
#include "split_select.hpp"

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
// One query per grid row; the query's waves share its positions chunk by
// chunk.  A chunk is 16 consecutive key rows, one contiguous run of 16 x ROWB
// bytes, and each wave moves its chunks into a ring of R LDS slots of its
// own with global->LDS copies of 1 KB each: every copy covers whole 128-byte
// lines, where a load straight into B-operand registers covers 16 rows x 64
// bytes (half a line per row), and the key path holds no registers.  A slot
// is refilled as soon as its chunk is in registers, so with two slots two
// chunks are in flight during each chunk's contraction.  A slot stores row
// r's 16-byte piece p at piece p ^ (r mod pieces-per-row), so the B-operand
// reads of 16 rows at one piece hit distinct banks.  The loop body is free of
// conditional memory operations: copies are always issued (rows past the
// range are clamped to its last valid row and their scores ignored), and
// scores go to a per-wave LDS buffer.  The scores (times the fp8 scale) leave
// with coalesced stores after the loop.
constexpr int kDecRing = 2;
constexpr int kDecBuf = kDecMaxSpan + 16 * kDecRing;  // + the ring's overrun

// With KEEP, the work-group also leaves its candidate list for the Top-K
// select (IdxKeep): n_w candidates here (positions < lim with a key), of
// which the row's top k hold about p n_w, p = min(1, k / lim), give or take
// sqrt(p n_w (1 - p)) when the large scores are spread over the row (the
// dealing of chunks to waves spreads every 64-position run of a 1024-position
// stretch over a different work-group).  The work-group keeps its r1 = p n_w
// + 5 sd + 2 largest keys, rounded down to a bin of a histogram fitted to its
// key range: every key >= the floor key of that bin.
template <int HT, int DI, bool FP8, bool KEEP>
__global__ __launch_bounds__(256) void idx_decode_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ kscale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kv_len,
    int T, int L, float* __restrict__ scores, IdxKeep kp) {
  constexpr int HI = 16 * HT;
  constexpr int ROWB = FP8 ? DI : 2 * DI;  // bytes per key row
  constexpr int NSC = kDecMaxSpan / 64;    // prefetched scales per lane
  constexpr int R = kDecRing;
  constexpr int CHB = 16 * ROWB;           // bytes per chunk
  constexpr int NB = CHB / 1024;           // 1 KB copies per chunk
  constexpr int PPR = ROWB / 16;           // 16-byte pieces per row
  static_assert(NB == 1 || NB == 2 || NB == 4, "chunk of 1, 2 or 4 KB");
  __shared__ float sbuf[4][kDecBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t kring[4][R][CHB];
  const int64_t bt = blockIdx.y;
  const int b = (int)(bt / T);
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int lim = candidate_limit(q_pos, kv_len, b, bt, L);
  float* out = scores + bt * L;
  const int v_end = min(lim, L);  // positions [0, v_end) need a score
  for (int s = v_end + (int)(blockIdx.x * 256 + threadIdx.x); s < L; s += (int)gridDim.x * 256)
    out[s] = -INFINITY;
  // The query's 16-position chunks are dealt to its W waves in turn: wave wq
  // takes chunks wq, wq + W, wq + 2 W, ..., so the waves sweep the key rows
  // together (contiguous ranges per wave finished up to a third apart).  A
  // wave has at most (positions per wave of the grid) / 16 <= 64 chunks.
  const int W = gridDim.x * 4, wq = blockIdx.x * 4 + wave;
  const int nch_all = (v_end + 15) / 16;
  const int nch = wq < nch_all ? (nch_all - wq + W - 1) / W : 0;
  // no wave of the work-group has a chunk (the same for all four waves)
  if (!KEEP && (int)blockIdx.x * 4 >= nch_all) return;
  const uint8_t* kb = k + (int64_t)b * L * ROWB;
  auto pos_of = [&](int c, int j) { return 16 * (wq + c * W) + j; };

  // Copy e of a chunk fills the slot's 1 KB block e: lane l writes 16-byte
  // position 64 e + l, row r = (64 e + l) / PPR, which holds piece
  // (position mod PPR) ^ (r mod PPR) of key row min(chunk start + r,
  // v_end - 1).  Rows and pieces are the same for every chunk.
  int crow[NB], cpiece[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int c = 64 * e + lane, r = c / PPR;
    crow[e] = r;
    cpiece[e] = 16 * ((c % PPR) ^ (r % PPR));
  }
  const uint32_t lring =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&kring[wave][0][0];
  auto issue = [&](int c, int slot) {
    const int p0 = 16 * (wq + c * W);
    const uint8_t* src[NB];
#pragma unroll
    for (int e = 0; e < NB; ++e)
      src[e] = kb + (int64_t)min(p0 + crow[e], v_end - 1) * ROWB + cpiece[e];
    const uint32_t dst = lring + (uint32_t)(slot * CHB);
    if constexpr (NB == 4) {
      dma16x4_addr(src[0], src[1], src[2], src[3], dst);
    } else {
#pragma unroll
      for (int e = 0; e < NB; ++e) dma16_addr(src[e], dst + 1024u * e);
    }
  };

  // The query block goes out first, then the fp8 scales, then the ring's
  // first R chunks; the wait after them completes the older loads and leaves
  // the ring in flight.  The loop is then entered, as it is continued, with
  // exactly the ring's copies outstanding, so each chunk's wait counts the
  // copies of the R - 1 younger chunks.  No load the compiler tracks may be
  // pending when the loop is entered with a use inside it: the compiler
  // cannot see the copies, so its own wait for such a load would count them
  // as done and drain the ring on every pass.  A query block that fits the
  // score buffer (with its weights) is therefore copied there once per
  // work-group (the four waves share it; row h's 16-byte piece p at
  // p ^ (h mod d^I/8), the weights after the block) and read into registers
  // before any score is written; a larger one is loaded by each wave and
  // waited for before the ring goes out.
  constexpr int QB = 2 * HI * DI;  // query block bytes
  constexpr int PPQ = DI / 8;      // 16-byte pieces per query row
  constexpr int NWC = (HI + 63) / 64;  // 256-byte weight copies
  constexpr bool QST = QB % 1024 == 0 && QB + 256 * NWC <= (int)sizeof(sbuf);
  QueryRegs<HT, DI, FP8> qr;
  if constexpr (QST) {
    const uint8_t* qg = uniform_ptr((const uint8_t*)(q + bt * HI * DI));
    const uint8_t* wg = uniform_ptr((const uint8_t*)(w + bt * HI));
    const uint32_t lq =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&sbuf[0][0];
    for (int e = wave; e < QB / 1024; e += 4) {
      const int c = 64 * e + lane, r = c / PPQ;
      dma16(qg, (uint32_t)(r * 2 * DI + 16 * ((c % PPQ) ^ (r % PPQ))), lq + 1024u * e);
    }
    if (wave == 0) {
#pragma unroll
      for (int e = 0; e < NWC; ++e)  // lanes past H^I repeat the last weight
        dma4(wg, 4u * (uint32_t)min(64 * e + lane, HI - 1), lq + (uint32_t)QB + 256u * e);
    }
  } else {
    qr.load(q + bt * HI * DI, w + bt * HI, lane);
    wait_vmcnt<0>();
  }
  float scr[FP8 ? NSC : 1];  // fp8 per-token scales of this lane's output slots
  if constexpr (FP8) {
    if (nch > 0) {
      const float* scb = kscale + (int64_t)b * L;
#pragma unroll
      for (int i = 0; i < NSC; ++i)
        scr[i] = scb[min(pos_of(4 * i + (lane >> 4), lane & 15), v_end - 1)];
    }
  }
  asm volatile("" ::: "memory");  // issued before the ring, as the waits assume
  if (nch > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) issue(i, i);
    wait_vmcnt<R * NB>();  // the query and the scales (older than the ring) have landed
  } else {
    wait_vmcnt<0>();
  }
  if constexpr (QST) {
    lds_barrier();  // every wave's query copies landed
    qr.load_lds((const uint8_t*)&sbuf[0][0], (const float*)((const uint8_t*)&sbuf[0][0] + QB),
                lane);
    wait_lgkm0();
    lds_barrier();  // every wave holds its query registers: the score buffer is free
  }
  if (!KEEP && nch == 0) return;  // the candidate list needs every wave

  float* sb = sbuf[wave];
  if (nch > 0) {
    for (int c0 = 0; c0 < nch; c0 += R) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = c0 + i;  // chunks past nch are computed and dropped
        wait_vmcnt<(R - 1) * NB>();  // chunk c landed; the younger one may not have
        asm volatile("" ::: "memory");
        KeyChunk<DI, FP8> kc;
        kc.load_swz(&kring[wave][i][n * ROWB], g, n & (PPR - 1));
        wait_lgkm0();  // the slot's reads are done before it is refilled
        issue(c + R, i);
        const float sc = qr.score(kc);
        sb[16 * c + n] = sc;  // the four lane groups write the same value
      }
    }
    wait_vmcnt<0>();  // no copy outlives the wave
  }
  // the wave's own LDS writes are ordered before these reads; slot i of a
  // lane is position j = lane % 16 of chunk 4 i + lane / 16 (64-byte runs)
  uint32_t key[KEEP ? NSC : 1];
#pragma unroll
  for (int i = 0; i < NSC; ++i) {
    const int c = 4 * i + (lane >> 4), s = pos_of(c, lane & 15);
    const bool valid = c < nch && s < v_end;
    if (valid) {
      float v = sb[16 * c + (lane & 15)];
      if constexpr (FP8) v *= scr[i];
      out[s] = v;
      if constexpr (KEEP) key[i] = score_key(v);
    } else if constexpr (KEEP) {
      key[i] = 0u;  // not a candidate
    }
  }
  if constexpr (KEEP) {
    __shared__ __align__(16) int hist[kSpBins];
    __shared__ int wn[4], nkept;
    __shared__ uint32_t wmin[4], wmax[4];
    const int tid = threadIdx.x;
    // ---- the work-group's candidates and their key range ----
    int nv = 0;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
      nv += key[i] != 0u;
      mn = key[i] ? min(mn, key[i]) : mn;
      mx = max(mx, key[i]);
    }
    nv = wave_total(nv);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    for (int i = tid; i < kSpBins; i += 256) hist[i] = 0;
    if (tid == 0) nkept = 0;
    if (lane == 0) {
      wn[wave] = nv;
      wmin[wave] = mn;
      wmax[wave] = mx;
    }
    __syncthreads();
    const int n_w = wn[0] + wn[1] + wn[2] + wn[3];
    const uint32_t kmin = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    const uint32_t kmax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float p = fminf(1.f, (float)kp.k / (float)max(lim, 1));
    const float mean = p * (float)n_w;
    const int r1 = min(n_w, (int)ceilf(mean + 5.f * sqrtf(mean * (1.f - p)) + 2.f));
    uint32_t lo = kmin;  // all of them
    if (n_w > r1) {      // uniform over the work-group
      const int sh = max(0, 32 - __clz(kmax - kmin) - 11);  // (range >> sh) < 2048
#pragma unroll
      for (int i = 0; i < NSC; ++i) hist_add(hist, (key[i] - kmin) >> sh, key[i] != 0u);
      __syncthreads();
      int bin, above, total;
      wave_rank_bin(hist, r1, bin, above, total);  // every wave, the same bin
      lo = kmin + ((uint32_t)bin << sh);
    }
    // ---- the keys >= lo, compacted (any order): one LDS atomic per wave ----
    int nk = 0;
#pragma unroll
    for (int i = 0; i < NSC; ++i) nk += key[i] != 0u && key[i] >= lo;
    const int inc = wave_scan_incl(nk);
    int wbase = 0;
    if (lane == 63) wbase = atomicAdd(&nkept, inc);
    int o = __builtin_amdgcn_readlane(wbase, 63) + inc - nk;
    const int64_t unit = bt * kp.nwg + blockIdx.x;
    uint2* dst = kp.keep + unit * kp.cap;
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
      if (key[i] != 0u && key[i] >= lo) {
        dst[o] = make_uint2(key[i], (uint32_t)pos_of(4 * i + (lane >> 4), lane & 15));
        ++o;
      }
    }
    __syncthreads();  // every wave's count is in
    if (tid == 0) kp.info[unit] = make_int4(nkept, n_w, (int)lo, (int)kmax);
  }
}

// Eight waves = eight consecutive queries of one sequence; 64-position key
// tiles staged in LDS (each row's 16-byte pieces swizzled by the row index,
// so the waves' operand reads and the staging stores avoid bank conflicts).
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
  constexpr int LROW = ROWB;                      // LDS row: pieces swizzled, not padded
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

  // staging: global->LDS copies, no registers in between.  Copy i of wave w
  // fills the tile's 1 KB block w + 8 i: lane l writes 16-byte slot 64 blk + l
  // (row r = slot / CPR, stored piece slot % CPR), so it reads piece
  // (slot % CPR) ^ (r % CPR) of key row r, clamped to the last candidate.
  constexpr int NBLK = CPT / 64;
  constexpr int PERW = (NBLK + kPfWaves - 1) / kPfWaves;
  const uint32_t lds_t = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&tile[0][0];
  const uint32_t lds_s = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&tscale[0][0];
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // in a scalar register
  auto gcopy = [&](int buf, int tl) {
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
      const int blk = wave_s + kPfWaves * i;
      if (blk < NBLK) {  // uniform over the wave
        const int slot = 64 * blk + lane;
        const int r = slot / CPR, o = (slot % CPR) ^ (r & (CPR - 1));
        const int sr = min(tl * kPfTile + r, lim_max - 1);
        dma16_addr(kb + (int64_t)sr * ROWB + 16 * o,
                   lds_t + (uint32_t)(buf * kPfTile * LROW + 1024 * blk));
      }
    }
    if (scb && wave_s == kPfWaves - 1)
      dma4(uniform_ptr((const uint8_t*)scb), 4u * (uint32_t)min(tl * kPfTile + lane, lim_max - 1),
           lds_s + (uint32_t)(4 * kPfTile * buf));
  };

  gcopy(0, 0);
  wait_vmcnt<0>();
  lds_barrier();
  for (int tl = 0; tl < ntiles; ++tl) {
    const int buf = tl & 1;
    // the other buffer was last read before the previous barrier
    if (tl + 1 < ntiles) gcopy(buf ^ 1, tl + 1);
    const int base = tl * kPfTile;
    if (active && base < lim) {
#pragma unroll
      for (int c = 0; c < kPfTile / 16; ++c) {
        const int s0 = base + 16 * c;
        if (s0 >= lim) break;
        KeyChunk<DI, FP8> kc;
        kc.load_swz(&tile[buf][(16 * c + n) * LROW], g, n & (CPR - 1));
        float sc = qr.score(kc);
        const int s = s0 + n;
        if (g == 0 && s < lim) {
          if (scb) sc *= tscale[buf][16 * c + n];
          out[s] = sc;
        }
      }
    }
    wait_vmcnt<0>();  // this wave's copies of the next tile landed
    lds_barrier();    // every wave's copies landed; this tile's reads are done
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
    const int64_t rows = (int64_t)a.B * a.T;
    const int s_per_wave = dec_span(rows, a.L);
    dim3 grid((a.L + 4 * s_per_wave - 1) / (4 * s_per_wave), (unsigned)rows);
    if (a.keep.info)  // the candidate lists' geometry follows this grid (keep_layout)
      idx_decode_kernel<HT, DI, FP8, true><<<grid, 256, 0, st>>>(
          q, a.w, k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L, a.scores, a.keep);
    else
      idx_decode_kernel<HT, DI, FP8, false><<<grid, 256, 0, st>>>(
          q, a.w, k, a.k_scale, a.q_pos, a.kv_len, a.T, a.L, a.scores, a.keep);
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
