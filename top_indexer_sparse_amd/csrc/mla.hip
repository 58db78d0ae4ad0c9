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
// heads each (one wave per SIMD) and walks a range of the query's slots 32
// rows at a time.  The 32 gathered rows (1152 bytes each: 1024 of c_kv, 128
// of k_rope) arrive in LDS by direct global->LDS copies
// (global_load_lds_dwordx4) into a ring of four tile buffers.  Per wave and
// tile:
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
// traffic); a single bf16 P would perturb each weight by up to 2^-8, which
// breaks a 2e-3 max-abs bound when few rows carry the mass.
// The tile loop is software-pipelined: step t computes S(t), then the
// previous tile's PV products with the softmax of S(t) issued between them;
// tiles t and t-1 are in use, t+1 and t+2 in flight.  At one wave per SIMD
// the loop is bound by LDS operand reads (each wave reads every K and V row
// of the tile), so K and V operands are fetched several MFMA steps ahead.
// The prologue also moves everything through global->LDS copies with explicit
// waits (index slice, then the queries, staged in two tile buffers), so the
// first tiles are requested while the queries are still arriving.
// Long index sets are split over work-groups (KV split); a combine kernel
// merges the partial (m, l, o) by log-sum-exp.
//
// mla_vector_kernel: fp32 vector ALU, any dc <= 512, dR <= 64, for fp32
// inputs (and bf16 outside the MFMA shape); one work-group per query.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace sa {

// f(integral_constant<I>) for I = B .. E-1, in order, at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA path
// ---------------------------------------------------------------------------
constexpr int kMlaDc = 512, kMlaDr = 64, kMlaD = kMlaDc + kMlaDr;
constexpr int kMlaRowB = kMlaD * 2;              // 1152 bytes per gathered row
constexpr int kMlaPieces = kMlaRowB / 16;        // 72 pieces of 16 bytes
constexpr int kMlaTile = 32;                     // rows per tile
constexpr int kMlaTileB = kMlaTile * kMlaRowB;   // 36864 bytes
constexpr int kMlaTileLoads = kMlaTileB / 1024;  // 36 wave-wide 16-byte-per-lane loads
constexpr int kMlaBuf = 4;                       // LDS tiles: 3 in flight + 1 in use
constexpr int kMlaMaxSplitSlots = 2048;          // index slice of one work-group

// Row r of a tile stores its 16-byte piece p at position p ^ swz(r) (inside
// the aligned group of 8 pieces, so c_kv and k_rope pieces stay apart).  With
// swz the Gray code of r's low bits, both the QK reads (16 rows, one piece
// each) and the PV transpose reads (4 rows x 4 half-pieces per lane group)
// hit distinct LDS banks.
__device__ __forceinline__ int row_swz(int r) { return (r ^ (r >> 1)) & 7; }

struct MlaKernelArgs {
  const uint16_t* q_lat;   // [BT, H, 512]
  const uint16_t* q_rope;  // [BT, H, 64]
  const uint8_t* c_kv;     // row (b,s) at + (b*L+s)*c_stride_b
  const uint8_t* k_rope;   // row (b,s) at + (b*L+s)*r_stride_b
  int64_t c_stride_b, r_stride_b;  // bytes
  const int32_t* idx;      // [BT, k]
  int k, T, L, H;
  int nsplit, slots_per_split;
  int packed;              // k_rope row = c_kv row + 1024 bytes, same stride
  float scale_log2;        // sm_scale * log2(e)
  float* out;              // [BT, H, 512]
  float* lse;              // [BT, H] or null
  float* part_o;           // [BT, H, nsplit, 512] when nsplit > 1
  float* part_ml;          // [BT, H, nsplit, 2]
  const uint8_t* win;      // row i of sequence b at + (b*n_win+i)*win_stride_b
  int64_t win_stride_b;
  int n_win;               // slots k .. k+n_win-1 read win rows 0 .. n_win-1
  int zero_rope;           // no RoPE part: q_rope and k_rope read as zeros
  // DENSE kernels: no index list; slot j of query (b, t) is position j for
  // every candidate j < min(q_pos[bt] + 1, kv_len[b], L) (either bound may be
  // null), and a split's slice is not bounded by the slot buffer.
  const int32_t* q_pos;
  const int32_t* kv_len;
  // optional [BT]: only the first count[bt] index slots can hold a position
  // (an ascending, -1 padded list), so later tiles are not fetched
  const int32_t* count;
};

// 128 zero bytes: the RoPE operand of rows that have none.
__device__ __attribute__((aligned(256))) uint8_t g_mla_zero[128];

// NW waves; one work-group per (query, head group, KV split).  Each wave owns
// 16 heads and 512 / DS of the output dims: with DS = 2, the two waves of a
// pair compute the same scores and softmax and split the value product, which
// halves the accumulators and lets two waves share a SIMD.
// PACKED: k_rope row = c_kv row + 1024 bytes with one stride ([B, L, 576]).
// DENSE: every candidate position, in order, instead of an index list.
template <int NW, bool PACKED, int DS, bool DENSE>
__global__ __launch_bounds__(64 * NW, 1) void mla_mfma_kernel(MlaKernelArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kMlaBuf][kMlaTileB];
  __shared__ int spos[kMlaMaxSplitSlots];                  // row to fetch (always valid)
  __shared__ uint32_t svmask[kMlaMaxSplitSlots / kMlaTile];  // bit r: row r counts

  // block -> (bt, head group, split); blocks that share (bt, split) are placed
  // on the same XCD (blocks are dealt to the 8 XCDs round-robin) so the head
  // groups' re-reads of the gathered rows hit that XCD's L2.
  constexpr int NH = NW / DS;  // head blocks of 16 per work-group
  constexpr int HW = 16 * NH;
  constexpr int ND = 32 / DS;  // d-tiles of 16 output dims per wave
  const int hgroups = a.H / HW;
  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int hg = lin % hgroups;
  const int split = (lin / hgroups) % a.nsplit;
  int64_t bt = lin / (hgroups * a.nsplit);
  // dense rows grow with the query position: the longest rows go first
  if constexpr (DENSE) bt = nblk / (hgroups * a.nsplit) - 1 - bt;
  const int b = (int)(bt / a.T);

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int hb = wave % NH, dh = wave / NH;  // head block, output-dim part
  const int h = hg * HW + hb * 16 + n;       // this lane's head

  const int j_begin = split * a.slots_per_split;
  // index slots, then window slots; dense: the query's candidate positions
  int kt = DENSE ? candidate_limit(a.q_pos, a.kv_len, b, bt, a.L) : a.k + a.n_win;
  if (!DENSE && a.count) kt = min(kt, max(0, a.count[bt]));
  const int nslots = max(0, min(kt, j_begin + a.slots_per_split) - j_begin);
  const uint32_t nrows = (uint32_t)(a.L + a.n_win);  // valid slot values

  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&tiles[0][0];
  const uint32_t lds_spos = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)&spos[0];

  // ---- prologue: every load is a global->LDS copy with an explicit wait ----
  // (the compiler tracks none of them, so no wait of its own drains the tile
  // copies issued later).  First the split's index slice into spos (slot j at
  // spos[j]; slots past the slice read a clamped in-row address and are
  // masked below), then the work-group's queries into tile buffers 2
  // and 3, laid out per (head block, k-step) as 1 KB runs in the MFMA B
  // operand order, so that the register loads below are conflict-free.
  const int wu = __builtin_amdgcn_readfirstlane(wave);  // wave index in an SGPR
  if constexpr (!DENSE) {
    const uint8_t* ib = uniform_ptr((const uint8_t*)(a.idx + bt * a.k));
    const int nrun = (nslots + 63) / 64;
    for (int r = wu; r < nrun; r += NW) {
      const int j = min(j_begin + 64 * r + lane, a.k - 1);
      dma4(ib, 4u * (uint32_t)j, lds_spos + 256u * (uint32_t)r);
    }
  }
  static_assert(kMlaBuf >= 4 && NH * 18 % NW == 0, "query staging layout");
  constexpr int kQRuns = NH * 18 / NW;  // 1 KB query runs per wave
  {
    const uint8_t* qlb = uniform_ptr((const uint8_t*)(a.q_lat + (bt * a.H + (int64_t)hg * HW) * kMlaDc));
    const uint8_t* qrb =
        a.zero_rope ? g_mla_zero
                    : uniform_ptr((const uint8_t*)(a.q_rope + (bt * a.H + (int64_t)hg * HW) * kMlaDr));
    const uint32_t qr_head = a.zero_rope ? 0u : 2u * kMlaDr;  // zero rows: one 128-byte row
    const int qn = lane >> 2, qg = lane & 3;
#pragma unroll
    for (int i = 0; i < kQRuns; ++i) {
      const int q = wu + NW * i;  // run q = (head block q / 18, k-step q % 18)
      const int qhb = q / 18, ks = q % 18;
      const uint32_t head = (uint32_t)(16 * qhb + qn);
      const uint32_t dst = lds0 + 2u * kMlaTileB + 1024u * (uint32_t)q;
      if (ks < 16)
        dma16(qlb, head * (2u * kMlaDc) + 64u * ks + 16u * qg, dst);
      else
        dma16(qrb, head * qr_head + 64u * (ks - 16) + 16u * qg, dst);
    }
  }
  wait_vmcnt<kQRuns>();  // this wave's index slice landed (the query runs may not)
  lds_barrier();         // every wave's slice landed
  if (a.n_win > 0 && j_begin + nslots > a.k) {  // window slots: positions L, L+1, ...
    for (int j = max(0, a.k - j_begin) + tid; j < nslots; j += 64 * NW) spos[j] = a.L + j_begin + j - a.k;
    wait_lgkm0();
    lds_barrier();
  }
  // Every slot of the slice is processed; a slot that holds no position in
  // [0, L) fetches row 0 and is masked out of the softmax.
  const int ntiles = (nslots + kMlaTile - 1) / kMlaTile;

  // ---- tile fetch: wave w < NH issues the 1 KB pieces q = NLD w .. NLD w + NLD - 1 ----
  // Lane l of load i fills 16-byte slot c = 64 q + l of the tile: row c / 72,
  // position c % 72, which holds piece (c % 72) ^ swz(row).  Rows and pieces
  // are the same for every tile, so they are computed once; per load only the
  // gathered row's position changes.  The packed layout (k_rope right after
  // c_kv in one row, as a [B, L, 576] cache) needs one base and one stride; a
  // split cache takes the piece's own base.
  static_assert(kMlaTileLoads % NH == 0, "equal loads per wave");
  constexpr int NLD = kMlaTileLoads / NH;  // loads per tile and issuing wave
  const uint8_t* cb = a.c_kv + (int64_t)b * a.L * a.c_stride_b;
  const uint8_t* rb = a.k_rope + (int64_t)b * a.L * a.r_stride_b;
  const uint8_t* wb = a.win + (int64_t)b * a.n_win * a.win_stride_b;
  const int wv = __builtin_amdgcn_readfirstlane(hb);
  const bool issuer = __builtin_amdgcn_readfirstlane(dh) == 0;
  uint32_t drow[NLD], dpiece[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int c = 64 * (NLD * wv + i) + lane;
    const int r = c / kMlaPieces, pp = c % kMlaPieces;
    drow[i] = 4 * r;                  // byte offset into a tile's slice of spos
    dpiece[i] = 16 * (pp ^ row_swz(r));
  }
  // Loads I0 <= i < I1 of this wave's share of tile tl.  A tile's loads are
  // issued in three parts spread over the previous tile's compute (each load
  // holds its wave at issue while the memory pipeline is busy), four at a
  // time behind one M0 write where the part allows.
  auto issue_part = [&](int tl, auto I0c, auto I1c) {
    constexpr int I0 = decltype(I0c)::value, I1 = decltype(I1c)::value;
    if (!issuer) return;
    const uint32_t dst = lds0 + (uint32_t)((tl % kMlaBuf) * kMlaTileB);
    const uint8_t* sp = (const uint8_t*)spos + 4 * tl * kMlaTile;
    // every row position first: the DMA asm carries a memory clobber, so a
    // position read placed after one DMA would wait out a full LDS round trip
    uint32_t srow[NLD];
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      if constexpr (DENSE) {  // slot j is position j_begin + j; past the slice: row 0
        const int j = tl * kMlaTile + (int)(drow[i] >> 2);
        srow[i] = j < nslots ? (uint32_t)(j_begin + j) : 0u;
      } else {
        srow[i] = *(const uint32_t*)(sp + drow[i]);
      }
    }
    auto voff = [&](int i) {  // packed layout: per-lane byte offset from cb
      const uint32_t s = srow[i] < nrows ? srow[i] : 0u;  // skipped slot: row 0
      return s * (uint32_t)a.c_stride_b + dpiece[i];
    };
    auto src = [&](int i) {  // split layout: per-lane address
      const uint32_t s = srow[i] < nrows ? srow[i] : 0u;
      if (dpiece[i] >= 1024u)
        return a.zero_rope ? g_mla_zero + (dpiece[i] & 1023u)
                           : rb + (s * (uint32_t)a.r_stride_b + (dpiece[i] & 1023u));
      if (s < (uint32_t)a.L) return cb + (s * (uint32_t)a.c_stride_b + dpiece[i]);
      return wb + ((s - (uint32_t)a.L) * (uint32_t)a.win_stride_b + dpiece[i]);
    };
    static_for<I0, I1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t ldst = dst + 1024u * (uint32_t)(NLD * wv + i);
      if constexpr ((i - I0) % 4 == 0 && i + 4 <= I1) {  // a group of four
        if constexpr (PACKED)
          dma16x4(cb, voff(i), voff(i + 1), voff(i + 2), voff(i + 3), ldst);
        else
          dma16x4_addr(src(i), src(i + 1), src(i + 2), src(i + 3), ldst);
      } else if constexpr ((i - I0) / 4 * 4 + 4 > I1 - I0) {  // past the last group
        if constexpr (PACKED)
          dma16(cb, voff(i), ldst);
        else
          dma16_addr(src(i), ldst);
      }
    });
  };
  static_assert(NLD == 9, "parts of 4, 4 and 1 loads");
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 4>;
  using P2 = std::integral_constant<int, 8>;
  using P3 = std::integral_constant<int, NLD>;
  auto issue = [&](int tl) { issue_part(tl, P0{}, P3{}); };

  // Tiles 0 and 1 go out now, behind the query runs; tile t + 2 is issued
  // while tile t is consumed.
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < ntiles) issue(t);
  // per-tile validity masks (bit r: slot 32 t + r holds a position in [0, L))
  constexpr int kSlotsPerThread = DENSE ? 0 : kMlaMaxSplitSlots / (64 * NW);
#pragma unroll
  for (int i = 0; i < kSlotsPerThread; ++i) {
    const int j0 = 64 * NW * i;
    if (j0 >= ntiles * kMlaTile) break;  // uniform
    const int j = j0 + tid;
    const bool ok = j < nslots && (uint32_t)spos[j] < nrows;
    const uint64_t m = __ballot(ok);  // 64 slots = two tiles
    const int t0 = j0 / kMlaTile + 2 * wave;  // this wave's first tile
    if (lane == 0 && t0 < ntiles) {
      svmask[t0] = (uint32_t)m;
      if (t0 + 1 < ntiles) svmask[t0 + 1] = (uint32_t)(m >> 32);
    }
  }
  // the query runs landed (they precede the tile copies); Q^T operand
  // qb[ks] = q[h][32 ks + 8 g .. +8], ks < 16 from q_lat, 16..17 from q_rope
  if (issuer && ntiles >= 2)
    wait_vmcnt<2 * NLD>();
  else if (issuer && ntiles == 1)
    wait_vmcnt<NLD>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  bf16x8 qb[18];
  {
    const uint8_t* qs = &tiles[2][0] + 18 * 1024 * hb + 16 * (4 * n + g);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qb[ks] = as_bf16x8(*(const uintx4*)(qs + 1024 * ks));
  }
  wait_lgkm0();
  lds_barrier();  // buffers 2 and 3 are free again
  // The step before the first multiplies a zero P by buffer 3: clear it so
  // that no stale LDS bits (a NaN pattern) reach the accumulators.
  {
    uintx4* zb = (uintx4*)tiles[kMlaBuf - 1];
    for (int i = tid; i < kMlaTileB / 16; i += 64 * NW) zb[i] = uintx4{0u, 0u, 0u, 0u};
  }

  floatx4 o[ND];  // d-tile ND dh + i
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane byte offsets of the swizzled reads
  const int mq = row_swz(n);                 // QK rows 16 jt + n
  const int qoff0 = 16 * (g ^ mq), qoff1 = 16 * ((4 + g) ^ mq);
  const int R = 4 * g + (n >> 2);            // PV rows R and R + 16
  const int mv = row_swz(R);
  int voff[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) voff[d4] = 16 * ((2 * d4 + ((n & 3) >> 1)) ^ mv) + 8 * (n & 1);

  // P = exp2(x - m_use) as bf16 hi + lo; returns the row sum of P.  The pair
  // carries ~16 significant bits, so the product stays at fp32-level accuracy
  // while the MFMAs stay bf16.
  auto make_p = [&](const float (&x)[8], float m_use, uint32_t (&ph)[4], uint32_t (&pl)[4]) {
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[e] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(x[e + 1] - m_use);
      psum += p0 + p1;
      const uint32_t hi = pack_bf16x2_rne(p0, p1);
      ph[e / 2] = hi;
      pl[e / 2] = pack_bf16x2_rne(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
    }
    return psum;
  };

  // O^T += V^T P^T for the tile in tb.  V^T operand: rows R..R+3 -> lane group
  // g, column 16 dt + lane%16 (see the transpose-read note in common.hpp);
  // piece 2 dt + (lane%4)/2, half lane%2.  The wave's ND d-tiles go in
  // chunks of two: a chunk loads the next chunk's operands, multiplies its own (the hi
  // and lo products of one accumulator separated by the other d-tile's
  // product) and then runs piece(chunk), a slice of other VALU work; a
  // scheduling barrier closes each chunk, so that work issues while the
  // matrix unit runs the chunk's four products.
  auto pv_mfma = [&](const uint8_t* tb, const uint32_t (&ph)[4], const uint32_t (&pl)[4],
                     auto&& piece) {
    const bf16x8 pBh = __builtin_bit_cast(bf16x8, uintx4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 pBl = __builtin_bit_cast(bf16x8, uintx4{pl[0], pl[1], pl[2], pl[3]});
    const uint8_t* v0 = tb + R * kMlaRowB + 32 * ND * dh;  // the wave's output dims
    const uint8_t* v1 = v0 + 16 * kMlaRowB;
    auto vop = [&](int dt) {
      const int off = 128 * (dt >> 2) + voff[dt & 3];
      shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (shortx4 __attribute__((address_space(3)))*)(v0 + off));
      shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (shortx4 __attribute__((address_space(3)))*)(v1 + off));
      return __builtin_bit_cast(
          bf16x8, uintx4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))});
    };
    // kPvAhead chunks of operands in flight: LDS reads return after a few
    // hundred cycles when the unit is busy, so one chunk ahead would stall
    // every chunk on its operands
    constexpr int kPvAhead = 3;
    bf16x8 vr[kPvAhead + 1][2];
    static_for<0, kPvAhead>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      vr[i][0] = vop(2 * i);
      vr[i][1] = vop(2 * i + 1);
    });
    static_for<0, ND / 2>([&](auto kc) {
      constexpr int c = decltype(kc)::value, dt = 2 * c;
      if constexpr (c + kPvAhead < ND / 2) {
        vr[(c + kPvAhead) % (kPvAhead + 1)][0] = vop(2 * (c + kPvAhead));
        vr[(c + kPvAhead) % (kPvAhead + 1)][1] = vop(2 * (c + kPvAhead) + 1);
      }
      const bf16x8 va = vr[c % (kPvAhead + 1)][0], vb = vr[c % (kPvAhead + 1)][1];
      o[dt] = mfma16x16x32(va, pBh, o[dt]);
      o[dt + 1] = mfma16x16x32(vb, pBh, o[dt + 1]);
      o[dt] = mfma16x16x32(va, pBl, o[dt]);
      o[dt + 1] = mfma16x16x32(vb, pBl, o[dt + 1]);
      piece(kc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_piece = [](auto) {};

  // Software pipeline over the tiles: step t multiplies S(t) = K(t) Q^T, then
  // runs the previous tile's PV products with the softmax of S(t) placed
  // between them, so the exponentials and conversions issue while the matrix
  // unit works.  Tiles t and t-1 are in use during step t; t+1 and t+2 are
  // in flight.  The accumulators are touched only by MFMAs inside the loop,
  // so they stay in AGPRs.  A wave leaves the loop when a score of tile t
  // exceeds its reference max by more than 8 (log2 units; always at the
  // first tile with a visible row): the rescale O *= 2^(m_old - m_new) runs
  // outside the loop, after the previous tile's products, redoes P(t) and
  // re-enters.  Weights exp2(x - m_run) therefore stay below 256.
  uint32_t pbh[4] = {0u, 0u, 0u, 0u}, pbl[4] = {0u, 0u, 0u, 0u};  // P(t - 1)
  int tl = 0;
  float x[8];
  float mt = -INFINITY;
  for (;;) {
    bool rescale = false;
  for (; tl < ntiles; ++tl) {
    // this wave's part of tile tl landed (loads return in order; tile tl+1
    // may still be in flight)
    if (tl + 1 < ntiles)
      wait_vmcnt<NLD>();
    else
      wait_vmcnt<0>();
    wait_lgkm0();
    lds_barrier();  // every wave's part landed; tile tl-2 no longer read
    const bool more = tl + 2 < ntiles;  // a tile left to fetch
    if (more) issue_part(tl + 2, P0{}, P1{});
    const uint8_t* tb = tiles[tl % kMlaBuf];
    const uint8_t* tp = tiles[(tl + kMlaBuf - 1) % kMlaBuf];
    uint32_t vm;
    if constexpr (DENSE) {  // the slice's first nslots slots count
      const int left = nslots - tl * kMlaTile;
      vm = (left >= kMlaTile ? 0xffffffffu : (1u << left) - 1u) >> (4 * g);
    } else {
      vm = svmask[tl] >> (4 * g);
    }

    // S^T[jt]: rows 16 jt + 4 g + r, head n.  The two row blocks are two
    // independent accumulator chains, interleaved.  K operands run kQkAhead
    // k-steps ahead of their products; scheduling barriers keep the reads in
    // k-step order, so the first product waits only for its own operands.
    floatx4 st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* r0 = tb + n * kMlaRowB;
      const uint8_t* r1 = r0 + 16 * kMlaRowB;
      auto kop = [&](const uint8_t* rp, int ks) {
        return *(const uintx4*)(rp + 128 * (ks >> 1) + ((ks & 1) ? qoff1 : qoff0));
      };
      constexpr int kQkAhead = 5;
      uintx4 k0[kQkAhead + 1], k1[kQkAhead + 1];
      static_for<0, kQkAhead>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        k0[i] = kop(r0, i);
        k1[i] = kop(r1, i);
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<0, 18>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + kQkAhead < 18) {
          k0[(ks + kQkAhead) % (kQkAhead + 1)] = kop(r0, ks + kQkAhead);
          k1[(ks + kQkAhead) % (kQkAhead + 1)] = kop(r1, ks + kQkAhead);
        }
        st0 = mfma16x16x32(as_bf16x8(k0[ks % (kQkAhead + 1)]), qb[ks], st0);
        st1 = mfma16x16x32(as_bf16x8(k1[ks % (kQkAhead + 1)]), qb[ks], st1);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    if (more) issue_part(tl + 2, P1{}, P2{});

    // previous tile's PV, with this tile's softmax in pieces between its
    // products: scale to log2 units and mask skipped slots, tile max per head
    // (then across the four lane groups), and P against the current
    // reference max.  P is computed even when the rescale path will redo it.
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
    uint32_t nph[4], npl[4];
    pv_mfma(tp, pbh, pbl, [&](auto kc) {
      constexpr int c = decltype(kc)::value;
      if constexpr (c < 2) {
        const floatx4& st = c == 0 ? st0 : st1;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          x[4 * c + r] = (vm >> (16 * c + r)) & 1u ? st[r] * a.scale_log2 : -INFINITY;
      } else if constexpr (c == 2) {
        mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                   fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      } else if constexpr (c >= 3 && c < 7) {
        const int e = 2 * (c - 3);
        const float p0 = __builtin_amdgcn_exp2f(x[e] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(x[e + 1] - m_use);
        psum += p0 + p1;
        const uint32_t hi = pack_bf16x2_rne(p0, p1);
        nph[e / 2] = hi;
        npl[e / 2] = pack_bf16x2_rne(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
      } else if constexpr (c == 7) {
        mt = max_over_lane_groups_vx(mt);
      }
    });
    // keep P in this block: only the rescale path discards it
    asm volatile("" ::"v"(nph[0]), "v"(nph[1]), "v"(nph[2]), "v"(nph[3]), "v"(npl[0]),
                 "v"(npl[1]), "v"(npl[2]), "v"(npl[3]), "v"(psum));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pbh[i] = nph[i];
      pbl[i] = npl[i];
    }
    if (more) issue_part(tl + 2, P2{}, P3{});
    if (__ballot(mt > m_run + 8.f)) {
      rescale = true;
      break;
    }
    l_run += psum;
  }
    if (!rescale) break;
    {
      // O holds the products up to tile tl-1; P(tl) is redone against the
      // new reference max
      const bool grow = mt > m_run + 8.f;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // 0 at first
      if (grow) m_run = mt;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i) o[i] *= alpha;
      l_run += make_p(x, m_run == -INFINITY ? 0.f : m_run, pbh, pbl);
      ++tl;
    }
  }
  // the last tile's products
  if (ntiles > 0) {
    pv_mfma(tiles[(ntiles - 1) % kMlaBuf], pbh, pbl, no_piece);
  }
  // ---- finish ----
  const float l_tot = sum_over_lane_groups(l_run);
  if (a.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = a.out + (bt * a.H + h) * (int64_t)kMlaDc;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      *(floatx4*)(orow + 16 * (ND * dh + dt) + 4 * g) = o[dt] * inv;
    if (a.lse && g == 0 && dh == 0)
      a.lse[bt * a.H + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t u = (bt * a.H + h) * a.nsplit + split;
    float* orow = a.part_o + u * kMlaDc;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) *(floatx4*)(orow + 16 * (ND * dh + dt) + 4 * g) = o[dt];
    if (g == 0 && dh == 0) {
      a.part_ml[2 * u] = m_run;
      a.part_ml[2 * u + 1] = l_tot;
    }
  }
}

// Merge of (query, head) u's nsplit <= NS partials, 512 dims, 128 threads:
// every load first (clamped split index, zero weight past nsplit), so the
// work-group waits for one memory round trip instead of three.
template <int NS>
__device__ __forceinline__ void mla_combine_small(const float* __restrict__ part_o,
                                                  const float* __restrict__ part_ml, int nsplit,
                                                  int64_t u, float* __restrict__ out,
                                                  float* __restrict__ lse) {
  constexpr int dc = 4 * 128;
  float2 ml[NS];
  floatx4 po[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int64_t us = u * nsplit + min(s, nsplit - 1);
    ml[s] = *(const float2*)(part_ml + 2 * us);
    po[s] = *(const floatx4*)(part_o + us * dc + 4 * threadIdx.x);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = s < nsplit ? fmaxf(M, ml[s].x) : M;
  const float Mu = M == -INFINITY ? 0.f : M;
  float Lsum = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = s < nsplit ? exp2f(ml[s].x - Mu) : 0.f;
    Lsum += wgt * ml[s].y;
    acc += wgt * po[s];
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  *(floatx4*)(out + u * dc + 4 * threadIdx.x) = acc * inv;
  if (lse && threadIdx.x == 0) lse[u] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : -INFINITY;
}

// Merge nsplit partial (m, l, o) of one (query, head): one 128-thread group,
// four output columns per thread.
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int nsplit, int dc,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lse) {
  // (bt, h), laid out over the XCDs as the MLA kernel lays out its blocks
  // (blocks go to the 8 XCDs round-robin; each XCD takes a contiguous run of
  // queries), so the partials are read from the L2 that they were written to
  int64_t u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (dc == 4 * 128) {  // uniform
    if (nsplit <= 4) return mla_combine_small<4>(part_o, part_ml, nsplit, u, out, lse);
    if (nsplit <= 8) return mla_combine_small<8>(part_o, part_ml, nsplit, u, out, lse);
    if (nsplit <= 16) return mla_combine_small<16>(part_o, part_ml, nsplit, u, out, lse);
  }
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
constexpr int kMlaWaves = 4;  // one wave per SIMD
constexpr int kMlaDs = 1;     // each wave computes all 512 output dims of its 16 heads
constexpr int kMlaHeadsWg = 16 * kMlaWaves / kMlaDs;  // 64

bool mla_uses_mfma(const MlaArgs& a) {
  return a.dtype == SA_BF16 && a.dc == kMlaDc && a.dR == kMlaDr && a.H % kMlaHeadsWg == 0;
}

bool mla_supported(const MlaArgs& a) {
  // the bf16 path addresses a sequence's rows with 32-bit byte offsets
  if (mla_uses_mfma(a))
    // (with 8 KB to spare: grouped copies raise the offsets by up to 4 KB)
    return (int64_t)a.L * a.c_stride * 2 < (1LL << 32) - 8192 &&
           (int64_t)a.L * a.r_stride * 2 < (1LL << 32) - 8192 &&
           (int64_t)a.n_win * a.win_stride * 2 < (1LL << 32) && (a.n_win == 0 || a.zero_rope) &&
           (a.dense == 0 || (a.k == a.L && a.n_win == 0));
  if (a.n_win || a.zero_rope || a.dense) return false;  // bf16 MFMA path only
  if (a.dc > 512 || a.dR > 64 || a.dR < 0 || a.dc < 1) return false;
  if ((int64_t)a.H * a.dc > 256 * kVecMaxOut) return false;
  return vector_lds_bytes(a.H, a.dc, a.dR) <= 64 * 1024;
}

// KV-split count for the MFMA path: enough work-groups to cover the CUs.
static int mla_nsplit(int64_t bt, int H, int k, bool dense) {
  const int64_t groups = bt * (H / kMlaHeadsWg);
  const int max_split = (k + 2 * kMlaTile - 1) / (2 * kMlaTile);  // >= 64 rows per split
  int ns = 1;
  // an index slice must fit the slot buffer; dense slices have none
  while (!dense && (int64_t)ns * kMlaMaxSplitSlots < k) ns *= 2;
  while (groups * ns < 256 && ns * 2 <= max_split) ns *= 2;
  return ns;
}

size_t mla_workspace_bytes(int dtype, int B, int T, int k, int H, int dc, bool dense) {
  if (dtype != SA_BF16 || dc != kMlaDc || H % kMlaHeadsWg) return 0;
  const int64_t bt = (int64_t)B * T;
  const int ns = mla_nsplit(bt, H, k, dense);
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
    m.packed = a.c_stride == a.r_stride && !a.zero_rope && a.n_win == 0 &&
               (const uint8_t*)a.k_rope == (const uint8_t*)a.c_kv + 2 * kMlaDc;
    m.win = (const uint8_t*)a.win;
    m.win_stride_b = a.win_stride * 2;
    m.n_win = a.n_win;
    m.zero_rope = a.zero_rope;
    m.q_pos = a.dense_q_pos;
    m.kv_len = a.dense_kv_len;
    m.count = a.count;
    // slots: the index set, then the window; dense: positions 0 .. L-1 (k = L)
    const int kt = a.k + a.n_win;
    m.idx = a.idx;
    m.k = a.k;
    m.T = a.T;
    m.L = a.L;
    m.H = a.H;
    m.nsplit = mla_nsplit(bt, a.H, kt, a.dense);
    m.slots_per_split = ((kt + m.nsplit - 1) / m.nsplit + kMlaTile - 1) / kMlaTile * kMlaTile;
    m.scale_log2 = scale_log2;
    m.out = a.out;
    m.lse = a.lse;
    if (m.nsplit > 1) {
      m.part_o = (float*)a.ws;
      m.part_ml = m.part_o + bt * a.H * m.nsplit * kMlaDc;
    }
    const int64_t nblk = bt * (a.H / kMlaHeadsWg) * m.nsplit;
    const dim3 grid((unsigned)nblk), block(64 * kMlaWaves);
    if (a.dense) {
      if (m.packed)
        mla_mfma_kernel<kMlaWaves, true, kMlaDs, true><<<grid, block, 0, st>>>(m);
      else
        mla_mfma_kernel<kMlaWaves, false, kMlaDs, true><<<grid, block, 0, st>>>(m);
    } else if (m.packed) {
      mla_mfma_kernel<kMlaWaves, true, kMlaDs, false><<<grid, block, 0, st>>>(m);
    } else {
      mla_mfma_kernel<kMlaWaves, false, kMlaDs, false><<<grid, block, 0, st>>>(m);
    }
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
