// index_core.hpp -- register operands of the lightning-indexer contraction,
// shared by the score kernels and the fused prefill select.
//
// The index score of query t at position s ("Sparse Attention 数学学习笔记"
// §9, I_{t,s} equation) is sum_h w_{t,h} ReLU(q_{t,h} . k_s).  One wave holds
// a query's H^I x d^I block as MFMA A operands and takes 16 positions per
// step; QueryRegs::score returns the same bits wherever it runs, so every
// kernel built on it computes identical scores for identical inputs.
#pragma once
#include "common.hpp"

namespace sa {

// Contraction-index map of k-step ks for lane group g (8 consecutive dims):
//   bf16 keys: dims [32 ks + 8 g, +8)       -> one 16-byte key load per step
//   fp8 keys : dims [64 (ks/2) + 16 g + 8 (ks%2), +8) -> one 16-byte key load
//              (16 codes) per two steps
template <bool FP8>
__device__ __forceinline__ int kmap(int ks, int g) {
  return FP8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g;
}

// ReLU of a contraction result in one VALU instruction, v_med3_f32(x, 0,
// +inf): max(x, 0) for every x that is not NaN, and 0 for a NaN (an MFMA
// result is a quiet NaN, and a median with a NaN operand is the smaller of
// the other two) -- what fmaxf(x, 0) gives.  fmaxf takes two instructions,
// the first quieting a signaling NaN that the compiler cannot rule out.  The
// bound is +inf in a scalar register (`inf` from inf_sgpr()): as a constant
// the compiler folds the median back into fmaxf.
__device__ __forceinline__ float inf_sgpr() {
  float v;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(v));
  return v;
}
__device__ __forceinline__ float relu_acc(float x, float inf) {
  return __builtin_amdgcn_fmed3f(x, 0.f, inf);
}

// Registers of one 16-position key chunk: KS bf16x8 B operands.
template <int DI, bool FP8>
struct KeyChunk {
  static constexpr int KS = DI / 32;
  static constexpr int NL = FP8 ? KS / 2 : KS;  // 16-byte loads per lane
  uintx4 raw[NL];
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int off = FP8 ? (64 * i + 16 * g) : (2 * (32 * i + 8 * g));
      raw[i] = *(const uintx4*)(row + off);
    }
  }
  // The same 16-byte pieces from a row stored with piece p at p ^ x (an LDS
  // tile swizzled against bank conflicts; the piece index of load i, lane
  // group g is 4 i + g for both key types).
  __device__ __forceinline__ void load_swz(const uint8_t* row, int g, int x) {
#pragma unroll
    for (int i = 0; i < NL; ++i) raw[i] = *(const uintx4*)(row + 16 * ((4 * i + g) ^ x));
  }
  __device__ __forceinline__ bf16x8 operand(int ks) const {
    if constexpr (!FP8) {
      return as_bf16x8(raw[ks]);
    } else {
      const uintx4& r = raw[ks >> 1];
      uint32_t c0 = (ks & 1) ? r[2] : r[0];
      uint32_t c1 = (ks & 1) ? r[3] : r[1];
      uint32_t o0, o1, o2, o3;
      fp8x4_to_bf16x4(c0, o0, o1);
      fp8x4_to_bf16x4(c1, o2, o3);
      return as_bf16x8(uintx4{o0, o1, o2, o3});
    }
  }
};

// Query operand: qa[ht][ks] = q[h = 16 ht + l%16][kmap(ks, l/16) .. +8]
template <int HT, int DI, bool FP8>
struct QueryRegs {
  static constexpr int KS = DI / 32;
  bf16x8 a[HT][KS];
  float wr[HT][4];
  __device__ __forceinline__ void load(const uint16_t* qrow, const float* wrow,
                                       int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a[ht][ks] = as_bf16x8(
            *(const uintx4*)(qrow + (int64_t)(16 * ht + n) * DI + kmap<FP8>(ks, g)));
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[ht][r] = wrow[16 * ht + 4 * g + r];
    }
  }
  // The same operands from the query rows staged in LDS (qs), row h's
  // 16-byte piece p stored at piece p ^ (h mod d^I/8), and the weights from
  // LDS too (ws, one float per head).
  __device__ __forceinline__ void load_lds(const uint8_t* qs, const float* ws, int lane) {
    constexpr int PPQ = DI / 8;  // 16-byte pieces per query row
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = 16 * ht + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int p = kmap<FP8>(ks, g) / 8;
        a[ht][ks] = as_bf16x8(*(const uintx4*)(qs + h * 2 * DI + 16 * (p ^ (h % PPQ))));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[ht][r] = ws[16 * ht + 4 * g + r];
    }
  }
  // Score of position (s0 + l%16), summed over all heads, valid in every lane.
  template <typename Chunk>
  __device__ __forceinline__ float score(const Chunk& kc) const {
    bf16x8 kb[KS];  // widened once, shared by every head tile
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = kc.operand(ks);
    const float inf = inf_sgpr();
    // head tiles in pairs, k-steps inside: the pair's products are
    // independent, so they issue back to back instead of waiting on one
    // accumulator chain
    float part = 0.f;
#pragma unroll
    for (int h0 = 0; h0 < HT; h0 += 2) {
      constexpr int NP = HT >= 2 ? 2 : 1;
      floatx4 acc[NP];
#pragma unroll
      for (int j = 0; j < NP; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < NP; ++j) acc[j] = mfma16x16x32(a[h0 + j][ks], kb[ks], acc[j]);
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) part = fmaf(wr[h0 + j][r], relu_acc(acc[j][r], inf), part);
    }
    return sum_over_lane_groups_vx(part);  // callers run it with the whole wave
  }
};

// Scores of two queries for the same key chunk, which is widened once.  Per
// head tile the two queries' products form two independent accumulator
// chains; each query's arithmetic is score()'s, in the same order, so the
// results carry the same bits.
template <int HT, int DI, bool FP8, typename Chunk>
__device__ __forceinline__ void score_pair(const QueryRegs<HT, DI, FP8>& q0,
                                           const QueryRegs<HT, DI, FP8>& q1, const Chunk& kc,
                                           float& s0, float& s1) {
  constexpr int KS = DI / 32;
  bf16x8 kb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kb[ks] = kc.operand(ks);
  const float inf = inf_sgpr();
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a0 = mfma16x16x32(q0.a[ht][ks], kb[ks], a0);
      a1 = mfma16x16x32(q1.a[ht][ks], kb[ks], a1);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) p0 = fmaf(q0.wr[ht][r], relu_acc(a0[r], inf), p0);
#pragma unroll
    for (int r = 0; r < 4; ++r) p1 = fmaf(q1.wr[ht][r], relu_acc(a1[r], inf), p1);
  }
  s0 = sum_over_lane_groups_vx(p0);
  s1 = sum_over_lane_groups_vx(p1);
}

}  // namespace sa
