// common.hpp -- device helpers shared by the gfx950 kernels of libsparse_attn.
//
// Lane layouts of the bf16 MFMA instructions used here (checked on gfx950):
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     lane l supplies A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16], e < 8,
//     and holds D[4*(l/16) + r][l%16], r < 4.
// The contraction index may be permuted freely as long as A and B use the same
// permutation; the kernels rely on that to load 16-byte runs.
//
// ds_read_b64_tr_b16 (gfx950 LDS transpose read): inside each group of 16
// lanes, lane i receives as element r the 16-bit value at position i%4 of the
// 8-byte chunk addressed by lane 4*r + i/4 of the same group.  Pointing lane
// 4*r + q at row (R0 + r), columns (C0 + 4q .. C0 + 4q + 3) of a row-major
// bf16 tile therefore gives lane i the column C0 + i of rows R0 .. R0 + 3: the
// operand layout of a product contracted over rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __builtin_bit_cast(float, packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __builtin_bit_cast(float, packed & 0xffff0000u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{lo, hi}, bf16x2));
}
// Exact packing of two fp32 values that are representable in bf16.
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi),
                               __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

// Four OCP e4m3fn codes (one dword) -> four bf16 values (two dwords), exact:
// every e4m3fn value, subnormals included, is representable in bf16.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t codes, uint32_t& out01,
                                                uint32_t& out23) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
  out01 = pack_bf16x2_exact(lo[0], lo[1]);
  out23 = pack_bf16x2_exact(hi[0], hi[1]);
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b,
                                                const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uintx4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum / max over the four lanes {l, l^16, l^32, l^48}.
__device__ __forceinline__ float sum_over_lane_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ float max_over_lane_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// The same maximum through gfx950's v_permlane16_swap / v_permlane32_swap
// (VALU lane exchanges, no LDS round trip).  With both operands equal, the
// swap hands every lane the pair {v[l], v[l ^ 16]} (then {.., v[l ^ 32]}) in
// its two results, so max(r0, r1) is the pair maximum in every lane.  Needs
// all 64 lanes active.
__device__ __forceinline__ float max_over_lane_groups_vx(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  u = __builtin_bit_cast(uint32_t, v);
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)t[0]), __builtin_bit_cast(float, (uint32_t)t[1]));
}

// Sum over the four lanes {l, l^16, l^32, l^48} by the same lane exchanges.
// The result is pinned (empty asm) where it is computed, so the compiler
// cannot sink the exchanges into a divergent branch that uses the sum: with
// lanes switched off they would read stale values.  Needs all 64 lanes
// active at the call.
__device__ __forceinline__ float sum_over_lane_groups_vx(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  u = __builtin_bit_cast(uint32_t, v);
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)t[0]) + __builtin_bit_cast(float, (uint32_t)t[1]);
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ---- global->LDS DMA and explicit waits ----
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// One wave-wide global->LDS load: lane l's 16 bytes at gbase + voff land at
// LDS byte lds_base + 16 l.  Issued as inline asm so that the compiler neither
// tracks it nor inserts its own (whole-queue) waits before LDS reads; the
// pipeline waits explicitly with wait_vmcnt.  The instruction has no register
// result.
__device__ __forceinline__ void dma16(const uint8_t* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// The same with a full 64-bit per-lane address.
__device__ __forceinline__ void dma16_addr(const uint8_t* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(gaddr)
               : "memory", "m0");
}
// Four wave-wide global->LDS loads behind one M0 write: load e (e < 4) copies
// lane l's 16 bytes at gbase + v_e to LDS byte lds_base + 1024 e + 16 l.  The
// instruction offset 1024 e moves both the global and the LDS address, so it
// is taken back out of the per-lane offset; the SGPR base is lowered by 4096
// and every offset raised by as much, so that no offset wraps (callers keep
// v_e + 4096 below 2^32).  Four copies with one M0 write leave the issuing
// wave sooner than four separately issued ones.
__device__ __forceinline__ void dma16x4(const uint8_t* gbase, uint32_t v0, uint32_t v1,
                                        uint32_t v2, uint32_t v3, uint32_t lds_base) {
  const uint8_t* gb = gbase - 4096;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072"
      :
      : "s"(lds_base), "v"(v0 + 4096u), "v"(v1 + 3072u), "v"(v2 + 2048u), "v"(v3 + 1024u), "s"(gb)
      : "memory", "m0");
}
// The same with full 64-bit per-lane addresses.
__device__ __forceinline__ void dma16x4_addr(const uint8_t* a0, const uint8_t* a1,
                                             const uint8_t* a2, const uint8_t* a3,
                                             uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "global_load_lds_dwordx4 %2, off offset:1024\n\t"
      "global_load_lds_dwordx4 %3, off offset:2048\n\t"
      "global_load_lds_dwordx4 %4, off offset:3072"
      :
      : "s"(lds_base), "v"(a0), "v"(a1 - 1024), "v"(a2 - 2048), "v"(a3 - 3072)
      : "memory", "m0");
}
// One wave-wide global->LDS load of 4 bytes per lane: lane l's dword at
// gbase + voff lands at LDS byte lds_base + 4 l.
__device__ __forceinline__ void dma4(const uint8_t* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// A wave-uniform pointer, moved to SGPRs (for the SGPR base of the copies).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// Work-group barrier without the memory fence of __syncthreads (which would
// also wait for the tiles still in flight); "memory" keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Candidate limit of a query row: positions s < limit are candidates.
__device__ __forceinline__ int candidate_limit(const int32_t* q_pos,
                                               const int32_t* kv_len, int b,
                                               int64_t bt, int L) {
  int lim = L;
  if (kv_len) lim = min(lim, max(kv_len[b], 0));
  if (q_pos) lim = min(lim, max(q_pos[bt] + 1, 0));
  return lim;
}

}  // namespace sa
