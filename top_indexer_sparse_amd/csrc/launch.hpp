// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel
// translation units.  Arguments arrive validated; launchers only enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// Candidate lists the decode indexer leaves for the Top-K select (few query
// rows, T = 1): every score work-group keeps the keys of its positions at or
// above a floor set so that, with high probability, it keeps all of its
// positions that are in the row's top k.  The select checks that afterwards
// and reads the score row instead when it does not hold.
struct IdxKeep {
  int4* info;   // [rows][nwg]: kept, candidates, floor key, max key
  uint2* keep;  // [rows][nwg][cap]: (key, position) of the kept keys, any order
  int nwg, cap, k;
};

struct IndexerArgs {
  const void* q;
  int q_dtype;
  const float* w;
  const void* k;
  int k_dtype;
  const float* k_scale;
  const int32_t* q_pos;
  const int32_t* kv_len;
  int B, T, L, HI, dI;
  float* scores;
  IdxKeep keep{};  // info == nullptr: scores only
};
bool indexer_uses_mfma(const IndexerArgs& a);
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st);

// Grid of the decode score kernel (few query rows): work-groups of 4 waves,
// each wave over at most kDecMaxSpan positions; long ranges amortise the
// query registers, so they are halved only until the grid has kDecTargetWgs
// work-groups (about 2 waves per SIMD).  Returns positions per wave.
constexpr int kDecMaxSpan = 1024;
constexpr int kDecTargetWgs = 512;
inline int dec_span(int64_t rows, int L) {
  int s = kDecMaxSpan;
  while (s > 64 && rows * ((L + 4 * s - 1) / (4 * s)) < kDecTargetWgs) s /= 2;
  return s;
}

// The select over the candidate lists (one work-group per row).
constexpr int kKeepMaxL = 131072;  // row bitmaps held in LDS
constexpr int kKeepMaxRows = 128;
bool keep_supported(const IndexerArgs& a, int k);
size_t keep_workspace_bytes(int64_t rows, int L);
IdxKeep keep_layout(void* ws, int64_t rows, int L, int k);
hipError_t launch_keep_select(const IdxKeep& kp, const float* scores, const int32_t* kv_len,
                              int rows, int L, int32_t* idx, int32_t* count, hipStream_t st);

// Fused prefill select (indexer scores + Top-K, the row held in LDS).
constexpr int kPrefillSelectMaxL = 32768;
constexpr int kPrefillSelectPairMaxL = 16384;  // two rows per work-group up to here
bool prefill_select_supported(const IndexerArgs& a, int topk);
hipError_t launch_prefill_select(const IndexerArgs& a, int topk, int32_t* idx, int32_t* count,
                                 hipStream_t st);

struct TopkArgs {
  const float* scores;
  const int32_t* q_pos;
  const int32_t* kv_len;
  int B, T, L, k;
  int32_t* idx;
  int32_t* count;
  void* ws;
};
constexpr int kTopkMaxK = 4096;
size_t topk_workspace_bytes(int B, int T, int L, int k);
bool topk_supported(int L, int k);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

struct MlaArgs {
  const void* q_lat;
  const void* q_rope;
  int dtype;  // q and kv dtype (equal)
  const void* c_kv;
  const void* k_rope;
  int64_t c_stride, r_stride;  // elements
  const int32_t* idx;
  int k, B, T, L, H, dc, dR;
  float sm_scale;
  float* out;
  float* lse;
  void* ws;
  // Optional (bf16 MFMA path): a second row source of n_win rows, reached by
  // n_win extra slots after the k index slots (slot k + i reads win row i),
  // and zero_rope = 1 for rows without a RoPE part (q_rope, k_rope unused).
  const void* win = nullptr;
  int64_t win_stride = 0;  // elements
  int n_win = 0;
  int zero_rope = 0;
  // Optional (bf16 MFMA path): dense = 1 attends to every candidate position
  // s < min(q_pos[bt] + 1, kv_len[b], L) with no index list (idx unused; k
  // must equal L).
  const int32_t* dense_q_pos = nullptr;
  const int32_t* dense_kv_len = nullptr;
  int dense = 0;
  // Optional (bf16 MFMA path): count[bt] bounds the index slots that can hold
  // a position (idx ascending and -1 padded after them).
  const int32_t* count = nullptr;
};
bool mla_uses_mfma(const MlaArgs& a);
bool mla_supported(const MlaArgs& a);
size_t mla_workspace_bytes(int dtype, int B, int T, int k, int H, int dc, bool dense = false);
hipError_t launch_mla(const MlaArgs& a, hipStream_t st);

struct BlockArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* krep;  // bf16 pooled block keys
  int B, L, Hq, Hkv, d, blk, nsel, n_sink, n_win;
  float sm_scale;
  int shared_choice;  // 1: one block choice per KV group (sum of its heads' scores)
  float* out;
  int32_t* blocks_out;
  void* ws;
};
bool block_supported(const BlockArgs& a);
size_t block_workspace_bytes(int B, int Hq, int L, int nsel, int Hkv, int d, int blk);
hipError_t launch_block_pool(const void* k, int B, int L, int Hkv, int d,
                             int blk, void* krep, hipStream_t st);
hipError_t launch_block_decode(const BlockArgs& a, hipStream_t st);

}  // namespace sa
