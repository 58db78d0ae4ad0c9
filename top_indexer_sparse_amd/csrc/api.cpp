// api.cpp -- the extern "C" entry points of libsparse_attn.so.
//
// Each entry point validates every argument on the host, then enqueues the
// kernels on the caller's stream.  Nothing is allocated and nothing waits.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "sparse_attn.h"

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SA_OK;
  return fail(SA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

size_t dtype_size(int dt) { return dt == SA_F32 ? 4 : dt == SA_BF16 ? 2 : dt == SA_FP8_E4M3 ? 1 : 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

int check_indexer(const sa::IndexerArgs& a) {
  REQUIRE(a.q && a.w && a.k && a.scores, SA_ERR_NULL, "indexer: q_idx, w, k_idx and scores are required");
  REQUIRE(a.B >= 0 && a.T >= 0 && a.L >= 0, SA_ERR_SHAPE, "indexer: negative size B=%d T=%d L=%d", a.B, a.T, a.L);
  REQUIRE(a.HI >= 1 && a.dI >= 1, SA_ERR_SHAPE, "indexer: HI=%d dI=%d must be >= 1", a.HI, a.dI);
  REQUIRE(a.q_dtype == SA_F32 || a.q_dtype == SA_BF16, SA_ERR_DTYPE, "indexer: q_dtype %d not in {F32, BF16}", a.q_dtype);
  REQUIRE(a.k_dtype == SA_F32 || a.k_dtype == SA_BF16 || a.k_dtype == SA_FP8_E4M3, SA_ERR_DTYPE,
          "indexer: k_dtype %d not in {F32, BF16, FP8_E4M3}", a.k_dtype);
  REQUIRE((a.k_dtype == SA_FP8_E4M3) == (a.k_scale != nullptr), SA_ERR_NULL,
          "indexer: k_scale is required for fp8 keys and must be NULL otherwise");
  REQUIRE(a.dI == 64 || a.dI == 128, SA_ERR_UNSUPPORTED, "indexer: dI=%d not in {64, 128}", a.dI);
  REQUIRE(a.HI <= 128, SA_ERR_UNSUPPORTED, "indexer: HI=%d > 128", a.HI);
  REQUIRE(sa::indexer_uses_mfma(a) || a.HI <= 64, SA_ERR_UNSUPPORTED,
          "indexer: HI=%d > 64 needs the bf16 MFMA path (bf16 q, bf16/fp8 k, HI in {16,32,64,128})", a.HI);
  REQUIRE(aligned16(a.q) && aligned16(a.w) && aligned16(a.k) && aligned16(a.scores) &&
              aligned16(a.k_scale) && aligned16(a.q_pos) && aligned16(a.kv_len),
          SA_ERR_ALIGN, "indexer: every pointer must be 16-byte aligned");
  return SA_OK;
}

int check_topk(const sa::TopkArgs& a, size_t ws_bytes) {
  REQUIRE(a.scores && a.idx, SA_ERR_NULL, "topk: scores and idx are required");
  REQUIRE(a.B >= 0 && a.T >= 0 && a.L >= 0, SA_ERR_SHAPE, "topk: negative size B=%d T=%d L=%d", a.B, a.T, a.L);
  REQUIRE(a.k >= 1, SA_ERR_SHAPE, "topk: k=%d must be >= 1", a.k);
  REQUIRE(sa::topk_supported(a.L, a.k), SA_ERR_UNSUPPORTED,
          "topk: k=%d, L=%d outside the compiled set (k <= %d, ceil(L/32768)*k <= 32768)", a.k, a.L,
          sa::kTopkMaxK);
  REQUIRE(aligned16(a.scores) && aligned16(a.idx) && aligned16(a.count) && aligned16(a.q_pos) &&
              aligned16(a.kv_len) && aligned16(a.ws),
          SA_ERR_ALIGN, "topk: every pointer must be 16-byte aligned");
  const size_t need = sa::topk_workspace_bytes(a.B, a.T, a.L, a.k);
  REQUIRE(need == 0 || (a.ws && ws_bytes >= need), SA_ERR_WORKSPACE,
          "topk: workspace of %zu bytes required, %zu given", need, a.ws ? ws_bytes : (size_t)0);
  return SA_OK;
}

int check_mla(const sa::MlaArgs& a, size_t ws_bytes) {
  REQUIRE(a.q_lat && a.c_kv && a.idx && a.out, SA_ERR_NULL, "mla: q_lat, c_kv, idx and out are required");
  REQUIRE(a.dR == 0 || (a.q_rope && a.k_rope), SA_ERR_NULL, "mla: q_rope and k_rope are required when dR > 0");
  REQUIRE(a.B >= 0 && a.T >= 0 && a.L >= 1 && a.k >= 1 && a.H >= 1 && a.dc >= 1 && a.dR >= 0, SA_ERR_SHAPE,
          "mla: bad size B=%d T=%d L=%d k=%d H=%d dc=%d dR=%d", a.B, a.T, a.L, a.k, a.H, a.dc, a.dR);
  REQUIRE(a.dtype == SA_F32 || a.dtype == SA_BF16, SA_ERR_DTYPE, "mla: dtype %d not in {F32, BF16}", a.dtype);
  REQUIRE(a.c_stride >= a.dc && (a.dR == 0 || a.r_stride >= a.dR), SA_ERR_SHAPE,
          "mla: row strides (%lld, %lld) shorter than the rows (%d, %d)", (long long)a.c_stride,
          (long long)a.r_stride, a.dc, a.dR);
  REQUIRE(sa::mla_supported(a), SA_ERR_UNSUPPORTED,
          "mla: (dtype=%d, H=%d, dc=%d, dR=%d) outside the compiled set", a.dtype, a.H, a.dc, a.dR);
  const size_t es = dtype_size(a.dtype);
  REQUIRE(aligned16(a.q_lat) && aligned16(a.q_rope) && aligned16(a.c_kv) && aligned16(a.k_rope) &&
              aligned16(a.idx) && aligned16(a.out) && aligned16(a.lse) && aligned16(a.ws) &&
              (a.c_stride * es) % 16 == 0 && (a.dR == 0 || (a.r_stride * es) % 16 == 0),
          SA_ERR_ALIGN, "mla: pointers and row strides must keep 16-byte alignment");
  const size_t need = sa::mla_workspace_bytes(a.dtype, a.B, a.T, a.k, a.H, a.dc, a.dense != 0);
  REQUIRE(need == 0 || (a.ws && ws_bytes >= need), SA_ERR_WORKSPACE,
          "mla: workspace of %zu bytes required, %zu given", need, a.ws ? ws_bytes : (size_t)0);
  return SA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// decode workspace layout: scores [B, L] f32 | idx [B, k] | count [B] | topk ws or the
// indexer's candidate lists | mla ws
struct DecodeWs {
  size_t scores, idx, count, topk, mla, total;
};
// n_win window slots follow the k index slots in the attention stage
DecodeWs decode_ws(int B, int L, int k, int H, int dc, int kv_dtype, int n_win = 0) {
  DecodeWs w{};
  size_t off = 0;
  w.scores = off;
  off = align256(off + (size_t)B * L * sizeof(float));
  w.idx = off;
  off = align256(off + (size_t)B * k * sizeof(int32_t));
  w.count = off;
  off = align256(off + (size_t)B * sizeof(int32_t));
  w.topk = off;  // the top-k's scratch, or the indexer's candidate lists
  const size_t tk = sa::topk_workspace_bytes(B, 1, L, k), kl = sa::keep_workspace_bytes(B, L);
  off = align256(off + (tk > kl ? tk : kl));
  w.mla = off;
  off = align256(off + sa::mla_workspace_bytes(kv_dtype, B, 1, k + n_win, H, dc));
  w.total = off;
  return w;
}

// Scores and Top-K of a decode step (T = 1).  Where the MFMA score kernel
// runs, it also leaves per-work-group candidate lists in the top-k region of
// the workspace and the select reads those (falling back to the scores row
// by itself); otherwise the top-k runs over the scores.
int index_and_select(sa::IndexerArgs ia, const sa::TopkArgs& ta, void* topk_ws, hipStream_t st) {
  const bool keep = sa::keep_supported(ia, ta.k);
  if (keep) ia.keep = sa::keep_layout(topk_ws, ia.B, ia.L, ta.k);
  int s = hip_status(sa::launch_indexer(ia, st), "decode indexer launch");
  if (s != SA_OK) return s;
  if (keep)
    return hip_status(sa::launch_keep_select(ia.keep, ta.scores, ta.kv_len, ta.B, ta.L, ta.idx,
                                             ta.count, st),
                      "decode select launch");
  return hip_status(sa::launch_topk(ta, st), "decode topk launch");
}

// The prefill select runs staged (stage 1 into a score buffer, then stage 2)
// where that is faster than the fused select, and wherever rows are longer
// than the fused select holds on chip.  Measured on MI355X (k = 2048, H^I =
// 64, d^I = 128, bf16, the last T queries of an L-token context), staged
// against fused: 93 against 99 us at T = L = 2048, 250 against 300 at T = L
// = 4096, 1.03 against 1.19 ms at T = 4096, L = 16384, 2.48 against 2.89 ms
// at T = L = 16384, 0.96 against 1.12 ms at T = 1024, L = 32768 (the fused
// select keeps one row per work-group there).  The fused select wins with
// fewer rows: 111 against 153 us (fused against staged) at T = 1024, L =
// 4096, 346 against 496 us at T = 1024, L = 16384, and by nearly 3x at
// T <= 256.
constexpr int kPrefillStagedMinRows = 2048;
constexpr int kPrefillStagedMinL = 2048;
constexpr int kPrefillStagedLongRows = 1024;  // rows per sequence when L > 16384
// Staged chunks of query rows per sequence: as many as a 1 GiB score buffer
// holds, at least 4096 (512 score work-groups, enough to fill the GPU), at
// most T.  One chunk keeps the score kernel's heaviest-rows-first order over
// the whole sequence.
constexpr size_t kPrefillScoreBudget = 1ull << 30;
constexpr int kPrefillChunkRows = 4096;
bool prefill_staged(int T, int L, int k) {
  if (T <= 0) return false;
  if (L > sa::kPrefillSelectMaxL) return true;
  return sa::topk_supported(L, k) &&
         ((T >= kPrefillStagedMinRows && L >= kPrefillStagedMinL) ||
          (T >= kPrefillStagedLongRows && L > 16384));
}

// prefill workspace layout: idx [B, T, k] | count [B, T] | mla ws (the larger
// of the sparse and the dense attention's) | when the select runs staged:
// chunk scores [chunk, L] | top-k ws of one chunk
struct PrefillWs {
  size_t idx, count, mla, scores, topk, total;
  int chunk;  // query rows per staged chunk (0: the fused select runs)
};
PrefillWs prefill_ws(int B, int T, int L, int k, int H, int dc) {
  PrefillWs w{};
  size_t off = 0;
  w.idx = off;
  off = align256(off + (size_t)B * T * k * sizeof(int32_t));
  w.count = off;
  off = align256(off + (size_t)B * T * sizeof(int32_t));
  w.mla = off;
  const size_t ms = sa::mla_workspace_bytes(SA_BF16, B, T, k, H, dc);
  const size_t md = sa::mla_workspace_bytes(SA_BF16, B, T, L < 1 ? 1 : L, H, dc, true);
  off = align256(off + (ms > md ? ms : md));
  w.chunk = 0;
  w.scores = w.topk = off;
  if (prefill_staged(T, L, k)) {
    const int64_t fit = (int64_t)(kPrefillScoreBudget / ((size_t)L * sizeof(float)));
    const int64_t rows = fit > kPrefillChunkRows ? fit : kPrefillChunkRows;
    w.chunk = T < rows ? T : (int)rows;
    off = align256(off + (size_t)w.chunk * L * sizeof(float));
    w.topk = off;
    off = align256(off + sa::topk_workspace_bytes(1, w.chunk, L, k < 1 ? 1 : k));
  }
  w.total = off;
  return w;
}

// staged: the prefill entry point selects through chunked score buffers, so
// rows above the fused select's limit are accepted
int check_prefill_select(const sa::IndexerArgs& a, int k, bool staged = false) {
  int s = check_indexer(a);
  if (s != SA_OK) return s;
  REQUIRE(k >= 1, SA_ERR_SHAPE, "prefill_select: k=%d must be >= 1", k);
  REQUIRE(a.L >= 1, SA_ERR_SHAPE, "prefill_select: L=%d must be >= 1", a.L);
  REQUIRE(sa::prefill_select_supported(a, k) ||
              (staged && sa::indexer_uses_mfma(a)),
          SA_ERR_UNSUPPORTED,
          "prefill_select: (q_dtype=%d, k_dtype=%d, HI=%d, dI=%d, L=%d) outside the compiled set "
          "(bf16 queries, bf16/fp8 keys, HI in {16,32,64,128}, dI in {64,128}, L <= %d)",
          a.q_dtype, a.k_dtype, a.HI, a.dI, a.L, sa::kPrefillSelectMaxL);
  return SA_OK;
}

// Scratch of sparse_attn_decode_noalloc: one array per GPU the library runs
// on, held until the process ends.  Host code never uses the array's name as
// an address (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device,
// and is kept in g_scratch_ptr.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (resolved on first use).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_ERR_UNSUPPORTED, "decode_noalloc: device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "decode_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

int sparse_attn_indexer_scores(const void* q_idx, int q_dtype, const float* w, const void* k_idx,
                               int k_dtype, const float* k_scale, const int32_t* q_pos,
                               const int32_t* kv_len, int B, int T, int L, int HI, int dI,
                               float* scores, void* stream) {
  clear_error();
  sa::IndexerArgs a{q_idx, q_dtype, w, k_idx, k_dtype, k_scale, q_pos, kv_len, B, T, L, HI, dI, scores};
  int s = check_indexer(a);
  if (s != SA_OK) return s;
  return hip_status(sa::launch_indexer(a, (hipStream_t)stream), "indexer launch");
}

int sparse_attn_topk(const float* scores, const int32_t* q_pos, const int32_t* kv_len, int B, int T,
                     int L, int k, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                     void* stream) {
  clear_error();
  sa::TopkArgs a{scores, q_pos, kv_len, B, T, L, k, idx, count, ws};
  int s = check_topk(a, ws_bytes);
  if (s != SA_OK) return s;
  return hip_status(sa::launch_topk(a, (hipStream_t)stream), "topk launch");
}

int sparse_attn_mla_forward(const void* q_lat, const void* q_rope, int q_dtype, const void* c_kv,
                            const void* k_rope, int kv_dtype, int64_t c_stride, int64_t r_stride,
                            const int32_t* idx, int k, int B, int T, int L, int H, int dc, int dR,
                            float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  clear_error();
  if (q_dtype != kv_dtype) return fail(SA_ERR_DTYPE, "mla: q_dtype %d != kv_dtype %d", q_dtype, kv_dtype);
  sa::MlaArgs a{q_lat, q_rope, q_dtype, c_kv, k_rope, c_stride, r_stride, idx, k, B, T, L, H, dc, dR,
                sm_scale, out, lse, ws};
  int s = check_mla(a, ws_bytes);
  if (s != SA_OK) return s;
  return hip_status(sa::launch_mla(a, (hipStream_t)stream), "mla launch");
}

int sparse_attn_decode(const void* q_idx, int q_idx_dtype, const float* w, const void* k_idx,
                       int k_dtype, const float* k_scale, const int32_t* kv_len, int B, int L,
                       int HI, int dI, int k, const void* q_lat, const void* q_rope, int q_dtype,
                       const void* c_kv, const void* k_rope, int kv_dtype, int64_t c_stride,
                       int64_t r_stride, int H, int dc, int dR, float sm_scale, float* out,
                       float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (q_dtype != kv_dtype) return fail(SA_ERR_DTYPE, "decode: q_dtype %d != kv_dtype %d", q_dtype, kv_dtype);
  if (!ws) return fail(SA_ERR_WORKSPACE, "decode: a workspace is required");
  if (!aligned16(ws)) return fail(SA_ERR_ALIGN, "decode: workspace must be 16-byte aligned");
  const DecodeWs lay = decode_ws(B < 0 ? 0 : B, L < 0 ? 0 : L, k < 1 ? 1 : k, H, dc, kv_dtype);
  char* base = (char*)ws;
  float* scores = (float*)(base + lay.scores);
  int32_t* idx = idx_out ? idx_out : (int32_t*)(base + lay.idx);
  int32_t* count = (int32_t*)(base + lay.count);
  sa::IndexerArgs ia{q_idx, q_idx_dtype, w, k_idx, k_dtype, k_scale, nullptr, kv_len, B, 1, L, HI, dI, scores};
  sa::TopkArgs ta{scores, nullptr, kv_len, B, 1, L, k, idx, count, base + lay.topk};
  sa::MlaArgs ma{q_lat, q_rope, q_dtype, c_kv, k_rope, c_stride, r_stride, idx, k, B, 1, L, H, dc, dR,
                 sm_scale, out, lse, base + lay.mla};
  int s = check_indexer(ia);
  if (s == SA_OK) s = check_topk(ta, lay.mla - lay.topk);
  if (s == SA_OK) s = check_mla(ma, lay.total - lay.mla);
  if (s == SA_OK && ws_bytes < lay.total)
    s = fail(SA_ERR_WORKSPACE, "decode: workspace of %zu bytes required, %zu given", lay.total, ws_bytes);
  if (s != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  s = index_and_select(ia, ta, base + lay.topk, st);
  if (s == SA_OK) s = hip_status(sa::launch_mla(ma, st), "decode mla launch");
  return s;
}

int sparse_attn_decode_noalloc(const void* q_idx, int q_idx_dtype, const float* w, const void* k_idx,
                               int k_dtype, const float* k_scale, const int32_t* kv_len, int B, int L,
                               int HI, int dI, int k, const void* q_lat, const void* q_rope,
                               int q_dtype, const void* c_kv, const void* k_rope, int kv_dtype,
                               int64_t c_stride, int64_t r_stride, int H, int dc, int dR,
                               float sm_scale, float* out, float* lse, int32_t* idx_out,
                               void* stream) {
  clear_error();
  REQUIRE(B >= 0 && L >= 0, SA_ERR_SHAPE, "decode_noalloc: negative size B=%d L=%d", B, L);
  const size_t need = decode_ws(B, L, k < 1 ? 1 : k, H, dc, kv_dtype).total;
  REQUIRE(need <= kScratchBytes, SA_ERR_WORKSPACE,
          "decode_noalloc: these sizes need %zu bytes of scratch, above the library's fixed %zu "
          "(use sparse_attn_decode with a workspace)",
          need, kScratchBytes);
  void* ws = nullptr;
  int s = scratch_address(&ws);
  if (s != SA_OK) return s;
  return sparse_attn_decode(q_idx, q_idx_dtype, w, k_idx, k_dtype, k_scale, kv_len, B, L, HI, dI, k,
                            q_lat, q_rope, q_dtype, c_kv, k_rope, kv_dtype, c_stride, r_stride, H, dc,
                            dR, sm_scale, out, lse, idx_out, ws, kScratchBytes, stream);
}

int sparse_attn_prefill_select(const void* q_idx, int q_dtype, const float* w, const void* k_idx,
                               int k_dtype, const float* k_scale, const int32_t* q_pos,
                               const int32_t* kv_len, int B, int T, int L, int HI, int dI, int k,
                               int32_t* idx, int32_t* count, void* stream) {
  clear_error();
  // the score buffer is not used: any non-null pointer passes the indexer checks
  sa::IndexerArgs a{q_idx, q_dtype, w, k_idx, k_dtype, k_scale, q_pos, kv_len, B, T, L, HI, dI,
                    (float*)idx};
  REQUIRE(idx, SA_ERR_NULL, "prefill_select: idx is required");
  int s = check_prefill_select(a, k);
  if (s != SA_OK) return s;
  REQUIRE(aligned16(count), SA_ERR_ALIGN, "prefill_select: count must be 16-byte aligned");
  return hip_status(sa::launch_prefill_select(a, k, idx, count, (hipStream_t)stream),
                    "prefill_select launch");
}

int sparse_attn_prefill(const void* q_idx, int q_idx_dtype, const float* w, const void* k_idx,
                        int k_dtype, const float* k_scale, const int32_t* q_pos,
                        const int32_t* kv_len, int B, int T, int L, int HI, int dI, int k,
                        const void* q_lat, const void* q_rope, const void* c_kv,
                        const void* k_rope, int64_t c_stride, int64_t r_stride, int H, int dc,
                        int dR, float sm_scale, int mode, float* out, float* lse,
                        int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  REQUIRE(mode == SA_PREFILL_SPARSE || mode == SA_PREFILL_DENSE || mode == SA_PREFILL_AUTO,
          SA_ERR_SHAPE, "prefill: mode %d not in {SPARSE, DENSE, AUTO}", mode);
  REQUIRE(B >= 0 && T >= 0 && L >= 1 && k >= 1, SA_ERR_SHAPE,
          "prefill: bad size B=%d T=%d L=%d k=%d", B, T, L, k);
  const bool dense = mode == SA_PREFILL_DENSE || (mode == SA_PREFILL_AUTO && L <= k);
  if (!ws) return fail(SA_ERR_WORKSPACE, "prefill: a workspace is required");
  if (!aligned16(ws)) return fail(SA_ERR_ALIGN, "prefill: workspace must be 16-byte aligned");
  const PrefillWs lay = prefill_ws(B, T, L, k, H, dc);
  char* base = (char*)ws;
  int32_t* idx = idx_out ? idx_out : (int32_t*)(base + lay.idx);
  int32_t* count = (int32_t*)(base + lay.count);
  sa::IndexerArgs ia{q_idx, q_idx_dtype, w, k_idx, k_dtype, k_scale, q_pos, kv_len, B, T, L, HI, dI,
                     (float*)idx};
  sa::MlaArgs ma{q_lat, q_rope, SA_BF16, c_kv, k_rope, c_stride, r_stride, idx, k, B, T, L, H, dc, dR,
                 sm_scale, out, lse, base + lay.mla};
  if (dense) {
    ma.idx = idx;  // unused by the dense attention
    ma.k = L;
    ma.dense = 1;
    ma.dense_q_pos = q_pos;
    ma.dense_kv_len = kv_len;
  }
  int s = dense ? SA_OK : check_prefill_select(ia, k, lay.chunk > 0);
  if (s == SA_OK && !dense && lay.chunk > 0) {
    REQUIRE(sa::topk_supported(L, k), SA_ERR_UNSUPPORTED,
            "prefill: k=%d, L=%d outside the top-k set", k, L);
  }
  if (s == SA_OK) s = check_mla(ma, lay.total - lay.mla);
  if (s == SA_OK && !sa::mla_uses_mfma(ma))
    s = fail(SA_ERR_UNSUPPORTED, "prefill: the attention needs the bf16 MLA path (dc=512, dR=64, H %% 64 == 0)");
  if (s == SA_OK && (!aligned16(q_pos) || !aligned16(kv_len) || !aligned16(idx_out)))
    s = fail(SA_ERR_ALIGN, "prefill: pointers must be 16-byte aligned");
  if (s == SA_OK && ws_bytes < lay.total)
    s = fail(SA_ERR_WORKSPACE, "prefill: workspace of %zu bytes required, %zu given", lay.total, ws_bytes);
  if (s != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (!dense && lay.chunk == 0) {
    s = hip_status(sa::launch_prefill_select(ia, k, idx, count, st), "prefill select launch");
  } else if (!dense) {
    // staged select per sequence and chunk of query rows (one-sequence views)
    const size_t qrow = (size_t)HI * dI * 2, krow = (size_t)dI * (k_dtype == SA_FP8_E4M3 ? 1 : 2);
    float* scores = (float*)(base + lay.scores);
    for (int b = 0; b < B && s == SA_OK; ++b) {
      for (int t0 = 0; t0 < T && s == SA_OK; t0 += lay.chunk) {
        const int tc = T - t0 < lay.chunk ? T - t0 : lay.chunk;
        const int64_t r0 = (int64_t)b * T + t0;
        sa::IndexerArgs ci{(const char*)q_idx + r0 * qrow, q_idx_dtype, w + r0 * HI,
                           (const char*)k_idx + (int64_t)b * L * krow, k_dtype,
                           k_scale ? k_scale + (int64_t)b * L : nullptr, q_pos ? q_pos + r0 : nullptr,
                           kv_len ? kv_len + b : nullptr, 1, tc, L, HI, dI, scores};
        sa::TopkArgs ct{scores, q_pos ? q_pos + r0 : nullptr, kv_len ? kv_len + b : nullptr, 1, tc, L, k,
                        idx + r0 * k, count + r0, base + lay.topk};
        s = hip_status(sa::launch_indexer(ci, st), "prefill chunk indexer launch");
        if (s == SA_OK) s = hip_status(sa::launch_topk(ct, st), "prefill chunk topk launch");
      }
    }
  }
  if (!dense) ma.count = count;  // the select's lists are ascending and -1 padded
  if (s == SA_OK) s = hip_status(sa::launch_mla(ma, st), "prefill attention launch");
  return s;
}

int sparse_attn_csa_decode(const void* q_idx, int q_idx_dtype, const float* w, const void* k_idx,
                           int k_dtype, const float* k_scale, const int32_t* n_comp, int B, int Lc,
                           int HI, int dI, int k, const void* q, const void* comp, const void* win,
                           int n_win, int H, int c, float sm_scale, float* out, float* lse,
                           int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  REQUIRE(q && comp && out, SA_ERR_NULL, "csa_decode: q, comp and out are required");
  REQUIRE(n_win >= 0 && (n_win == 0 || win), SA_ERR_NULL, "csa_decode: win is required when n_win > 0");
  REQUIRE(c == 512 && H >= 64 && H % 64 == 0, SA_ERR_UNSUPPORTED,
          "csa_decode: c=%d, H=%d outside the compiled set (c = 512, H a multiple of 64)", c, H);
  REQUIRE(aligned16(win), SA_ERR_ALIGN, "csa_decode: win must be 16-byte aligned");
  if (!ws) return fail(SA_ERR_WORKSPACE, "csa_decode: a workspace is required");
  if (!aligned16(ws)) return fail(SA_ERR_ALIGN, "csa_decode: workspace must be 16-byte aligned");
  const DecodeWs lay = decode_ws(B < 0 ? 0 : B, Lc < 0 ? 0 : Lc, k < 1 ? 1 : k, H, c, SA_BF16, n_win);
  char* base = (char*)ws;
  float* scores = (float*)(base + lay.scores);
  int32_t* idx = idx_out ? idx_out : (int32_t*)(base + lay.idx);
  int32_t* count = (int32_t*)(base + lay.count);
  sa::IndexerArgs ia{q_idx, q_idx_dtype, w, k_idx, k_dtype, k_scale, nullptr, n_comp, B, 1, Lc, HI, dI, scores};
  sa::TopkArgs ta{scores, nullptr, n_comp, B, 1, Lc, k, idx, count, base + lay.topk};
  // keys = values = entries: the latent part is the entry, the RoPE part is absent
  sa::MlaArgs ma{q, nullptr, SA_BF16, comp, nullptr, c, 0, idx, k, B, 1, Lc, H, c, 64,
                 sm_scale, out, lse, base + lay.mla};
  ma.win = win;
  ma.win_stride = c;
  ma.n_win = n_win;
  ma.zero_rope = 1;
  int s = check_indexer(ia);
  if (s == SA_OK) s = check_topk(ta, lay.mla - lay.topk);
  if (s == SA_OK) {
    REQUIRE(sa::mla_supported(ma), SA_ERR_UNSUPPORTED, "csa_decode: entries beyond 4 GiB per sequence");
    REQUIRE(aligned16(q) && aligned16(comp) && aligned16(out) && aligned16(lse) && aligned16(idx_out),
            SA_ERR_ALIGN, "csa_decode: pointers must be 16-byte aligned");
    if (ws_bytes < lay.total)
      s = fail(SA_ERR_WORKSPACE, "csa_decode: workspace of %zu bytes required, %zu given", lay.total,
               ws_bytes);
  }
  if (s != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  s = index_and_select(ia, ta, base + lay.topk, st);
  if (s == SA_OK) s = hip_status(sa::launch_mla(ma, st), "csa attention launch");
  return s;
}

int sparse_attn_block_pool(const void* k, int B, int L, int Hkv, int d, int blk, void* krep,
                           void* stream) {
  clear_error();
  REQUIRE(B >= 0 && L >= 0 && Hkv >= 1 && blk >= 1, SA_ERR_SHAPE, "block_pool: bad size");
  // krep holds L / blk blocks: with no complete block it may be NULL
  REQUIRE(k && (krep || L / blk == 0), SA_ERR_NULL, "block_pool: k and krep are required");
  REQUIRE(d == 128, SA_ERR_UNSUPPORTED, "block_pool: d=%d not 128", d);
  REQUIRE(blk == 32 || blk == 64 || blk == 128, SA_ERR_UNSUPPORTED, "block_pool: blk=%d not in {32,64,128}", blk);
  REQUIRE(aligned16(k) && aligned16(krep), SA_ERR_ALIGN, "block_pool: pointers must be 16-byte aligned");
  return hip_status(sa::launch_block_pool(k, B, L, Hkv, d, blk, krep, (hipStream_t)stream), "block_pool launch");
}

int sparse_attn_block_decode(const void* q, const void* k, const void* v, const void* krep, int B,
                             int L, int Hq, int Hkv, int d, int blk, int nsel, int n_sink,
                             int n_win, float sm_scale, int shared_choice, float* out,
                             int32_t* blocks_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  sa::BlockArgs a{q, k, v, krep, B, L, Hq, Hkv, d, blk, nsel, n_sink, n_win, sm_scale,
                  shared_choice, out, blocks_out, ws};
  REQUIRE(shared_choice == 0 || shared_choice == 1, SA_ERR_SHAPE,
          "block_decode: shared_choice must be 0 or 1");
  REQUIRE(B >= 0 && L >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && n_sink >= 0 && n_win >= 0 && nsel >= 1,
          SA_ERR_SHAPE, "block_decode: bad size");
  // with no complete block (L < blk) krep holds nothing and may be NULL
  REQUIRE(q && k && v && out && (krep || L / blk == 0), SA_ERR_NULL,
          "block_decode: q, k, v, krep and out are required");
  REQUIRE(sa::block_supported(a), SA_ERR_UNSUPPORTED, "block_decode: dims outside the compiled set");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(krep) && aligned16(out) &&
              aligned16(blocks_out) && aligned16(ws),
          SA_ERR_ALIGN, "block_decode: pointers must be 16-byte aligned");
  const size_t need = sa::block_workspace_bytes(B, Hq, L, nsel, Hkv, d, blk);
  REQUIRE(need == 0 || (ws && ws_bytes >= need), SA_ERR_WORKSPACE,
          "block_decode: workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
  return hip_status(sa::launch_block_decode(a, (hipStream_t)stream), "block_decode launch");
}

size_t sparse_attn_workspace_bytes(int op, int B, int T, int L, int k, int H, int dc) {
  if (B < 0 || T < 0 || L < 0 || k < 1) return 0;
  switch (op) {
    case SA_OP_TOPK:
      return sa::topk_workspace_bytes(B, T, L, k);
    case SA_OP_MLA_FORWARD:
      return sa::mla_workspace_bytes(SA_BF16, B, T, k, H, dc);
    case SA_OP_DECODE:
      return decode_ws(B, L, k, H, dc, SA_BF16).total;
    case SA_OP_BLOCK_DECODE:  // (B, Hq, L, nsel, Hkv, d) passed as (B, T, L, k, H, dc)
      return sa::block_workspace_bytes(B, T, L, k, H, dc, 32);
    case SA_OP_CSA_DECODE:  // (B, n_win, Lc, k, H, c) passed as (B, T, L, k, H, dc)
      return decode_ws(B, L, k, H, dc, SA_BF16, T).total;
    case SA_OP_PREFILL:
      return prefill_ws(B, T, L, k, H, dc).total;
  }
  return 0;
}

const char* sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
  }
  return "SA_UNKNOWN_STATUS";
}

const char* sparse_attn_last_error(void) { return g_err; }

}  // extern "C"
