/*
 * sparse_attn.h -- C ABI of libsparse_attn.so: DSA-style top-k sparse
 * attention on AMD Instinct MI355X (gfx950).
 *
 * The hot path has three stages.
 *   1. Lightning indexer: every cached position s gets an index score
 *        I[t,s] = sum_h w[t,h] * ReLU(q_idx[t,h,:] . k_idx[s,:])
 *      ("Sparse Attention 数学学习笔记", §9 DSA; "MLA 与稀疏注意力：少存一点，
 *      还是少看一点？", DSA section, index-score equation).
 *   2. Top-K: S_t = the k candidates with the largest I[t,s], causal
 *      (s <= t) in prefill, ties to the lower position (same DSA sections;
 *      the selected-position helper of the second page orders by
 *      (-score, position)).
 *   3. Sparse MLA over S_t only, read from the latent cache: the score of a
 *      row j for head h is
 *        s[h,j] = (q_lat[h,:] . c_kv[j,:] + q_rope[h,:] . k_rope[j,:]) * sm_scale
 *      where q_lat = U_K^T q^C is the absorbed query and q_rope, k_rope are
 *      already rotated ("MLA 与稀疏注意力", full-score section); one softmax over
 *      S_t ("Sparse Attention 数学学习笔记", §2-§3); the value is aggregated
 *      in latent space, out[h,:] = sum_j softmax(s[h,:])_j c_kv[j,:], and U_V
 *      is applied by the caller ("MLA 与稀疏注意力", absorption section).
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no device memory and keeps no state between calls; scratch
 *    memory comes from the caller through (ws, ws_bytes), sized by
 *    sparse_attn_workspace_bytes().
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without waiting for it.
 *  - Arguments are validated before anything is enqueued: a non-zero return
 *    means no work was enqueued (except SA_ERR_HIP, returned when a launch
 *    itself fails).  sparse_attn_last_error() then gives a description.
 *  - Tensors are dense, row-major (C order), in the shapes given, except the
 *    latent cache rows, which may be strided (c_stride / r_stride elements
 *    between consecutive rows, so a packed [B, L, dc + dR] cache passes
 *    k_rope = c_kv + dc and c_stride = r_stride = dc + dR).
 *  - Every pointer must be 16-byte aligned, and every row stride must keep
 *    the rows 16-byte aligned (SA_ERR_ALIGN).
 *  - Positions are 0-based int32.
 *  - Floating point: inputs in the given storage dtype; all products are
 *    accumulated in fp32; scores and attention outputs are fp32.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  SA_ERR_SHAPE = 2,       /* a size is out of range (<= 0, T > L, ...)         */
  SA_ERR_DTYPE = 3,       /* unknown dtype code or unsupported combination     */
  SA_ERR_ALIGN = 4,       /* a pointer or a row stride breaks 16-byte alignment */
  SA_ERR_UNSUPPORTED = 5, /* dims outside the compiled set                     */
  SA_ERR_WORKSPACE = 6,   /* ws is NULL or smaller than required               */
  SA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed        */
} sa_status;

typedef enum {
  SA_F32 = 0,
  SA_BF16 = 1,
  SA_FP8_E4M3 = 2 /* OCP FP8 E4M3 ("e4m3fn": no infinities, max 448) */
} sa_dtype;

/* Operation codes for sparse_attn_workspace_bytes. */
typedef enum {
  SA_OP_TOPK = 0,
  SA_OP_MLA_FORWARD = 1,
  SA_OP_DECODE = 2,
  SA_OP_BLOCK_DECODE = 3,
  SA_OP_CSA_DECODE = 4,
  SA_OP_PREFILL = 5
} sa_op;

/* Attention modes of sparse_attn_prefill. */
typedef enum {
  SA_PREFILL_SPARSE = 0, /* indexer -> Top-K -> MLA over the k selected rows  */
  SA_PREFILL_DENSE = 1,  /* MLA over every causal candidate (MHA + mask)      */
  SA_PREFILL_AUTO = 2    /* DENSE when L <= k, else SPARSE                    */
} sa_prefill_mode;

/* ---------------------------------------------------------------------------
 * Stage 1: lightning indexer scores.
 *   "Sparse Attention 数学学习笔记" §9 (I_{t,s} equation);
 *   "MLA 与稀疏注意力" DSA section (I_{t,s} and TopK_{s<=t}).
 *
 *   q_idx  [B, T, HI, dI]  q_dtype in {SA_F32, SA_BF16}
 *   w      [B, T, HI]      fp32 head weights (any sign)
 *   k_idx  [B, L, dI]      k_dtype in {SA_F32, SA_BF16, SA_FP8_E4M3}
 *   k_scale[B, L]          fp32, required iff k_dtype == SA_FP8_E4M3, else NULL.
 *                          The key of row s is k_scale[s] * fp8value; scales
 *                          must be >= 0 (finite), because the kernel applies
 *                          the scale after the ReLU (ReLU(a x) = a ReLU(x), a >= 0).
 *   q_pos  [B, T]          optional: causal bound, s is a candidate only if
 *                          s <= q_pos[b,t].  NULL: no bound (decode: every
 *                          cached position, including the current token's,
 *                          is a candidate).
 *   kv_len [B]             optional: s is a candidate only if s < kv_len[b]
 *                          (values above L are clamped to L).  NULL: L.
 *   scores [B, T, L]       fp32 output; -inf where s is not a candidate.
 * Compiled set: 1 <= HI <= 128; dI in {64, 128}.  q_dtype SA_BF16 with k_dtype
 * SA_BF16 or SA_FP8_E4M3, HI a multiple of 16, runs on the bf16 MFMA path;
 * every other combination runs the fp32 vector path (exact for small
 * integers).  T <= L is not required.
 * ------------------------------------------------------------------------- */
int sparse_attn_indexer_scores(const void* q_idx, int q_dtype, const float* w,
                               const void* k_idx, int k_dtype,
                               const float* k_scale, const int32_t* q_pos,
                               const int32_t* kv_len, int B, int T, int L,
                               int HI, int dI, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * Stage 2: per-query Top-K over index scores.
 *   "Sparse Attention 数学学习笔记" §9 (S_t = TopK of I_{t,:}, |S| = k per §2);
 *   "MLA 与稀疏注意力" DSA section: TopK over s <= t, and its selected-position
 *   helper that keeps the first k positions ordered by (-score, position).
 *
 *   scores [B, T, L] fp32 (as written by sparse_attn_indexer_scores; any
 *          finite values are accepted, -inf marks a non-candidate).
 *   q_pos, kv_len: the same optional candidate bounds as the indexer.
 *   idx    [B, T, k] int32 output: the selected positions in ASCENDING
 *          order; slots past the count are -1.
 *   count  [B, T] int32 output (may be NULL): min(k, #candidates).
 * Selection: exactly min(k, #candidates) candidates; a candidate with a
 * strictly larger score always beats a smaller one; among equal scores
 * (-0.0 == +0.0) the lower position wins.  NaN scores are never selected
 * (the source pages reject non-finite index scores; the library excludes
 * them instead of failing asynchronously).
 * ws: workspace of sparse_attn_workspace_bytes(SA_OP_TOPK, B, T, L, k, 0, 0)
 * bytes (may be 0 -> ws may be NULL).  Compiled set: 1 <= k <= 4096,
 * L <= 2^31 - 1.
 * ------------------------------------------------------------------------- */
int sparse_attn_topk(const float* scores, const int32_t* q_pos,
                     const int32_t* kv_len, int B, int T, int L, int k,
                     int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Stage 3: sparse MLA over given index sets.
 *   "MLA 与稀疏注意力" full-score section (score = ((U_K^T q^C) . c_j +
 *   q^R . k^R_j) / sqrt(d_C + d_R), one softmax over both terms);
 *   "Sparse Attention 数学学习笔记" §2 (normalise over S only), §8 (sparse MLA
 *   output), §9 (gather only {c_s : s in S_t}).
 *
 *   q_lat  [B, T, H, dc], q_rope [B, T, H, dR]: q_dtype in {SA_F32, SA_BF16}
 *   c_kv   rows of dc elements, row (b, s) at c_kv + (b*L + s) * c_stride
 *   k_rope rows of dR elements, row (b, s) at k_rope + (b*L + s) * r_stride
 *          kv_dtype in {SA_F32, SA_BF16}; must equal q_dtype.
 *   idx    [B, T, k] int32: a slot holding a position outside [0, L) is
 *          skipped (so -1 padding is allowed); duplicates count twice.
 *   sm_scale: the score scale, normally 1/sqrt(d_C + d_R).
 *   out    [B, T, H, dc] fp32 output (latent space).
 *   lse    [B, T, H] fp32 output (may be NULL): natural-log sum of exp(s).
 * A query whose slots are all skipped gets out = 0 and lse = -inf.
 * Compiled set: fp32 path dc <= 512, dR <= 64, H * dc <= 8192; bf16 path
 * (dc, dR) = (512, 64), H a multiple of 64, and one sequence's rows within
 * 4 GiB less 8 KiB (L * row stride * 2 bytes < 2^32 - 8192).  k >= 1.
 * ws: sparse_attn_workspace_bytes(SA_OP_MLA_FORWARD, B, T, L, k, H, dc).
 * ------------------------------------------------------------------------- */
int sparse_attn_mla_forward(const void* q_lat, const void* q_rope, int q_dtype,
                            const void* c_kv, const void* k_rope, int kv_dtype,
                            int64_t c_stride, int64_t r_stride,
                            const int32_t* idx, int k, int B, int T, int L,
                            int H, int dc, int dR, float sm_scale, float* out,
                            float* lse, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Fused decode step (T = 1): stages 1 -> 2 -> 3 enqueued back to back with
 * one workspace ("Sparse Attention 数学学习笔记" §8, decode order
 * h_t -> (q^I, w^I) -> {I_t,j} -> S_t -> {c_j : j in S_t} -> o_t).
 * Arguments as in the three stages with T = 1 and q_pos = NULL.
 *   idx_out [B, k] int32 (may be NULL): the selected set, ascending, -1 padded.
 * The selected set is the one sparse_attn_topk returns for the scores that
 * sparse_attn_indexer_scores computes, with the same tie rule.  When the
 * indexer runs on matrix cores (bf16 queries, H^I in {16, 32, 64, 128}) and
 * L <= 131072, B <= 128, the score kernel also leaves per-work-group
 * candidate lists in the workspace and the selection reads those, checking
 * that they hold every selected position and otherwise reading the scores.
 * ws: sparse_attn_workspace_bytes(SA_OP_DECODE, B, 1, L, k, H, dc): the scores,
 *   the index sets, the candidate lists or the Top-K scratch, and the MLA's
 *   split partials; its contents need no initialisation and are overwritten.
 * ------------------------------------------------------------------------- */
int sparse_attn_decode(const void* q_idx, int q_idx_dtype, const float* w,
                       const void* k_idx, int k_dtype, const float* k_scale,
                       const int32_t* kv_len, int B, int L, int HI, int dI,
                       int k, const void* q_lat, const void* q_rope,
                       int q_dtype, const void* c_kv, const void* k_rope,
                       int kv_dtype, int64_t c_stride, int64_t r_stride, int H,
                       int dc, int dR, float sm_scale, float* out, float* lse,
                       int32_t* idx_out, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The scratch is a fixed 64 MiB array
 * inside the library, one per GPU, held until the process ends; this call
 * allocates nothing and calls no allocating routine.  Arguments, outputs and
 * errors as sparse_attn_decode; sizes whose workspace
 * (sparse_attn_workspace_bytes(SA_OP_DECODE, ...)) exceeds 64 MiB return
 * SA_ERR_WORKSPACE before anything is enqueued.  The scratch is shared by
 * every call on the same GPU: calls that overlap in time on one GPU (other
 * streams or threads) race on it, so callers serialise them.  It needs no
 * clearing: every part of it is written before it is read.
 * ------------------------------------------------------------------------- */
int sparse_attn_decode_noalloc(const void* q_idx, int q_idx_dtype,
                               const float* w, const void* k_idx, int k_dtype,
                               const float* k_scale, const int32_t* kv_len,
                               int B, int L, int HI, int dI, int k,
                               const void* q_lat, const void* q_rope,
                               int q_dtype, const void* c_kv,
                               const void* k_rope, int kv_dtype,
                               int64_t c_stride, int64_t r_stride, int H,
                               int dc, int dR, float sm_scale, float* out,
                               float* lse, int32_t* idx_out, void* stream);

/* ---------------------------------------------------------------------------
 * Fused prefill select: stages 1 and 2 in one kernel, with no [B, T, L] score
 * tensor.  "MLA 与稀疏注意力" DSA section (I_{t,s}, then TopK over s <= t);
 * "Sparse Attention 数学学习笔记" §9.  One work-group per query row computes
 * the row's index scores into on-chip memory (4 bytes per position) and
 * selects from them there; only idx and count are written.  The scores carry
 * the same bits as sparse_attn_indexer_scores' for the same inputs, and the
 * selection follows the rule of sparse_attn_topk, so idx and count equal
 * what those two calls produce.
 *   Arguments as sparse_attn_indexer_scores (q_idx [B,T,HI,dI], w [B,T,HI],
 *   k_idx [B,L,dI], k_scale, q_pos, kv_len) and sparse_attn_topk (k, idx
 *   [B,T,k] ascending and -1 padded, count [B,T] or NULL).
 * Compiled set: q_dtype SA_BF16, k_dtype SA_BF16 or SA_FP8_E4M3, HI in
 * {16, 32, 64, 128}, dI in {64, 128}, 1 <= L <= 32768, k >= 1.  No workspace.
 * ------------------------------------------------------------------------- */
int sparse_attn_prefill_select(const void* q_idx, int q_dtype, const float* w,
                               const void* k_idx, int k_dtype,
                               const float* k_scale, const int32_t* q_pos,
                               const int32_t* kv_len, int B, int T, int L,
                               int HI, int dI, int k, int32_t* idx,
                               int32_t* count, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill: every query of a causal prefill, in one call.
 *   mode SA_PREFILL_SPARSE: the selected sets, then stage 3 over the
 *     selected rows ("Sparse Attention 数学学习笔记" §8-§9).  The sets come
 *     from sparse_attn_prefill_select, or from stages 1 and 2 run per
 *     sequence in chunks of query rows through a [chunk, L] score buffer in
 *     the workspace (the same sets) where that is faster on MI355X: T >= 2048
 *     with L >= 2048, or T >= 1024 with L > 16384 (k in the top-k set), and
 *     every L above the fused select's 32768.  A chunk holds as many query
 *     rows as 1 GiB of scores does, at least 4096 (at most T).
 *   mode SA_PREFILL_DENSE: stage 3 over every candidate position s <
 *     min(q_pos[b,t] + 1, kv_len[b], L), with no indexer and no Top-K: the
 *     dense attention with a causal mask that "LLM注意力优化：稀疏注意力" (DSA
 *     section) names as the better choice for short sequences.  The result is
 *     the sparse one whenever no row has more than k candidates.
 *   mode SA_PREFILL_AUTO: DENSE when L <= k, else SPARSE.  With L <= k no row
 *     has more than k candidates, so both modes attend to the same rows and
 *     the dense one skips the indexer and the Top-K; above k the sparse mode
 *     is the faster one on MI355X already from L = 1.5 k (k = 2048, H = 128:
 *     1.27x at L = 3072, 1.64x at 4096, 5.6x at 16384), so the switch never
 *     changes a result.
 * Arguments as sparse_attn_prefill_select (the indexer inputs may be NULL in
 * the dense mode) and sparse_attn_mla_forward (q_lat [B,T,H,dc], q_rope
 * [B,T,H,dR], strided c_kv / k_rope rows).  idx_out [B,T,k] (may be NULL;
 * sparse mode only) receives the selected sets.
 * Compiled set: the prefill select's (any L in the sparse mode: rows above
 * 32768 take the staged path, whose top-k set is 1 <= k <= 4096), and the bf16
 * MLA path ((dc, dR) = (512, 64), H a multiple of 64).
 * ws: sparse_attn_workspace_bytes(SA_OP_PREFILL, B, T, L, k, H, dc), which
 * covers every mode.
 * ------------------------------------------------------------------------- */
int sparse_attn_prefill(const void* q_idx, int q_idx_dtype, const float* w,
                        const void* k_idx, int k_dtype, const float* k_scale,
                        const int32_t* q_pos, const int32_t* kv_len, int B,
                        int T, int L, int HI, int dI, int k, const void* q_lat,
                        const void* q_rope, const void* c_kv,
                        const void* k_rope, int64_t c_stride, int64_t r_stride,
                        int H, int dc, int dR, float sm_scale, int mode,
                        float* out, float* lse, int32_t* idx_out, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Selection over compressed entries (CSA-style decode step, T = 1).
 *   "LLM注意力优化：稀疏注意力" DeepSeek CSA & HCA section: each m tokens of
 *   KV cache are compressed into one entry (the compression is learned and is
 *   the caller's); the indexer scores the query against the entries' index
 *   keys, the top-k entries are kept, and core attention is MQA with the
 *   selected entries as both keys and values; the most recent raw entries of a
 *   sliding window are attended as well.  Reading: the window branch joins the
 *   selected entries in one softmax (equal to merging the two branches'
 *   outputs by log-sum-exp), a query head's output is
 *     o_h = sum_{j in S U W} softmax_j(q_h . e_j * sm_scale) e_j.
 *   Stages: indexer over the Lc entries' index keys (as sparse_attn_decode,
 *   with n_comp[b] present entries, NULL = Lc), top-k, then the attention.
 *   q [B, H, c] bf16; comp [B, Lc, c] bf16 entries; win [B, n_win, c] bf16
 *   raw entries (may be NULL when n_win = 0); out [B, H, c] fp32; lse [B, H]
 *   (may be NULL); idx_out [B, k] (may be NULL): the selected entries,
 *   ascending, -1 padded.
 * Compiled set: c = 512, H a multiple of 64; indexer and top-k as above.
 * ws: sparse_attn_workspace_bytes(SA_OP_CSA_DECODE, B, n_win, Lc, k, H, c).
 * ------------------------------------------------------------------------- */
int sparse_attn_csa_decode(const void* q_idx, int q_idx_dtype, const float* w,
                           const void* k_idx, int k_dtype, const float* k_scale,
                           const int32_t* n_comp, int B, int Lc, int HI, int dI,
                           int k, const void* q, const void* comp,
                           const void* win, int n_win, int H, int c,
                           float sm_scale, float* out, float* lse,
                           int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Block-sparse variant: GQA decode over whole blocks.
 *   "第 11 章 稀疏注意力" §12.5 (select and read whole contiguous blocks),
 *   §12.6 (block representative = mean of the block's keys, top-k over block
 *   scores); "LLM注意力优化：稀疏注意力" MoBA section (affinity of a query to a
 *   block = inner product with the mean-pooled block key; window and sink are
 *   fixed blocks); "Sparse Attention 数学学习笔记" §4 (sliding window).
 *
 * sparse_attn_block_pool: krep[b, n, g, :] = mean over the blk tokens of block
 * n of k[b, :, g, :], for the complete blocks n < L / blk.
 *   k [B, L, Hkv, d] bf16; krep [B, L/blk, Hkv, d] bf16 output, the fp32 mean
 *   rounded to nearest even (may be NULL when L < blk: there is no complete
 *   block).
 *
 * sparse_attn_block_decode: per query head h (KV head g = h / (Hq / Hkv)):
 *   block score n = q[b,h,:] . krep[b,n,g,:]; the nsel highest (ties to the
 *   lower block index); visible set = those blocks' tokens, union the first
 *   n_sink tokens, union the last n_win tokens; one softmax with sm_scale over
 *   the union (each token once); out[b,h,:] = sum softmax * v[b,j,g,:].
 *   shared_choice = 1: the query heads of a KV group share one block choice,
 *   ranked by the sum of the group's block scores, ties to the lower block
 *   ("MLA 与稀疏注意力" section on choosing blocks and merging outputs, and its
 *   worked example); 0: each query head chooses by its own scores.
 *   q [B, Hq, d] bf16; k, v [B, L, Hkv, d] bf16; krep from block_pool (may
 *   be NULL when L < blk: then only sinks and window are visible).
 *   out [B, Hq, d] fp32; blocks_out [B, Hq, nsel] int32 (may be NULL): the
 *   selected block indices in ascending order (-1 when fewer blocks exist).
 * Compiled set: d = 128, blk in {32, 64, 128}, Hq / Hkv in {1, 2, 4, 8},
 * 1 <= nsel <= 64, L / blk <= 8192.
 * ws: sparse_attn_workspace_bytes(SA_OP_BLOCK_DECODE, B, Hq, L, nsel, Hkv, d)
 *   (the block scores, [B, Hq, L / blk] fp32, sized for blk = 32; may be
 *   NULL when that is 0 bytes).
 * Errors as for the other entry points; a query head whose visible set is
 * empty (L < blk, no sinks, no window) gets out = 0.
 * ------------------------------------------------------------------------- */
int sparse_attn_block_pool(const void* k, int B, int L, int Hkv, int d,
                           int blk, void* krep, void* stream);

int sparse_attn_block_decode(const void* q, const void* k, const void* v,
                             const void* krep, int B, int L, int Hq, int Hkv,
                             int d, int blk, int nsel, int n_sink, int n_win,
                             float sm_scale, int shared_choice, float* out,
                             int32_t* blocks_out, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Helpers.
 * sparse_attn_workspace_bytes: scratch bytes an entry point needs for the
 *   given sizes (0 when none).  Unused arguments may be 0.  Returns 0 for an
 *   unknown op.
 * sparse_attn_status_string: static name of a status code.
 * sparse_attn_last_error: description of the last failure on the calling
 *   thread (thread-local; empty string when none).
 * ------------------------------------------------------------------------- */
size_t sparse_attn_workspace_bytes(int op, int B, int T, int L, int k, int H,
                                   int dc);
const char* sparse_attn_status_string(int status);
const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
