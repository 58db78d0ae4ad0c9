/*
 * sa_oracle.h -- plain CPU oracle for top-k sparse attention (DSA-style
 * lightning indexer, per-query Top-K, sparse MLA over the latent cache).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Everything is computed in IEEE double.  Inputs arrive already decoded to
 * double (see the two decoders below, written from the bf16 bit layout and the
 * OCP 8-bit floating point E4M3 definition).  OpenMP parallelises the outer
 * (batch, query) loop only; every inner loop is the textbook sum.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Sparse Attention 数学学习笔记" (echobase-5bl.pages.dev, 2026.09.14):
 *       §1 dense attention, §2 renormalising over the visible set, §3 the mask
 *       form, §6 the error bound, §8 sparse MLA, §9 DSA indexer and Top-K.
 *  [P4] "第 11 章 稀疏注意力" (book.shippingwang.com): §12.5 block sparsity,
 *       §12.6 block representatives (mean of the block's keys) and block top-k.
 *  [P5] "MLA 与稀疏注意力：少存一点，还是少看一点？" (tianyi-zhang-02.github.io):
 *       the absorbed score, the full score with a decoupled RoPE key, the
 *       masking example, the DSA section with causal Top-K, the selected-position
 *       helper that orders by (-score, position).
 *  [P2] "LLM注意力优化：稀疏注意力" (wln20.github.io): MoBA block gating by the
 *       mean-pooled block key; sliding window and sink as fixed blocks.
 *
 * Error codes: 0 ok; negative values below.  On error the outputs of the
 * offending row may be partially written.
 */
#ifndef SA_ORACLE_H
#define SA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,       /* bad size or NULL pointer                      */
  ORC_ERR_NONFINITE = -2, /* a candidate's index score is NaN or infinite  */
  ORC_ERR_EMPTY = -3,     /* a softmax over an empty visible set           */
  ORC_ERR_NOMEM = -4
};

/* Number of OpenMP threads the oracle uses. */
int orc_num_threads(void);

/* Decoders.  bf16: the upper half of a binary32 bit pattern.
 * e4m3fn (OCP FP8 E4M3): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is
 * no infinity; the largest finite magnitude is 448. */
void orc_decode_bf16(const uint16_t* in, double* out, int64_t n);
void orc_decode_e4m3fn(const uint8_t* in, double* out, int64_t n);

/* Lightning indexer [P1 §9; P5 DSA section]:
 *   I[b,t,s] = sum_h w[b,t,h] * max(0, sum_i q[b,t,h,i] * k[b,s,i])
 * for candidate s, -inf otherwise.  Candidates: s < kv_len[b] (all L when
 * kv_len is NULL) and s <= q_pos[b,t] (no bound when q_pos is NULL; this is the
 * causal TopK_{s<=t} of [P5]).
 * Shapes: q[B,T,HI,dI], w[B,T,HI], k[B,L,dI], scores[B,T,L]. */
int orc_indexer(const double* q, const double* w, const double* k,
                const int32_t* q_pos, const int32_t* kv_len, int B, int T,
                int L, int HI, int dI, double* scores);

/* Top-K [P1 §9; P5 DSA section, selected-position helper]:
 * the min(k, #candidates) candidates with the largest score, equal scores
 * ordered by the lower position.  Candidates as in orc_indexer.  A candidate
 * whose score is not finite is an error (ORC_ERR_NONFINITE).  The selected
 * positions are written in ascending order into idx[B,T,k]; unused slots are
 * -1; count[B,T] (may be NULL) receives the number selected. */
int orc_topk(const double* scores, const int32_t* q_pos, const int32_t* kv_len,
             int B, int T, int L, int k, int32_t* idx, int32_t* count);

/* Sparse MLA over a gathered set [P5 full-score section; P1 §2, §8]:
 *   s_j = (sum_c q_lat[c] * c_kv[j,c] + sum_r q_rope[r] * k_rope[j,r]) * sm_scale
 *   o   = sum_j softmax(s)_j * c_kv[j, 0:dc]      (latent-space output)
 *   lse = log sum_j exp(s_j)
 * over the slots j of idx[b,t,:] holding a position in [0, L).  Rows of the
 * caches are c_kv + (b*L + s) * c_stride and k_rope + (b*L + s) * r_stride.
 * An empty set is ORC_ERR_EMPTY (the pages' helper rejects a query with no
 * visible position).  out[B,T,H,dc], lse[B,T,H] (lse may be NULL). */
int orc_sparse_mla(const double* q_lat, const double* q_rope,
                   const double* c_kv, const double* k_rope, int64_t c_stride,
                   int64_t r_stride, const int32_t* idx, int k, int B, int T,
                   int L, int H, int dc, int dR, double sm_scale, double* out,
                   double* lse);

/* The mask form [P1 §3]: softmax(s + M) over all L positions with M = 0 where
 * visible[b,t,s] != 0 and -inf elsewhere, value = c_kv[s, 0:dc].  With every
 * position visible this is dense attention [P1 §1]. */
int orc_masked_mla(const double* q_lat, const double* q_rope,
                   const double* c_kv, const double* k_rope, int64_t c_stride,
                   int64_t r_stride, const uint8_t* visible, int B, int T,
                   int L, int H, int dc, int dR, double sm_scale, double* out,
                   double* lse);

/* Block-sparse decode with GQA [P4 §12.5-12.6; P2 MoBA; P1 §4 window].
 *   k, v: [B, L, Hkv, d]; q: [B, Hq, d]; query head h reads KV head h / (Hq/Hkv).
 *   Block representatives: krep[b, n, g, :] = mean of k[b, n*blk .. n*blk+blk-1, g, :]
 *   over the complete blocks n < L / blk (orc_block_pool).
 *   Per query head: block score = q_h . krep[n, g(h)]; the nsel highest, ties to
 *   the lower block index.  Visible set = selected blocks' tokens, union sinks
 *   [0, n_sink), union window [L - n_win, L); one softmax with scale sm_scale
 *   over the union; output o[b, h, :] = sum softmax * v.
 *   blocks_out[B, Hq, nsel] (may be NULL) receives the selected block indices
 *   in ascending order.
 *   shared != 0: the block choice is shared by the query heads of a KV group,
 *   by the sum of their block scores, ties to the lower block index
 *   ["MLA 与稀疏注意力" section on block choice and merging, worked example].
 *   given_blocks[B, Hq, nsel] (may be NULL): when given, no block is chosen;
 *   the visible set is built from these block indices instead (entries
 *   outside [0, L / blk) are ignored, a block listed twice counts once), so a
 *   caller can evaluate the attention of a choice made elsewhere.  With the
 *   oracle's own choice passed in, the output is the same as without.
 *   Returns ORC_ERR_EMPTY (out = 0) when some head's visible set is empty. */
int orc_block_pool(const double* k, int B, int L, int Hkv, int d, int blk,
                   double* krep);
int orc_block_sparse_decode(const double* q, const double* k, const double* v,
                            const double* krep, int B, int L, int Hq, int Hkv,
                            int d, int blk, int nsel, int n_sink, int n_win,
                            double sm_scale, int shared,
                            const int32_t* given_blocks, double* out,
                            int32_t* blocks_out);

#ifdef __cplusplus
}
#endif
#endif /* SA_ORACLE_H */
