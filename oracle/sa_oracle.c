/*
 * sa_oracle.c -- plain CPU oracle (double precision).  TEST INFRASTRUCTURE:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it;
 * nothing here is shared with the GPU library.
 *
 * Every function writes the definition out as loops, in the order the pages
 * state it; see sa_oracle.h for the sources.  Nothing is blocked, fused or
 * reordered.
 */
#include "sa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Decoders                                                                 */
/* ------------------------------------------------------------------------ */

/* bf16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of an
 * IEEE binary32; its value is that of the binary32 with the low half zero. */
void orc_decode_bf16(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t bits = (uint32_t)in[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    out[i] = (double)f;
  }
}

/* OCP 8-bit floating point, E4M3 ("fn": finite, NaN only): value of a code
 * S.EEEE.MMM is (-1)^S * 2^(E-7) * (1 + M/8) for E >= 1, (-1)^S * 2^-6 * M/8
 * for E = 0, and NaN for E = 15, M = 7. */
void orc_decode_e4m3fn(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    int s = (in[i] >> 7) & 1;
    int e = (in[i] >> 3) & 15;
    int m = in[i] & 7;
    double mag;
    if (e == 15 && m == 7) {
      out[i] = NAN;
      continue;
    }
    if (e == 0)
      mag = ldexp((double)m / 8.0, -6);
    else
      mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    out[i] = s ? -mag : mag;
  }
}

/* ------------------------------------------------------------------------ */
/* Candidate rule shared by indexer and top-k                               */
/* ------------------------------------------------------------------------ */

static int is_candidate(const int32_t* q_pos, const int32_t* kv_len, int b,
                        int t, int T, int L, int s) {
  int limit = kv_len ? kv_len[b] : L;
  if (limit > L) limit = L;
  if (s >= limit) return 0;
  if (q_pos && s > q_pos[(int64_t)b * T + t]) return 0;
  return 1;
}

/* ------------------------------------------------------------------------ */
/* Lightning indexer  [P1 §9, P5 DSA section]                               */
/* ------------------------------------------------------------------------ */

int orc_indexer(const double* q, const double* w, const double* k,
                const int32_t* q_pos, const int32_t* kv_len, int B, int T,
                int L, int HI, int dI, double* scores) {
  if (!q || !w || !k || !scores || B < 0 || T < 0 || L < 0 || HI < 1 || dI < 1)
    return ORC_ERR_ARG;
  int64_t rows = (int64_t)B * T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < rows; ++bt) {
    int b = (int)(bt / T), t = (int)(bt % T);
    const double* qb = q + bt * HI * dI;
    const double* wb = w + bt * HI;
    double* out = scores + bt * L;
    for (int s = 0; s < L; ++s) {
      if (!is_candidate(q_pos, kv_len, b, t, T, L, s)) {
        out[s] = -INFINITY;
        continue;
      }
      const double* ks = k + ((int64_t)b * L + s) * dI;
      double I = 0.0;
      for (int h = 0; h < HI; ++h) {
        double dot = 0.0;
        for (int i = 0; i < dI; ++i) dot += qb[(int64_t)h * dI + i] * ks[i];
        double relu = dot > 0.0 ? dot : 0.0;
        I += wb[h] * relu;
      }
      out[s] = I;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-K  [P1 §9; P5 DSA section: sort by (-score, position), keep count]   */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int32_t pos;
} cand_t;

/* Descending score; equal scores (including -0 == +0) by ascending position. */
static int by_neg_score_then_pos(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int by_pos(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int orc_topk(const double* scores, const int32_t* q_pos, const int32_t* kv_len,
             int B, int T, int L, int k, int32_t* idx, int32_t* count) {
  if (!scores || !idx || B < 0 || T < 0 || L < 0 || k < 1) return ORC_ERR_ARG;
  int64_t rows = (int64_t)B * T;
  int status = ORC_OK;
#pragma omp parallel
  {
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(L > 0 ? L : 1));
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    if (!c || !sel) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t bt = 0; bt < rows; ++bt) {
      if (!c || !sel) continue;
      int b = (int)(bt / T), t = (int)(bt % T);
      const double* row = scores + bt * L;
      int n = 0;
      for (int s = 0; s < L; ++s) {
        if (!is_candidate(q_pos, kv_len, b, t, T, L, s)) continue;
        if (!isfinite(row[s])) {
#pragma omp atomic write
          status = ORC_ERR_NONFINITE;
        }
        c[n].score = row[s];
        c[n].pos = s;
        ++n;
      }
      qsort(c, (size_t)n, sizeof(cand_t), by_neg_score_then_pos);
      int m = n < k ? n : k;
      for (int i = 0; i < m; ++i) sel[i] = c[i].pos;
      qsort(sel, (size_t)m, sizeof(int32_t), by_pos);
      int32_t* out = idx + bt * k;
      for (int i = 0; i < k; ++i) out[i] = i < m ? sel[i] : -1;
      if (count) count[bt] = m;
    }
    free(c);
    free(sel);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Sparse MLA over the gathered set  [P5 full score; P1 §2, §8]             */
/* ------------------------------------------------------------------------ */

/* score of one cached row for one head: content term through the absorbed
 * query plus the RoPE term, one sum, one scale. */
static double mla_score(const double* ql, const double* qr, const double* cj,
                        const double* kr, int dc, int dR, double sm_scale) {
  double content = 0.0, rope = 0.0;
  for (int c = 0; c < dc; ++c) content += ql[c] * cj[c];
  for (int r = 0; r < dR; ++r) rope += qr[r] * kr[r];
  return (content + rope) * sm_scale;
}

int orc_sparse_mla(const double* q_lat, const double* q_rope,
                   const double* c_kv, const double* k_rope, int64_t c_stride,
                   int64_t r_stride, const int32_t* idx, int k, int B, int T,
                   int L, int H, int dc, int dR, double sm_scale, double* out,
                   double* lse) {
  if (!q_lat || !c_kv || !idx || !out || k < 1 || B < 0 || T < 0 || L < 0 ||
      H < 1 || dc < 1 || dR < 0 || (dR > 0 && (!q_rope || !k_rope)))
    return ORC_ERR_ARG;
  int64_t units = (int64_t)B * T * H;
  int status = ORC_OK;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)k);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    if (!s || !pos) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 8)
    for (int64_t u = 0; u < units; ++u) {
      if (!s || !pos) continue;
      int64_t bt = u / H;
      int b = (int)(bt / T);
      const double* ql = q_lat + u * dc;
      const double* qr = dR > 0 ? q_rope + u * dR : NULL;
      const int32_t* row = idx + bt * k;
      int n = 0;
      for (int j = 0; j < k; ++j)
        if (row[j] >= 0 && row[j] < L) pos[n++] = row[j];
      double* o = out + u * dc;
      if (n == 0) {
        for (int c = 0; c < dc; ++c) o[c] = 0.0;
        if (lse) lse[u] = -INFINITY;
#pragma omp atomic write
        status = ORC_ERR_EMPTY;
        continue;
      }
      double m = -INFINITY;
      for (int j = 0; j < n; ++j) {
        int64_t r = (int64_t)b * L + pos[j];
        s[j] = mla_score(ql, qr, c_kv + r * c_stride,
                         dR > 0 ? k_rope + r * r_stride : NULL, dc, dR,
                         sm_scale);
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
      }
      for (int c = 0; c < dc; ++c) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
          acc += s[j] * c_kv[((int64_t)b * L + pos[j]) * c_stride + c];
        o[c] = acc / l;
      }
      if (lse) lse[u] = m + log(l);
    }
    free(s);
    free(pos);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Mask form / dense  [P1 §3, §1]                                           */
/* ------------------------------------------------------------------------ */

int orc_masked_mla(const double* q_lat, const double* q_rope,
                   const double* c_kv, const double* k_rope, int64_t c_stride,
                   int64_t r_stride, const uint8_t* visible, int B, int T,
                   int L, int H, int dc, int dR, double sm_scale, double* out,
                   double* lse) {
  if (!q_lat || !c_kv || !visible || !out || B < 0 || T < 0 || L < 1 ||
      H < 1 || dc < 1 || dR < 0 || (dR > 0 && (!q_rope || !k_rope)))
    return ORC_ERR_ARG;
  int64_t units = (int64_t)B * T * H;
  int status = ORC_OK;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 8)
    for (int64_t u = 0; u < units; ++u) {
      if (!z) continue;
      int64_t bt = u / H;
      int b = (int)(bt / T);
      const double* ql = q_lat + u * dc;
      const double* qr = dR > 0 ? q_rope + u * dR : NULL;
      const uint8_t* vis = visible + bt * L;
      double* o = out + u * dc;
      /* z = s + M over every position */
      double m = -INFINITY;
      for (int j = 0; j < L; ++j) {
        int64_t r = (int64_t)b * L + j;
        double sj = mla_score(ql, qr, c_kv + r * c_stride,
                              dR > 0 ? k_rope + r * r_stride : NULL, dc, dR,
                              sm_scale);
        double Mj = vis[j] ? 0.0 : -INFINITY;
        z[j] = sj + Mj;
        if (z[j] > m) m = z[j];
      }
      if (m == -INFINITY) {
        for (int c = 0; c < dc; ++c) o[c] = 0.0;
        if (lse) lse[u] = -INFINITY;
#pragma omp atomic write
        status = ORC_ERR_EMPTY;
        continue;
      }
      double l = 0.0;
      for (int j = 0; j < L; ++j) {
        z[j] = exp(z[j] - m); /* exp(-inf) = 0 for masked positions */
        l += z[j];
      }
      for (int c = 0; c < dc; ++c) {
        double acc = 0.0;
        for (int j = 0; j < L; ++j)
          acc += z[j] * c_kv[((int64_t)b * L + j) * c_stride + c];
        o[c] = acc / l;
      }
      if (lse) lse[u] = m + log(l);
    }
    free(z);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Block-sparse decode with GQA  [P4 §12.5-12.6; P2 MoBA; P1 §4]            */
/* ------------------------------------------------------------------------ */

int orc_block_pool(const double* k, int B, int L, int Hkv, int d, int blk,
                   double* krep) {
  if (!k || !krep || B < 0 || L < 0 || Hkv < 1 || d < 1 || blk < 1)
    return ORC_ERR_ARG;
  int nblk = L / blk;
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < nblk; ++n)
      for (int g = 0; g < Hkv; ++g)
        for (int i = 0; i < d; ++i) {
          double acc = 0.0;
          for (int j = 0; j < blk; ++j)
            acc += k[(((int64_t)b * L + (int64_t)n * blk + j) * Hkv + g) * d + i];
          krep[(((int64_t)b * nblk + n) * Hkv + g) * d + i] = acc / blk;
        }
  return ORC_OK;
}

int orc_block_sparse_decode(const double* q, const double* k, const double* v,
                            const double* krep, int B, int L, int Hq, int Hkv,
                            int d, int blk, int nsel, int n_sink, int n_win,
                            double sm_scale, int shared,
                            const int32_t* given_blocks, double* out,
                            int32_t* blocks_out) {
  if (!q || !k || !v || !krep || !out || B < 0 || L < 1 || Hq < 1 ||
      Hkv < 1 || Hq % Hkv || d < 1 || blk < 1 || nsel < 0 || n_sink < 0 ||
      n_win < 0)
    return ORC_ERR_ARG;
  int nblk = L / blk;
  int group = Hq / Hkv;
  int64_t units = (int64_t)B * Hq;
  int status = ORC_OK;
#pragma omp parallel
  {
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nblk > 0 ? nblk : 1));
    uint8_t* vis = (uint8_t*)malloc((size_t)L);
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nsel > 0 ? nsel : 1));
    if (!c || !vis || !z || !sel) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      if (!c || !vis || !z || !sel) continue;
      int b = (int)(u / Hq), h = (int)(u % Hq), g = h / group;
      const double* qh = q + u * d;
      /* block scores against the mean-pooled block keys: the head's own, or
         with `shared` the sum over the heads of its KV group; a given choice
         replaces the scoring and the ranking */
      int h0 = shared ? g * group : h, h1 = shared ? h0 + group : h + 1;
      for (int n = 0; n < nblk && !given_blocks; ++n) {
        const double* kr = krep + (((int64_t)b * nblk + n) * Hkv + g) * d;
        double total = 0.0;
        for (int hh = h0; hh < h1; ++hh) {
          const double* qs = q + ((int64_t)b * Hq + hh) * d;
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += qs[i] * kr[i];
          total += dot;
        }
        c[n].score = total;
        c[n].pos = n;
      }
      int m = 0;
      if (given_blocks) {
        for (int i = 0; i < nsel; ++i) {
          int32_t x = given_blocks[u * nsel + i];
          if (x >= 0 && x < nblk) sel[m++] = x;
        }
      } else {
        qsort(c, (size_t)nblk, sizeof(cand_t), by_neg_score_then_pos);
        m = nblk < nsel ? nblk : nsel;
        for (int i = 0; i < m; ++i) sel[i] = c[i].pos;
      }
      qsort(sel, (size_t)m, sizeof(int32_t), by_pos);
      if (blocks_out)
        for (int i = 0; i < nsel; ++i)
          blocks_out[u * nsel + i] = i < m ? sel[i] : -1;
      /* visible set: selected blocks, sinks and window, each position once */
      memset(vis, 0, (size_t)L);
      for (int i = 0; i < m; ++i)
        for (int j = 0; j < blk; ++j) vis[(int64_t)sel[i] * blk + j] = 1;
      for (int j = 0; j < n_sink && j < L; ++j) vis[j] = 1;
      for (int j = L - n_win; j < L; ++j)
        if (j >= 0) vis[j] = 1;
      /* one softmax over the union */
      double mx = -INFINITY;
      for (int j = 0; j < L; ++j) {
        if (!vis[j]) continue;
        const double* kj = k + (((int64_t)b * L + j) * Hkv + g) * d;
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += qh[i] * kj[i];
        z[j] = dot * sm_scale;
        if (z[j] > mx) mx = z[j];
      }
      double* o = out + u * d;
      if (mx == -INFINITY) {
        for (int i = 0; i < d; ++i) o[i] = 0.0;
#pragma omp atomic write
        status = ORC_ERR_EMPTY;
        continue;
      }
      double l = 0.0;
      for (int j = 0; j < L; ++j) {
        if (!vis[j]) continue;
        z[j] = exp(z[j] - mx);
        l += z[j];
      }
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < L; ++j)
          if (vis[j]) acc += z[j] * v[(((int64_t)b * L + j) * Hkv + g) * d + i];
        o[i] = acc / l;
      }
    }
    free(c);
    free(vis);
    free(z);
    free(sel);
  }
  return status;
}
