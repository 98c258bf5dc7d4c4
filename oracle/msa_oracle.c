/*
 * msa_oracle.c -- plain, slow CPU oracle for MiniMax Sparse Attention (MSA):
 * the index branch (block max-pool of a single-head index key, q.blockmax
 * scores, per-query causal top-K) and the sparse branch (standard GQA over
 * the union of the selected KV blocks).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the HIP library, and neither includes
 * the other.
 *
 * Everything is the plain definition written out: the max-pool is exact in
 * fp32 (a max rounds nothing); scores and attention are fp64 over exactly
 * upcast inputs; the softmax is the textbook two-pass form over the full key
 * set of a query -- no tiling, no online softmax, no log-sum-exp merge.
 *
 * Pages cited (title, address):
 *   [YLY] "MiniMax M3模型算力成本大幅降低原因深度解析",
 *         youleyou.com/wenzhang/3016623.html
 *   [CXT] "MiniMax M3 深度实战：当稀疏注意力打破百万 Token 墙 ...",
 *         chenxutan.com/d/3746.html
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - the block summary is an elementwise max over the block's valid tokens
 *     only (no zero padding of a partial last block);
 *   - the max uses the total order -0 < +0 so that the result is unique;
 *   - scores are a plain dot product (one index head, no scale, no
 *     activation), one selection per query token shared by all heads;
 *   - candidates are the blocks strictly before the query's own block; the own
 *     block is always kept and counts toward K; ties go to the lower index;
 *   - the selection is stored ascending and padded with -1;
 *   - query head h reads KV head h / (Hq/Hkv); keys t <= p inside the own
 *     block are visible (the query sees itself).
 *
 * Parallelism: OpenMP over queries (independent work, no reduction across
 * threads, so results do not depend on the thread count).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1

/* n consecutive elements starting at index i, upcast exactly to double
 * (bf16 -> fp32 is exact: the 16 bits are the top half of the fp32 pattern). */
static void elems(const void *p, int dtype, int64_t i, int32_t n, double *dst) {
  if (dtype == 0) {
    const float *f = (const float *)p + i;
    for (int32_t c = 0; c < n; ++c) dst[c] = (double)f[c];
  } else {
    const uint16_t *h = (const uint16_t *)p + i;
    for (int32_t c = 0; c < n; ++c) {
      uint32_t u = (uint32_t)h[c] << 16;
      float f;
      memcpy(&f, &u, sizeof f);
      dst[c] = (double)f;
    }
  }
}

/* Strict "a is larger than b" in the total order used for the max-pool:
 * the IEEE order, with -0 placed below +0. */
static int f32_above(float a, float b) {
  if (a > b) return 1;
  if (a == b && a == 0.0f && !signbit(a) && signbit(b)) return 1;
  return 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Index branch, step 1: block max-pool.  [YLY, "索引分支（Index Branch）"]
 * kmax[b][c] = max over t in [b*B, min(b*B+B, len)) of idx_k[t][c].
 * idx_k: [len][d_idx] fp32, kmax: [ceil(len/B)][d_idx] fp32.
 * ---------------------------------------------------------------------- */
int oracle_pool(const float *idx_k, int64_t len, int32_t d_idx, int32_t block,
                float *kmax) {
  if (!idx_k || !kmax || len < 1 || d_idx < 1 || block < 1) return ORC_EINVAL;
  int64_t nb = (len + block - 1) / block;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t t0 = b * block, t1 = t0 + block < len ? t0 + block : len;
    for (int32_t c = 0; c < d_idx; ++c) {
      float m = idx_k[t0 * d_idx + c];
      for (int64_t t = t0 + 1; t < t1; ++t) {
        float x = idx_k[t * d_idx + c];
        if (f32_above(x, m)) m = x;
      }
      kmax[b * d_idx + c] = m;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Block mean-pool of index keys: the block summary of [CXT §3.3]'s sketch
 * (the mean of the block's keys), an alternative to the max-pool above.
 * kmean[b][c] = (sum over the valid tokens t of block b of idx_k[t][c]) / n_b,
 * summed in fp64 and rounded to fp32 once.
 * ---------------------------------------------------------------------- */
int oracle_pool_mean(const float *idx_k, int64_t len, int32_t d_idx, int32_t block,
                     float *kmean) {
  if (!idx_k || !kmean || len < 1 || d_idx < 1 || block < 1) return ORC_EINVAL;
  int64_t nb = (len + block - 1) / block;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t t0 = b * block, t1 = t0 + block < len ? t0 + block : len;
    for (int32_t c = 0; c < d_idx; ++c) {
      double acc = 0.0;
      for (int64_t t = t0; t < t1; ++t) acc += (double)idx_k[t * d_idx + c];
      kmean[b * d_idx + c] = (float)(acc / (double)(t1 - t0));
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Index branch, steps 2-3: scores and causal top-K.
 * [YLY, "索引分支（Index Branch）"] single-head key, block max-pool, keep the
 * Top-K blocks; [CXT §3.3 "Prefilling 与 Decoding 的差异化优化"] prefill scores
 * every block for every query, decode scores the one new query.
 *
 * For query i at position pos = q_pos[i], own = pos / B:
 *   score[b] = sum_c idx_q[i][c] * kmax[b][c] (fp64), for b < own;
 *   rank the candidates by (score descending, b ascending), keep the first
 *   min(K-1, own), add own, store ascending, pad with -1.
 * Near-tie report (only when some candidate is left out and K >= 2):
 *   gap_abs  = s_(K-1) - s_(K)   (last kept minus first left out),
 *   gap_rel  = gap_abs / max(|s_(K-1)|, |s_(K)|),
 *   err_bnd  = gamma_d * (sum_c |q_c kmax_(K-1),c| + sum_c |q_c kmax_(K),c|),
 *              gamma_d = d*u/(1-d*u), u = 2^-24: the worst-case fp32 error of
 *              the two dot products in any summation order.
 *   All three are NaN when there is no cut.
 * kmax: [nb_avail][d_idx]; own must be < nb_avail.
 *
 * Local-window variant (oracle_select_window, after the sliding window that
 * [CXT §3.3]'s sketch always keeps): the blocks max(0, own-window+1) .. own
 * are forced, the candidates are the blocks below them, and the first
 * min(K-window, #candidates) by the same ranking are kept; the near-tie
 * report then concerns ranks K-window and K-window+1.  window = 1 is the
 * rule above.
 * ---------------------------------------------------------------------- */
typedef struct {
  double s;
  int32_t b;
} cand_t;

static int cand_cmp(const void *x, const void *y) {
  const cand_t *a = (const cand_t *)x, *b = (const cand_t *)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->b > b->b) - (a->b < b->b);
}

static int int_cmp(const void *x, const void *y) {
  int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
  return (a > b) - (a < b);
}

int oracle_select_window(const float *idx_q, int64_t n_q, const int64_t *q_pos,
                         const float *kmax, int64_t nb_avail, int32_t d_idx,
                         int32_t block, int32_t topk, int32_t window, int32_t *sel,
                         double *gap_rel, double *gap_abs, double *err_bnd) {
  if (!idx_q || !q_pos || !kmax || !sel || n_q < 0 || d_idx < 1 || block < 1 ||
      topk < 1 || window < 1 || window > topk)
    return ORC_EINVAL;
  for (int64_t i = 0; i < n_q; ++i)
    if (q_pos[i] < 0 || q_pos[i] / block >= nb_avail) return ORC_EINVAL;
  const double u = ldexp(1.0, -24);
  const double gamma = d_idx * u / (1.0 - d_idx * u);
  /* kmax transposed and upcast once, kt[c][b]: the scores below are then
   * accumulated over c in ascending order for every block, exactly as the
   * plain loop "for b: for c: s += q[c] * kmax[b][c]" would (the same
   * products and the same order of sums), with the loop over blocks inside */
  double *kt = (double *)malloc(sizeof(double) * (size_t)nb_avail * (size_t)d_idx);
  if (!kt) return ORC_EINVAL;
  for (int64_t b = 0; b < nb_avail; ++b)
    for (int32_t cc = 0; cc < d_idx; ++cc)
      kt[(int64_t)cc * nb_avail + b] = (double)kmax[b * d_idx + cc];
  int bad = 0;
#pragma omp parallel
  {
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb_avail + 1));
    double *sc = (double *)malloc(sizeof(double) * (size_t)(nb_avail + 1));
    int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)(topk + 1));
    if (!c || !sc || !keep) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_q; ++i) {
      if (!c || !sc || !keep) continue;
      const float *q = idx_q + i * d_idx;
      int64_t own = q_pos[i] / block;
      int64_t first = own - window + 1 > 0 ? own - window + 1 : 0;  /* forced: first..own */
      int64_t n_cand = first;                                        /* blocks below them */
      int64_t picks = topk - window;
      for (int64_t b = 0; b < n_cand; ++b) sc[b] = 0.0;
      for (int32_t cc = 0; cc < d_idx; ++cc) {
        const double qc = (double)q[cc];
        const double *kr = kt + (int64_t)cc * nb_avail;
        for (int64_t b = 0; b < n_cand; ++b) sc[b] += qc * kr[b];
      }
      for (int64_t b = 0; b < n_cand; ++b) {
        c[b].s = sc[b];
        c[b].b = (int32_t)b;
      }
      qsort(c, (size_t)n_cand, sizeof(cand_t), cand_cmp);
      int64_t m = n_cand < picks ? n_cand : picks;
      for (int64_t j = 0; j < m; ++j) keep[j] = c[j].b;
      qsort(keep, (size_t)m, sizeof(int32_t), int_cmp);
      int32_t *row = sel + i * topk;
      int64_t w = 0;
      for (int64_t j = 0; j < m; ++j) row[w++] = keep[j];
      for (int64_t b = first; b <= own; ++b) row[w++] = (int32_t)b;
      for (; w < topk; ++w) row[w] = -1;
      double gr = NAN, ga = NAN, eb = NAN;
      if (picks >= 1 && n_cand > picks) {
        const cand_t *a = &c[picks - 1], *z = &c[picks];
        ga = a->s - z->s;
        double den = fabs(a->s) > fabs(z->s) ? fabs(a->s) : fabs(z->s);
        gr = den > 0.0 ? ga / den : 0.0;
        double sa = 0.0, sz = 0.0;
        for (int32_t cc = 0; cc < d_idx; ++cc) {
          sa += fabs((double)q[cc] * (double)kmax[(int64_t)a->b * d_idx + cc]);
          sz += fabs((double)q[cc] * (double)kmax[(int64_t)z->b * d_idx + cc]);
        }
        eb = gamma * (sa + sz);
      }
      if (gap_rel) gap_rel[i] = gr;
      if (gap_abs) gap_abs[i] = ga;
      if (err_bnd) err_bnd[i] = eb;
    }
    free(c);
    free(sc);
    free(keep);
  }
  free(kt);
  return bad ? ORC_EINVAL : ORC_OK;
}

int oracle_select(const float *idx_q, int64_t n_q, const int64_t *q_pos,
                  const float *kmax, int64_t nb_avail, int32_t d_idx,
                  int32_t block, int32_t topk, int32_t *sel, double *gap_rel,
                  double *gap_abs, double *err_bnd) {
  return oracle_select_window(idx_q, n_q, q_pos, kmax, nb_avail, d_idx, block, topk, 1,
                              sel, gap_rel, gap_abs, err_bnd);
}

/* ------------------------------------------------------------------------
 * Inverse map: queries per KV block, as CSR.
 * [CXT §2.2 "KV Outer Gather Q：MSA 的关键设计"] the outer loop over KV
 * blocks needs, per block, the queries that hit it.
 * Walk queries in ascending order and append i to list[b] for each b in
 * sel[i]; row_ptr is the prefix sum of the list sizes; slot[i][k] is the
 * list position of (i, sel[i][k]) (-1 where sel is -1).
 * Returns nnz, or a negative error.
 * ---------------------------------------------------------------------- */
int64_t oracle_invert(const int32_t *sel, int64_t n_q, int32_t topk,
                      int64_t n_blocks, int32_t *row_ptr, int32_t *q_list,
                      int32_t *slot) {
  if (!sel || !row_ptr || !q_list || !slot || n_q < 0 || topk < 1 ||
      n_blocks < 1)
    return ORC_EINVAL;
  int64_t *cnt = (int64_t *)calloc((size_t)n_blocks, sizeof(int64_t));
  if (!cnt) return ORC_EINVAL;
  for (int64_t i = 0; i < n_q * topk; ++i) {
    int32_t b = sel[i];
    if (b < -1 || b >= n_blocks) {
      free(cnt);
      return ORC_EINVAL;
    }
    if (b >= 0) cnt[b]++;
  }
  row_ptr[0] = 0;
  for (int64_t b = 0; b < n_blocks; ++b)
    row_ptr[b + 1] = row_ptr[b] + (int32_t)cnt[b];
  for (int64_t b = 0; b < n_blocks; ++b) cnt[b] = row_ptr[b];
  for (int64_t i = 0; i < n_q; ++i)
    for (int32_t k = 0; k < topk; ++k) {
      int32_t b = sel[i * topk + k];
      if (b < 0) {
        slot[i * topk + k] = -1;
        continue;
      }
      int64_t s = cnt[b]++;
      q_list[s] = (int32_t)i;
      slot[i * topk + k] = (int32_t)s;
    }
  int64_t nnz = row_ptr[n_blocks];
  free(cnt);
  return nnz;
}

/* ------------------------------------------------------------------------
 * Sparse branch: standard GQA over the union of the selected blocks.
 * [YLY, "稀疏分支（Sparse Branch）"] GQA only over the K chosen blocks, the
 * rest neither loaded nor multiplied; [CXT §2.3 "MSA 算法实现"] softmax of
 * q.k/sqrt(d) over the gathered keys, weights times the gathered values.
 *
 * For eval entry e (query row q_row[e] at position q_pos[e]) and head h,
 * with g = h / (Hq/Hkv):
 *   keys  = union over b in sel[e] (b != -1) of {t : b*B <= t <= min(b*B+B-1, pos)}
 *   s_t   = scale * sum_c q[row][h][c] * k[g][t][c]            (fp64)
 *   m     = max_t s_t,  w_t = exp(s_t - m),  Z = sum_t w_t
 *   o     = sum_t w_t v[g][t][:] / Z,  lse = m + ln Z,  both rounded to fp32.
 * q: [*][Hq][d]; k, v: [Hkv][kv_stride][d]; dtype 0 = fp32, 1 = bf16 bits.
 * Entries of sel above the own block are rejected (they would see the future).
 * n_keys (nullable) receives |keys| per eval entry.
 * ---------------------------------------------------------------------- */
int oracle_attend(const void *q, const void *k, const void *v, int32_t dtype,
                  int64_t n_eval, const int64_t *q_row, const int64_t *q_pos,
                  const int32_t *sel, int32_t topk, int32_t hq, int32_t hkv,
                  int32_t d, int32_t block, int64_t kv_stride, double scale,
                  float *o, float *lse, int64_t *n_keys) {
  if (!q || !k || !v || !q_row || !q_pos || !sel || !o || n_eval < 0 ||
      topk < 1 || hq < 1 || hkv < 1 || hq % hkv || d < 1 || block < 1 ||
      (dtype != 0 && dtype != 1))
    return ORC_EINVAL;
  for (int64_t e = 0; e < n_eval; ++e) {
    int64_t own = q_pos[e] / block;
    if (q_pos[e] < 0 || q_pos[e] >= kv_stride) return ORC_EINVAL;
    for (int32_t j = 0; j < topk; ++j) {
      int32_t b = sel[e * topk + j];
      if (b < -1 || b > own) return ORC_EINVAL;
    }
  }
  const int32_t grp = hq / hkv;
  const int64_t cap = (int64_t)topk * block;   /* at most this many keys per query */
  enum { TILE = 256 };
  int bad = 0;
#pragma omp parallel
  {
    int32_t *blk = (int32_t *)malloc(sizeof(int32_t) * (size_t)topk);
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    double *s = (double *)malloc(sizeof(double) * (size_t)cap * grp);
    double *kt = (double *)malloc(sizeof(double) * (size_t)TILE * d);
    double *vrow = (double *)malloc(sizeof(double) * (size_t)d);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d * grp);
    double *mx = (double *)malloc(sizeof(double) * (size_t)grp);
    double *z = (double *)malloc(sizeof(double) * (size_t)grp);
    const int ok = blk && keys && s && kt && vrow && acc && mx && z;
    if (!ok) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t e = 0; e < n_eval; ++e) {
      if (!ok) continue;
      const int64_t pos = q_pos[e];
      /* the union of the selected blocks: sort, drop repeats and padding */
      int32_t nblk = 0;
      for (int32_t j = 0; j < topk; ++j)
        if (sel[e * topk + j] >= 0) blk[nblk++] = sel[e * topk + j];
      qsort(blk, (size_t)nblk, sizeof(int32_t), int_cmp);
      int64_t nk = 0;
      for (int32_t j = 0; j < nblk; ++j) {
        if (j > 0 && blk[j] == blk[j - 1]) continue;
        int64_t t0 = (int64_t)blk[j] * block, t1 = t0 + block - 1;
        if (t1 > pos) t1 = pos;
        for (int64_t t = t0; t <= t1; ++t) keys[nk++] = t;
      }
      if (n_keys) n_keys[e] = nk;
      /* One KV head at a time, for the grp query heads that read it.  The
       * loops are ordered so that the innermost runs over keys (or columns):
       * every sum below still adds the same products in the same order as
       * the plain per-head form -- s_t over c ascending, Z and o over keys
       * ascending -- so the results are identical to it. */
      for (int32_t g = 0; g < hkv; ++g) {
        /* s[hl][j] = q[row][g*grp+hl] . k[g][keys[j]] */
        for (int64_t j0 = 0; j0 < nk; j0 += TILE) {
          const int64_t nt = nk - j0 < TILE ? nk - j0 : TILE;
          for (int64_t jj = 0; jj < nt; ++jj) {
            const int64_t kb = ((int64_t)g * kv_stride + keys[j0 + jj]) * (int64_t)d;
            elems(k, dtype, kb, d, vrow);
            for (int32_t c = 0; c < d; ++c) kt[(int64_t)c * TILE + jj] = vrow[c];
          }
          for (int32_t hl = 0; hl < grp; ++hl) {
            const int64_t qb = (q_row[e] * hq + (int64_t)g * grp + hl) * (int64_t)d;
            double *sr = s + (int64_t)hl * cap + j0;
            for (int64_t jj = 0; jj < nt; ++jj) sr[jj] = 0.0;
            elems(q, dtype, qb, d, vrow);
            for (int32_t c = 0; c < d; ++c) {
              const double qc = vrow[c];
              const double *kr = kt + (int64_t)c * TILE;
              for (int64_t jj = 0; jj < nt; ++jj) sr[jj] += qc * kr[jj];
            }
          }
        }
        /* scale, row max, then the softmax-weighted sum of the values */
        for (int32_t hl = 0; hl < grp; ++hl) {
          double *sr = s + (int64_t)hl * cap;
          double m = -INFINITY;
          for (int64_t j = 0; j < nk; ++j) {
            sr[j] = scale * sr[j];
            if (sr[j] > m) m = sr[j];
          }
          mx[hl] = m;
          z[hl] = 0.0;
          for (int32_t c = 0; c < d; ++c) acc[(int64_t)hl * d + c] = 0.0;
        }
        for (int64_t j = 0; j < nk; ++j) {
          const int64_t vb = ((int64_t)g * kv_stride + keys[j]) * (int64_t)d;
          elems(v, dtype, vb, d, vrow);
          for (int32_t hl = 0; hl < grp; ++hl) {
            const double w = exp(s[(int64_t)hl * cap + j] - mx[hl]);
            double *ar = acc + (int64_t)hl * d;
            z[hl] += w;
            for (int32_t c = 0; c < d; ++c) ar[c] += w * vrow[c];
          }
        }
        for (int32_t hl = 0; hl < grp; ++hl) {
          const int64_t h = (int64_t)g * grp + hl;
          float *out = o + (e * hq + h) * (int64_t)d;
          for (int32_t c = 0; c < d; ++c) out[c] = (float)(acc[(int64_t)hl * d + c] / z[hl]);
          if (lse) lse[e * hq + h] = (float)(mx[hl] + log(z[hl]));
        }
      }
    }
    free(blk);
    free(keys);
    free(s);
    free(kt);
    free(vrow);
    free(acc);
    free(mx);
    free(z);
  }
  return bad ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------------------
 * FP8 KV pages, dequantised.  [CXT §3.3 "Prefilling 与 Decoding 的差异化优化"]
 * keeps the KV cache in blocks and in reduced precision; the reading taken
 * here is OCP FP8 E4M3 (the variant without infinities) with one fp32 scale
 * per (page, KV head) for K and one for V.
 *
 * A code is 1 sign bit s, 4 exponent bits e (bias 7) and 3 mantissa bits m:
 *   e >= 1:             (-1)^s * 2^(e-7) * (1 + m/8)      (e = 15, m = 7: NaN)
 *   e == 0:             (-1)^s * 2^-6 * (m/8)             (subnormals, signed 0)
 * out[p][g][i] = scale[p][g] * value(x[p][g][i]), the product rounded once to
 * fp32 (it is exact in double: 24 + 4 significant bits).
 * x: [n_pages][hkv][row_len] codes; scale: [n_pages][hkv]; out likewise fp32.
 * ---------------------------------------------------------------------- */
static double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

int oracle_dequant_e4m3(const uint8_t *x, int64_t n_pages, int32_t hkv, int64_t row_len,
                        const float *scale, float *out) {
  if (!x || !scale || !out || n_pages < 0 || hkv < 1 || row_len < 0) return ORC_EINVAL;
  for (int64_t p = 0; p < n_pages; ++p)
    for (int32_t g = 0; g < hkv; ++g) {
      const double sc = (double)scale[p * hkv + g];
      const int64_t base = (p * hkv + g) * row_len;
      for (int64_t i = 0; i < row_len; ++i) out[base + i] = (float)(sc * e4m3_value(x[base + i]));
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Work counters taken from an actual selection: the number of (query, block)
 * pairs and the number of attended (query, key) pairs.  The attended FLOPs
 * are 4*d*Hq per attended pair (2d for q.k, 2d for p*v).
 * ---------------------------------------------------------------------- */
int oracle_counts(const int32_t *sel, int64_t n_q, int32_t topk,
                  const int64_t *q_pos, int32_t block, int64_t *nnz,
                  int64_t *attended) {
  if (!sel || !q_pos || !nnz || !attended || topk < 1 || block < 1)
    return ORC_EINVAL;
  int64_t a = 0, z = 0;
  for (int64_t i = 0; i < n_q; ++i)
    for (int32_t j = 0; j < topk; ++j) {
      int32_t b = sel[i * topk + j];
      if (b < 0) continue;
      int64_t t0 = (int64_t)b * block, t1 = t0 + block - 1;
      if (t1 > q_pos[i]) t1 = q_pos[i];
      z += 1;
      a += t1 - t0 + 1;
    }
  *nnz = z;
  *attended = a;
  return ORC_OK;
}
