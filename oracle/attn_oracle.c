/*
 * attn_oracle.c -- plain, slow, f64 CPU oracle for the softmax-attention backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call this
 * file: only the test suite, the package smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the definition written out, no tiling, no fusion, no reordering):
 *   TileOPs PR #2281 page, "TileFoundry Description", the Reference program: the whole
 *   backward in one piece --
 *     delta_i  = sum_d O[i,d] * dO[i,d]                      (from the O the caller gives)
 *     s_ij     = q_i . k_j
 *     p_ij     = exp2(s_ij * scale * log2(e) - lse_i)        (lse is base 2)
 *     p_ij     = 0 where key j is masked for query i
 *     dV       = P^T dO
 *     dp_ij    = dO_i . v_j
 *     ds_ij    = p_ij * (dp_ij - delta_i)   [* scale]
 *     dQ       = dS K,   dK = dS^T Q
 *   The page applies the softmax scale to dS; the Tiled program on the same page moves it
 *   onto dQ and dK once at the end.  Both are the same number; here the scale multiplies
 *   dq and dk where they are formed.
 * Generalised, as the other pages ask, to
 *   - grouped-query attention (flash-linear-attention issue #8, "Problem" and the proposed
 *     KV-head-owned kernel): query head h reads KV head g = h / G with G = Hq / Hkv, and dK,
 *     dV of KV head g sum the contributions of all G query heads of the group;
 *   - a sliding window (same issue, correctness contract): key j is visible to query i iff
 *     i + off - window < j <= i + off;
 *   - a gathered top-k key set per query (TileLang PR #2592, sparse MLA backward): the keys
 *     of query (b,i) for KV head g are idx[b,i,g,0..topk); each entry counts once per
 *     occurrence; entries outside [0,Skv) or (when causal) beyond i + off are masked;
 *   - Sq != Skv with bottom-right causal alignment off = Skv - Sq, and Dqk != Dv.
 * Readings where the pages are silent: rows whose allowed key set is empty, or whose lse is
 * -inf, contribute nothing (dq row 0); key rows that no query reaches get dk = dv = 0.
 *
 * Layouts (BSHD, row-major, contiguous):
 *   q [B,Sq,Hq,Dqk]  k [B,Skv,Hkv,Dqk]  v [B,Skv,Hkv,Dv]  o, dout [B,Sq,Hq,Dv]
 *   lse [B,Hq,Sq]    idx [B,Sq,Hkv,topk] (int32) or NULL for dense
 * Element inputs are double arrays (the stored fp16/bf16 values widened exactly, or any f64
 * values for the finite-difference checks); every product and sum is carried out in double.
 * Outputs are double, same layouts.
 *
 * The backward runs in two race-free passes: pass A owns one query row and forms dq;
 * pass B owns one key row and walks every query that reaches it, recomputing p and ds,
 * to form dk and dv.  The two passes evaluate ds independently of each other.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t B, Sq, Skv, Hq, Hkv, Dqk, Dv, topk;
  double scale;
  int32_t causal;
  int32_t window;
} oracle_shape;

#define LOG2E 1.4426950408889634

/* element addresses */
static inline int64_t iq(const oracle_shape *s, int64_t b, int64_t i, int64_t h) { return ((b * s->Sq + i) * s->Hq + h) * s->Dqk; }
static inline int64_t io(const oracle_shape *s, int64_t b, int64_t i, int64_t h) { return ((b * s->Sq + i) * s->Hq + h) * s->Dv; }
static inline int64_t ik(const oracle_shape *s, int64_t b, int64_t j, int64_t g) { return ((b * s->Skv + j) * s->Hkv + g) * s->Dqk; }
static inline int64_t iv(const oracle_shape *s, int64_t b, int64_t j, int64_t g) { return ((b * s->Skv + j) * s->Hkv + g) * s->Dv; }
static inline int64_t il(const oracle_shape *s, int64_t b, int64_t h, int64_t i) { return (b * s->Hq + h) * s->Sq + i; }
static inline int64_t ii(const oracle_shape *s, int64_t b, int64_t i, int64_t g) { return ((b * s->Sq + i) * s->Hkv + g) * s->topk; }

static int check_shape(const oracle_shape *s) {
  if (s->B < 0 || s->Sq < 0 || s->Skv < 0 || s->Hq < 1 || s->Hkv < 1 || s->Dqk < 1 || s->Dv < 1) return -1;
  if (s->Hq % s->Hkv != 0) return -1;
  if (s->window < 0) return -1;
  return 0;
}

/* Dense mask: may query i see key j?  (bottom-right causal alignment, window counted in keys
 * including the diagonal). */
static int dense_allowed(const oracle_shape *s, int64_t i, int64_t j) {
  int64_t off = s->Skv - s->Sq;
  if (j < 0 || j >= s->Skv) return 0;
  if (s->causal && j > i + off) return 0;
  if (s->window > 0 && j <= i + off - s->window) return 0;
  return 1;
}

/* Sparse mask for one index entry. */
static int sparse_entry_valid(const oracle_shape *s, int64_t i, int64_t j) {
  int64_t off = s->Skv - s->Sq;
  if (j < 0 || j >= s->Skv) return 0;
  if (s->causal && j > i + off) return 0;
  return 1;
}

static double dot(const double *a, const double *b, int64_t n) {
  double acc = 0.0;
  for (int64_t d = 0; d < n; d++) acc += a[d] * b[d];
  return acc;
}

/* ------------------------------------------------------------------ forward (for inputs) */
/* O and base-2 lse of the masked softmax attention over the same key sets.  Used to build
 * the inputs O and lse; a row with no allowed key gets o = 0 and lse = -inf. */
int oracle_fwd(const oracle_shape *s, const double *q, const double *k, const double *v, const int32_t *idx,
               double *o, double *lse) {
  if (check_shape(s)) return -1;
  const int64_t G = s->Hq / s->Hkv;
  const double c = s->scale * LOG2E;
  const int64_t nrows = s->B * s->Sq * s->Hq;
#pragma omp parallel
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)s->Dv);
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < nrows; r++) {
      const int64_t h = r % s->Hq, i = (r / s->Hq) % s->Sq, b = r / (s->Hq * s->Sq);
      const int64_t g = h / G;
      const double *qi = q + iq(s, b, i, h);
      int64_t nkeys = idx ? s->topk : s->Skv;
      /* pass 1: max logit */
      double m = -INFINITY;
      int any = 0;
      for (int64_t t = 0; t < nkeys; t++) {
        int64_t j = idx ? (int64_t)idx[ii(s, b, i, g) + t] : t;
        if (idx ? !sparse_entry_valid(s, i, j) : !dense_allowed(s, i, j)) continue;
        double x = dot(qi, k + ik(s, b, j, g), s->Dqk) * c;
        if (x > m) m = x;
        any = 1;
      }
      double *orow = o + io(s, b, i, h);
      if (!any) {
        for (int64_t d = 0; d < s->Dv; d++) orow[d] = 0.0;
        lse[il(s, b, h, i)] = -INFINITY;
        continue;
      }
      /* pass 2: normaliser and weighted values */
      double sum = 0.0;
      for (int64_t d = 0; d < s->Dv; d++) acc[d] = 0.0;
      for (int64_t t = 0; t < nkeys; t++) {
        int64_t j = idx ? (int64_t)idx[ii(s, b, i, g) + t] : t;
        if (idx ? !sparse_entry_valid(s, i, j) : !dense_allowed(s, i, j)) continue;
        double w = exp2(dot(qi, k + ik(s, b, j, g), s->Dqk) * c - m);
        sum += w;
        const double *vj = v + iv(s, b, j, g);
        for (int64_t d = 0; d < s->Dv; d++) acc[d] += w * vj[d];
      }
      for (int64_t d = 0; d < s->Dv; d++) orow[d] = acc[d] / sum;
      lse[il(s, b, h, i)] = m + log2(sum);
    }
    free(acc);
  }
  return 0;
}

/* ------------------------------------------------------------------ backward pieces */
static double row_delta(const oracle_shape *s, const double *o, const double *dout, int64_t b, int64_t i, int64_t h) {
  return dot(o + io(s, b, i, h), dout + io(s, b, i, h), s->Dv);
}

/* delta [B,Hq,Sq] = rowsum(O * dO) */
int oracle_delta(const oracle_shape *s, const double *o, const double *dout, double *delta) {
  if (check_shape(s)) return -1;
  const int64_t nrows = s->B * s->Hq * s->Sq;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; r++) {
    const int64_t i = r % s->Sq, h = (r / s->Sq) % s->Hq, b = r / (s->Sq * s->Hq);
    delta[r] = row_delta(s, o, dout, b, i, h);
  }
  return 0;
}

/* Pass A: dq for one query row (b,i,h), written to out[0..Dqk). */
static void dq_row(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
                   const double *dout, const double *lse, const int32_t *idx, int64_t b, int64_t i, int64_t h,
                   double *out) {
  const int64_t G = s->Hq / s->Hkv, g = h / G;
  const double c = s->scale * LOG2E;
  for (int64_t d = 0; d < s->Dqk; d++) out[d] = 0.0;
  const double l = lse[il(s, b, h, i)];
  if (l == -INFINITY) return;
  const double delta = row_delta(s, o, dout, b, i, h);
  const double *qi = q + iq(s, b, i, h);
  const double *doi = dout + io(s, b, i, h);
  int64_t nkeys = idx ? s->topk : s->Skv;
  for (int64_t t = 0; t < nkeys; t++) {
    int64_t j = idx ? (int64_t)idx[ii(s, b, i, g) + t] : t;
    if (idx ? !sparse_entry_valid(s, i, j) : !dense_allowed(s, i, j)) continue;
    const double *kj = k + ik(s, b, j, g);
    double p = exp2(dot(qi, kj, s->Dqk) * c - l);
    double dp = dot(doi, v + iv(s, b, j, g), s->Dv);
    double ds = p * (dp - delta);
    for (int64_t d = 0; d < s->Dqk; d++) out[d] += s->scale * ds * kj[d];
  }
}

/* Inverse of the top-k index: for each (b,g,j), the query rows i that list key j, once per
 * occurrence.  CSR over key rows: start[(b*Hkv+g)*Skv + j] .. start[...+1]. */
typedef struct {
  int64_t *start;
  int64_t *qrow;
} inv_index;

static int build_inverse(const oracle_shape *s, const int32_t *idx, inv_index *inv) {
  const int64_t nkey = s->B * s->Hkv * s->Skv;
  inv->start = (int64_t *)calloc((size_t)nkey + 1, sizeof(int64_t));
  if (!inv->start) return -1;
  for (int64_t b = 0; b < s->B; b++)
    for (int64_t i = 0; i < s->Sq; i++)
      for (int64_t g = 0; g < s->Hkv; g++)
        for (int64_t t = 0; t < s->topk; t++) {
          int64_t j = idx[ii(s, b, i, g) + t];
          if (sparse_entry_valid(s, i, j)) inv->start[(b * s->Hkv + g) * s->Skv + j + 1]++;
        }
  for (int64_t x = 0; x < nkey; x++) inv->start[x + 1] += inv->start[x];
  inv->qrow = (int64_t *)malloc(sizeof(int64_t) * (size_t)(inv->start[nkey] > 0 ? inv->start[nkey] : 1));
  int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nkey > 0 ? nkey : 1));
  if (!inv->qrow || !fill) { free(fill); return -1; }
  for (int64_t x = 0; x < nkey; x++) fill[x] = inv->start[x];
  for (int64_t b = 0; b < s->B; b++)
    for (int64_t i = 0; i < s->Sq; i++)
      for (int64_t g = 0; g < s->Hkv; g++)
        for (int64_t t = 0; t < s->topk; t++) {
          int64_t j = idx[ii(s, b, i, g) + t];
          if (sparse_entry_valid(s, i, j)) inv->qrow[fill[(b * s->Hkv + g) * s->Skv + j]++] = i;
        }
  free(fill);
  return 0;
}

static void free_inverse(inv_index *inv) {
  free(inv->start);
  free(inv->qrow);
}

/* Contribution of query row (b,i,h) to key row (b,j,g): adds to dk_out and dv_out. */
static void add_pair(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
                     const double *dout, const double *lse, int64_t b, int64_t i, int64_t h, int64_t j, int64_t g,
                     double *dk_out, double *dv_out) {
  const double c = s->scale * LOG2E;
  const double l = lse[il(s, b, h, i)];
  if (l == -INFINITY) return;
  const double *qi = q + iq(s, b, i, h);
  const double *doi = dout + io(s, b, i, h);
  double p = exp2(dot(qi, k + ik(s, b, j, g), s->Dqk) * c - l);
  double dp = dot(doi, v + iv(s, b, j, g), s->Dv);
  double ds = p * (dp - row_delta(s, o, dout, b, i, h));
  for (int64_t d = 0; d < s->Dqk; d++) dk_out[d] += s->scale * ds * qi[d];
  for (int64_t d = 0; d < s->Dv; d++) dv_out[d] += p * doi[d];
}

/* Pass B: dk, dv for one key row (b,j,g). */
static void dkv_row(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
                    const double *dout, const double *lse, const inv_index *inv, int64_t b, int64_t j, int64_t g,
                    double *dk_out, double *dv_out) {
  const int64_t G = s->Hq / s->Hkv;
  for (int64_t d = 0; d < s->Dqk; d++) dk_out[d] = 0.0;
  for (int64_t d = 0; d < s->Dv; d++) dv_out[d] = 0.0;
  for (int64_t hh = 0; hh < G; hh++) {
    const int64_t h = g * G + hh;
    if (inv) {
      const int64_t x = (b * s->Hkv + g) * s->Skv + j;
      for (int64_t e = inv->start[x]; e < inv->start[x + 1]; e++)
        add_pair(s, q, k, v, o, dout, lse, b, inv->qrow[e], h, j, g, dk_out, dv_out);
    } else {
      for (int64_t i = 0; i < s->Sq; i++)
        if (dense_allowed(s, i, j)) add_pair(s, q, k, v, o, dout, lse, b, i, h, j, g, dk_out, dv_out);
    }
  }
}

/* ------------------------------------------------------------------ public entry points */
/* Full backward: dq [B,Sq,Hq,Dqk], dk [B,Skv,Hkv,Dqk], dv [B,Skv,Hkv,Dv]. */
int oracle_bwd(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
               const double *dout, const double *lse, const int32_t *idx, double *dq, double *dk, double *dv) {
  if (check_shape(s)) return -1;
  if (idx && s->topk < 1) return -1;
  inv_index inv = {0, 0};
  if (idx && build_inverse(s, idx, &inv)) return -2;
  const int64_t nq = s->B * s->Sq * s->Hq;
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t r = 0; r < nq; r++) {
    const int64_t h = r % s->Hq, i = (r / s->Hq) % s->Sq, b = r / (s->Hq * s->Sq);
    dq_row(s, q, k, v, o, dout, lse, idx, b, i, h, dq + iq(s, b, i, h));
  }
  const int64_t nk = s->B * s->Skv * s->Hkv;
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t r = 0; r < nk; r++) {
    const int64_t g = r % s->Hkv, j = (r / s->Hkv) % s->Skv, b = r / (s->Hkv * s->Skv);
    dkv_row(s, q, k, v, o, dout, lse, idx ? &inv : 0, b, j, g, dk + ik(s, b, j, g), dv + iv(s, b, j, g));
  }
  if (idx) free_inverse(&inv);
  return 0;
}

/* dq for a list of query rows: rows[3*n + {0,1,2}] = (b, i, h); out [n, Dqk]. */
int oracle_bwd_dq_rows(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
                       const double *dout, const double *lse, const int32_t *idx, const int64_t *rows, int64_t n,
                       double *out) {
  if (check_shape(s)) return -1;
  for (int64_t r = 0; r < n; r++)
    if (rows[3 * r] < 0 || rows[3 * r] >= s->B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= s->Sq ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= s->Hq)
      return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n; r++)
    dq_row(s, q, k, v, o, dout, lse, idx, rows[3 * r], rows[3 * r + 1], rows[3 * r + 2], out + r * s->Dqk);
  return 0;
}

/* dk, dv for a list of key rows: rows[3*n + {0,1,2}] = (b, j, g); dk_out [n, Dqk], dv_out [n, Dv]. */
int oracle_bwd_dkv_rows(const oracle_shape *s, const double *q, const double *k, const double *v, const double *o,
                        const double *dout, const double *lse, const int32_t *idx, const int64_t *rows, int64_t n,
                        double *dk_out, double *dv_out) {
  if (check_shape(s)) return -1;
  if (idx && s->topk < 1) return -1;
  for (int64_t r = 0; r < n; r++)
    if (rows[3 * r] < 0 || rows[3 * r] >= s->B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= s->Skv ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= s->Hkv)
      return -1;
  inv_index inv = {0, 0};
  if (idx && build_inverse(s, idx, &inv)) return -2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n; r++)
    dkv_row(s, q, k, v, o, dout, lse, idx ? &inv : 0, rows[3 * r], rows[3 * r + 1], rows[3 * r + 2],
            dk_out + r * s->Dqk, dv_out + r * s->Dv);
  if (idx) free_inverse(&inv);
  return 0;
}
