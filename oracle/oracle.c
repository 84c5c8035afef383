/*
 * CPU oracle for PARK block retrieval and block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or helper
 * with the GPU library; the two meet only through the seeded synthetic inputs.
 *
 * Everything is plain and slow on purpose: storage of inputs and of the quantities the
 * method itself keeps in single precision (transformed keys, centroids) is float, every
 * sum, product and transcendental is double, loops follow the definitions in the order
 * the pages write them.  OpenMP only splits independent rows over threads; no loop
 * reorders a sum.
 *
 * Source: "PARK: Accurate Block Retrieval for Sparse Attention in Video Diffusion
 * Transformers" (paperpeel.com/paper/2609.38978).  Section / equation references below
 * are to that page unless another page is named.
 *
 * Readings of the page where it is garbled or silent (each also listed in the design
 * notes):
 *   - the attention / PAMA score scale printed as "/d" is taken as 1/sqrt(d) (the caller
 *     passes the scale explicitly, so the literal 1/d can be run too);
 *   - the shrinkage formula after the s_Q definition (App. D.2, "Numerically stable
 *     Cholesky factorization") is lost; the text says alpha = 0 gives the query metric up
 *     to a small stability term and alpha = 1 an isotropic metric up to scale, so
 *     Gs = (1 - alpha) G + (alpha + eps) s_Q I;
 *   - k-means starts from keys at positions floor(v L / N_K) unless indices are given,
 *     runs exactly T Lloyd steps, breaks argmin ties to the lowest index and keeps the old
 *     centroid of an empty cluster;
 *   - an empty key block has log-mass -inf, never enters the top-p prefix and does not
 *     count toward the top-k floor;
 *   - top-p keeps the shortest prefix of the ranking (W descending, block id ascending)
 *     whose mass reaches p times the row total; the top-k floor is the union of that
 *     prefix with the first k of the same ranking (SCOPE, paperpeel.com/paper/2608.12780,
 *     appendix "Online Per-Head Top-k Selection": the union of two prefixes of one
 *     ranking holds max(t_p, k) items);
 *   - sparse attention is the softmax renormalised over the selected keys (what a
 *     block-sparse flash kernel computes); the unnormalised (A .* M) V of section 3.1 is
 *     recall times that output, and both follow from O and the log-sum-exp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------------------------
 * Query-response metric (section 5.2 and App. D.2 "Query-induced clustering metric",
 * "Euclidean realization", "Numerically stable Cholesky factorization").
 *   G_Q = (1/L) sum_i q_i q_i^T
 *   s_Q = max(tr(G_Q)/d, s_min)
 *   Gs  = (1 - alpha) G_Q + (alpha + eps) s_Q I
 *   Gs  = R R^T, R lower triangular (Cholesky)
 * metric 1 (Euclidean) sets R = I.  Returns 0, or 1 if the factorisation fails (a pivot
 * that is not a finite positive number, which for finite queries the (alpha + eps) s_Q I
 * term rules out); the head then falls back to R = I, the Euclidean metric, so that it is
 * still clustered (App. D.2 "Numerically stable Cholesky factorization" asks for a
 * per-head flag; the fallback is the reading the GPU path follows too).
 * G, Gs, R: d*d row-major doubles (may be NULL except R).
 * --------------------------------------------------------------------------------- */
ORC_EXPORT int orc_query_metric(const float* Q, long L, int d, int metric, double alpha,
                                double eps, double s_min, double* G_out, double* Gs_out,
                                double* R) {
  double* G = (double*)calloc((size_t)d * d, sizeof(double));
  double* Gs = (double*)calloc((size_t)d * d, sizeof(double));
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b) {
      double s = 0.0;
      for (long i = 0; i < L; ++i) s += (double)Q[i * d + a] * (double)Q[i * d + b];
      G[a * d + b] = s / (double)L;
    }
  double tr = 0.0;
  for (int a = 0; a < d; ++a) tr += G[a * d + a];
  double sQ = tr / d;
  if (!(sQ > s_min)) sQ = s_min;
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b)
      Gs[a * d + b] = (1.0 - alpha) * G[a * d + b] + (a == b ? (alpha + eps) * sQ : 0.0);
  int fail = 0;
  memset(R, 0, sizeof(double) * (size_t)d * d);
  if (metric == 1) {
    for (int a = 0; a < d; ++a) R[a * d + a] = 1.0;
  } else {
    /* Cholesky-Banachiewicz: row by row, R[i][j] for j <= i. */
    for (int i = 0; i < d && !fail; ++i) {
      for (int j = 0; j <= i; ++j) {
        double s = Gs[i * d + j];
        for (int k = 0; k < j; ++k) s -= R[i * d + k] * R[j * d + k];
        if (i == j) {
          if (!(s > 0.0) || !isfinite(s)) { fail = 1; break; }
          R[i * d + i] = sqrt(s);
        } else {
          R[i * d + j] = s / R[j * d + j];
        }
      }
    }
  }
  if (fail) {
    memset(R, 0, sizeof(double) * (size_t)d * d);
    for (int a = 0; a < d; ++a) R[a * d + a] = 1.0;
  }
  if (G_out) memcpy(G_out, G, sizeof(double) * (size_t)d * d);
  if (Gs_out) memcpy(Gs_out, Gs, sizeof(double) * (size_t)d * d);
  free(G);
  free(Gs);
  return fail;
}

/* Transformed keys (section 5.2, G_Q = R R^T, k~_j = R^T k_j), rounded to float. */
ORC_EXPORT void orc_transform(const float* K, long L, int d, const double* R, float* Kt) {
#pragma omp parallel for schedule(static)
  for (long j = 0; j < L; ++j)
    for (int a = 0; a < d; ++a) {
      double s = 0.0;
      for (int c = 0; c < d; ++c) s += R[c * d + a] * (double)K[j * d + c];  /* (R^T k)_a */
      Kt[j * d + a] = (float)s;
    }
}

/* Initial centroids: the transformed key at floor(v L / N_K), or at init_idx[v]. */
ORC_EXPORT void orc_init_centroids(const float* Kt, long L, int d, int nk, const int* init_idx,
                                   float* C) {
  for (int v = 0; v < nk; ++v) {
    long j = init_idx ? (long)init_idx[v] : (long)(((long long)v * L) / nk);
    memcpy(C + (size_t)v * d, Kt + (size_t)j * d, sizeof(float) * d);
  }
}

/* Squared Euclidean distance in the transformed space (the E10 form of the QRKC metric). */
static double sqdist(const float* x, const float* c, int d) {
  double s = 0.0;
  for (int a = 0; a < d; ++a) {
    double t = (double)x[a] - (double)c[a];
    s += t * t;
  }
  return s;
}

/* Lloyd assignment step: a_j = argmin_v ||k~_j - c~_v||^2, ties to the lowest v.
 * margin[j] = (D2 - D1) / D2 with D1 <= D2 the two smallest distances (1 if N_K = 1,
 * 0 if D2 = 0).  Returns J = sum_j D1(j). */
ORC_EXPORT double orc_assign(const float* Kt, long L, int d, const float* C, int nk, int* labels,
                             double* margin, double* dist) {
  double* D1 = (double*)malloc(sizeof(double) * (size_t)L);
#pragma omp parallel for schedule(static)
  for (long j = 0; j < L; ++j) {
    double b1 = INFINITY, b2 = INFINITY;
    int a = 0;
    for (int v = 0; v < nk; ++v) {
      double D = sqdist(Kt + (size_t)j * d, C + (size_t)v * d, d);
      if (D < b1) { b2 = b1; b1 = D; a = v; }
      else if (D < b2) b2 = D;
    }
    labels[j] = a;
    D1[j] = b1;
    if (margin) margin[j] = (nk == 1) ? 1.0 : (b2 > 0.0 ? (b2 - b1) / b2 : 0.0);
    if (dist) dist[j] = b1;
  }
  double J = 0.0;
  for (long j = 0; j < L; ++j) J += D1[j];
  free(D1);
  return J;
}

/* Lloyd update step: c~_v = mean of the transformed keys with label v, the sum in double in
 * key order, rounded to float; a cluster without keys keeps its centroid. */
ORC_EXPORT void orc_update(const float* Kt, long L, int d, const int* labels, int nk, float* C) {
  double* S = (double*)calloc((size_t)nk * d, sizeof(double));
  long* n = (long*)calloc((size_t)nk, sizeof(long));
  for (long j = 0; j < L; ++j) {
    int v = labels[j];
    n[v] += 1;
    for (int a = 0; a < d; ++a) S[(size_t)v * d + a] += (double)Kt[(size_t)j * d + a];
  }
  for (int v = 0; v < nk; ++v)
    if (n[v] > 0)
      for (int a = 0; a < d; ++a) C[(size_t)v * d + a] = (float)(S[(size_t)v * d + a] / (double)n[v]);
  free(S);
  free(n);
}

/* Objective with given labels and centroids: sum_j ||k~_j - c~_{a_j}||^2. */
ORC_EXPORT double orc_objective(const float* Kt, long L, int d, const float* C, const int* labels) {
  double J = 0.0;
  for (long j = 0; j < L; ++j) J += sqdist(Kt + (size_t)j * d, C + (size_t)labels[j] * d, d);
  return J;
}

/* Final clustering outputs (section 5.1 E7 and the reorder of section 5.2 "Clustering and
 * Reuse Strategy"): n_v, offsets = exclusive scan of n_v (offsets[N_K] = L), perm = key
 * indices in (label, index) order, c_v = mean of the ORIGINAL keys of cluster v (0 if
 * empty), summed in double and rounded to float. */
ORC_EXPORT void orc_finalize(const float* K, long L, int d, const int* labels, int nk, float* cent,
                             int* counts, int* perm, int* offsets) {
  double* S = (double*)calloc((size_t)nk * d, sizeof(double));
  memset(counts, 0, sizeof(int) * (size_t)nk);
  for (long j = 0; j < L; ++j) {
    int v = labels[j];
    counts[v] += 1;
    for (int a = 0; a < d; ++a) S[(size_t)v * d + a] += (double)K[(size_t)j * d + a];
  }
  offsets[0] = 0;
  for (int v = 0; v < nk; ++v) offsets[v + 1] = offsets[v] + counts[v];
  int* fill = (int*)malloc(sizeof(int) * (size_t)nk);
  for (int v = 0; v < nk; ++v) fill[v] = offsets[v];
  for (long j = 0; j < L; ++j) perm[fill[labels[j]]++] = (int)j;
  for (int v = 0; v < nk; ++v)
    for (int a = 0; a < d; ++a)
      cent[(size_t)v * d + a] = counts[v] > 0 ? (float)(S[(size_t)v * d + a] / (double)counts[v]) : 0.0f;
  free(fill);
  free(S);
}

/* Query blocks: 64-token (q_block) runs of consecutive queries; the last may be short. */
static long qblock_begin(long u, int qb) { return u * (long)qb; }
static long qblock_end(long u, int qb, long L) {
  long e = (u + 1) * (long)qb;
  return e < L ? e : L;
}

/* PAMA (section 5.1, E7 and E8):
 *   S_iv = scale q_i . c_v + log n_v        (n_v = 0  ->  -inf)
 *   P_iv = exp(S_iv) / sum_r exp(S_ir)       (computed as exp(S_iv - max_r S_ir) / ...)
 *   W_uv = (1/n_u) sum_{i in Q_u} P_iv
 * W: [NQ, N_K] doubles. */
ORC_EXPORT void orc_pama(const float* Q, long L, int d, const float* cent, const int* counts, int nk,
                         int qb, double scale, double* W) {
  long nq = (L + qb - 1) / qb;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < nq; ++u) {
    double* S = (double*)malloc(sizeof(double) * (size_t)nk);
    double* Wu = W + (size_t)u * nk;
    for (int v = 0; v < nk; ++v) Wu[v] = 0.0;
    long i0 = qblock_begin(u, qb), i1 = qblock_end(u, qb, L);
    for (long i = i0; i < i1; ++i) {
      double m = -INFINITY;
      for (int v = 0; v < nk; ++v) {
        if (counts[v] > 0) {
          double dot = 0.0;
          for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)cent[(size_t)v * d + a];
          S[v] = scale * dot + log((double)counts[v]);
        } else {
          S[v] = -INFINITY;
        }
        if (S[v] > m) m = S[v];
      }
      double z = 0.0;
      for (int v = 0; v < nk; ++v) z += exp(S[v] - m);
      for (int v = 0; v < nk; ++v) Wu[v] += exp(S[v] - m) / z;
    }
    for (int v = 0; v < nk; ++v) Wu[v] /= (double)(i1 - i0);
    free(S);
  }
}

/* Query-centroid ("w/o PAMA") estimate of section 4.1 / section 6.3:
 *   qbar_u = (1/n_u) sum_{i in Q_u} q_i,  W_uv = softmax_v(scale qbar_u . c_v + log n_v). */
ORC_EXPORT void orc_pooled_scores(const float* Q, long L, int d, const float* cent, const int* counts,
                                  int nk, int qb, double scale, double* W) {
  long nq = (L + qb - 1) / qb;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < nq; ++u) {
    double* qbar = (double*)calloc((size_t)d, sizeof(double));
    double* Wu = W + (size_t)u * nk;
    long i0 = qblock_begin(u, qb), i1 = qblock_end(u, qb, L);
    for (long i = i0; i < i1; ++i)
      for (int a = 0; a < d; ++a) qbar[a] += (double)Q[(size_t)i * d + a];
    for (int a = 0; a < d; ++a) qbar[a] /= (double)(i1 - i0);
    double m = -INFINITY;
    for (int v = 0; v < nk; ++v) {
      if (counts[v] > 0) {
        double dot = 0.0;
        for (int a = 0; a < d; ++a) dot += qbar[a] * (double)cent[(size_t)v * d + a];
        Wu[v] = scale * dot + log((double)counts[v]);
      } else {
        Wu[v] = -INFINITY;
      }
      if (Wu[v] > m) m = Wu[v];
    }
    double z = 0.0;
    for (int v = 0; v < nk; ++v) z += exp(Wu[v] - m);
    for (int v = 0; v < nk; ++v) Wu[v] = exp(Wu[v] - m) / z;
    free(qbar);
  }
}

/* Ranking used by the selection: W descending, then block id ascending; empty blocks last. */
typedef struct {
  double w;
  int v;
  int empty;
} rank_item;

static int rank_cmp(const void* pa, const void* pb) {
  const rank_item* a = (const rank_item*)pa;
  const rank_item* b = (const rank_item*)pb;
  if (a->empty != b->empty) return a->empty - b->empty;
  if (a->w > b->w) return -1;
  if (a->w < b->w) return 1;
  return a->v - b->v;
}

/* Top-p with a top-k floor, per query block (section 6.1, p = 0.9; SCOPE appendix
 * "Online Per-Head Top-k Selection" for the floor):
 *   t_p   = smallest t >= 1 with sum_{r<=t} W_(r) >= p * sum_v W_uv   (t_p = 0 when p = 0)
 *   count = min(max(t_p, k), number of non-empty blocks)
 * mask[u][v] = 1 for the first `count` of the ranking; list[u][:count] are those block
 * ids ascending, the rest of the row -1.  Margins (for the parity tests):
 *   cut_margin[u] = min(cum_{t_p} - p*total, p*total - cum_{t_p - 1})  (inf if p = 0)
 *   gap_margin[u] = W_(count) - W_(count+1) between the last kept and the first dropped
 *                   non-empty block (inf if none is dropped). */
ORC_EXPORT void orc_select(const double* W, long nq, int nk, const int* counts, double p, int k,
                           uint8_t* mask, int* list, int* count, double* cut_margin,
                           double* gap_margin) {
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < nq; ++u) {
    const double* Wu = W + (size_t)u * nk;
    rank_item* it = (rank_item*)malloc(sizeof(rank_item) * (size_t)nk);
    int nonempty = 0;
    for (int v = 0; v < nk; ++v) {
      it[v].w = Wu[v];
      it[v].v = v;
      it[v].empty = counts[v] == 0;
      nonempty += counts[v] > 0;
    }
    qsort(it, (size_t)nk, sizeof(rank_item), rank_cmp);
    /* The row total is summed in ranking order, the order of the prefix sums below, so
     * the full prefix always reaches p * total for p <= 1. */
    double total = 0.0;
    for (int r = 0; r < nk; ++r) total += it[r].w;
    double target = p * total;
    int tp = 0;
    double cm = INFINITY;
    if (p > 0.0) {
      double cum = 0.0, prev = 0.0;
      for (int t = 1; t <= nk; ++t) {
        prev = cum;
        cum += it[t - 1].w;
        if (cum >= target) {
          tp = t;
          double a = cum - target, b = target - prev;
          cm = a < b ? a : b;
          break;
        }
      }
    }
    int c = tp > k ? tp : k;
    if (c > nonempty) c = nonempty;
    uint8_t* mu = mask + (size_t)u * nk;
    int* lu = list + (size_t)u * nk;
    for (int v = 0; v < nk; ++v) mu[v] = 0;
    for (int r = 0; r < c; ++r) mu[it[r].v] = 1;
    int n = 0;
    for (int v = 0; v < nk; ++v)
      if (mu[v]) lu[n++] = v;
    for (int v = n; v < nk; ++v) lu[v] = -1;
    count[u] = c;
    if (cut_margin) cut_margin[u] = cm;
    if (gap_margin) gap_margin[u] = (c < nonempty && c > 0) ? it[c - 1].w - it[c].w : INFINITY;
    free(it);
  }
}

/* Block-sparse attention (section 3.1, E1/E2, with the renormalised reading): for every
 * query i of block u, over the keys J_u of the selected clusters
 *   s_ij = scale q_i . k_j,  O_i = sum_j exp(s_ij - m) v_j / sum_j exp(s_ij - m),
 *   lse_i = m + log sum_j exp(s_ij - m)        (m = max_j s_ij)
 * An empty selection gives O_i = 0 and lse_i = -inf.  Only the query blocks listed in
 * `ublocks` (n_ub of them; all blocks if NULL) are computed; O and lse are indexed by the
 * original query index and rows of other blocks are left untouched. */
ORC_EXPORT void orc_block_sparse_attn(const float* Q, const float* K, const float* V, long L, int d,
                                      const int* perm, const int* offsets, int nk, const int* list,
                                      const int* count, int qb, double scale, const long* ublocks,
                                      long n_ub, double* O, double* lse) {
  long nq = (L + qb - 1) / qb;
  long nu = ublocks ? n_ub : nq;
#pragma omp parallel for schedule(dynamic)
  for (long t = 0; t < nu; ++t) {
    long u = ublocks ? ublocks[t] : t;
    const int* lu = list + (size_t)u * nk;
    long nsel = 0;
    for (int r = 0; r < count[u]; ++r) nsel += offsets[lu[r] + 1] - offsets[lu[r]];
    long* J = (long*)malloc(sizeof(long) * (size_t)(nsel > 0 ? nsel : 1));
    long n = 0;
    for (int r = 0; r < count[u]; ++r)
      for (int p = offsets[lu[r]]; p < offsets[lu[r] + 1]; ++p) J[n++] = perm[p];
    double* s = (double*)malloc(sizeof(double) * (size_t)(nsel > 0 ? nsel : 1));
    long i0 = qblock_begin(u, qb), i1 = qblock_end(u, qb, L);
    for (long i = i0; i < i1; ++i) {
      double* Oi = O + (size_t)i * d;
      for (int a = 0; a < d; ++a) Oi[a] = 0.0;
      if (nsel == 0) {
        lse[i] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (long x = 0; x < nsel; ++x) {
        double dot = 0.0;
        for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)K[(size_t)J[x] * d + a];
        s[x] = scale * dot;
        if (s[x] > m) m = s[x];
      }
      double z = 0.0;
      for (long x = 0; x < nsel; ++x) {
        double e = exp(s[x] - m);
        z += e;
        for (int a = 0; a < d; ++a) Oi[a] += e * (double)V[(size_t)J[x] * d + a];
      }
      for (int a = 0; a < d; ++a) Oi[a] /= z;
      lse[i] = m + log(z);
    }
    free(s);
    free(J);
  }
}

/* ---------------------------------------------------------------------------------
 * Clustered query blocks (Figure 2 and section 6, "Implementations": the queries are
 * grouped by plain Euclidean k-means into N_Q = 128 query blocks).  Query block u holds
 * the queries qperm[qoffsets[u] .. qoffsets[u+1]), the permutation and offsets that the
 * k-means finalisation above writes when it clusters the queries; n_u = its size.
 * --------------------------------------------------------------------------------- */

/* PAMA over clustered query blocks, E7 and E8 as printed (the block sum runs over the
 * block's queries in qperm order):
 *   W_uv = (1/n_u) sum_{i in Q_u} P_iv,  P_iv = softmax_v(scale q_i . c_v + log n_v);
 * an empty query block gives a zero row. */
ORC_EXPORT void orc_pama_blocks(const float* Q, long L, int d, const float* cent, const int* counts, int nk,
                                const int* qperm, const int* qoffsets, long nq, double scale, double* W) {
  (void)L;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < nq; ++u) {
    double* S = (double*)malloc(sizeof(double) * (size_t)nk);
    double* Wu = W + (size_t)u * nk;
    for (int v = 0; v < nk; ++v) Wu[v] = 0.0;
    for (long pos = qoffsets[u]; pos < qoffsets[u + 1]; ++pos) {
      const float* q = Q + (size_t)qperm[pos] * d;
      double m = -INFINITY;
      for (int v = 0; v < nk; ++v) {
        if (counts[v] > 0) {
          double dot = 0.0;
          for (int a = 0; a < d; ++a) dot += (double)q[a] * (double)cent[(size_t)v * d + a];
          S[v] = scale * dot + log((double)counts[v]);
        } else {
          S[v] = -INFINITY;
        }
        if (S[v] > m) m = S[v];
      }
      double z = 0.0;
      for (int v = 0; v < nk; ++v) z += exp(S[v] - m);
      for (int v = 0; v < nk; ++v) Wu[v] += exp(S[v] - m) / z;
    }
    long n = qoffsets[u + 1] - qoffsets[u];
    if (n > 0)
      for (int v = 0; v < nk; ++v) Wu[v] /= (double)n;
    free(S);
  }
}

/* Block-sparse attention over clustered query blocks: for every query i of block u (the
 * queries qperm[qoffsets[u] .. qoffsets[u+1])), over the keys J_u of the clusters selected
 * for u, the renormalised softmax of section 3.1:
 *   s_ij = scale q_i . k_j,  O_i = sum_j exp(s_ij - m) v_j / sum_j exp(s_ij - m),
 *   lse_i = m + log sum_j exp(s_ij - m).
 * An empty selection gives O_i = 0 and lse_i = -inf.  Only the blocks in `ublocks` are
 * computed (all if NULL); O and lse are indexed by the original query index. */
ORC_EXPORT void orc_block_sparse_attn_blocks(const float* Q, const float* K, const float* V, long L, int d,
                                             const int* perm, const int* offsets, int nk, const int* qperm,
                                             const int* qoffsets, long nq, const int* list, const int* count,
                                             double scale, const long* ublocks, long n_ub, double* O,
                                             double* lse) {
  (void)L;
  long nu = ublocks ? n_ub : nq;
#pragma omp parallel for schedule(dynamic)
  for (long t = 0; t < nu; ++t) {
    long u = ublocks ? ublocks[t] : t;
    const int* lu = list + (size_t)u * nk;
    long nsel = 0;
    for (int r = 0; r < count[u]; ++r) nsel += offsets[lu[r] + 1] - offsets[lu[r]];
    long* J = (long*)malloc(sizeof(long) * (size_t)(nsel > 0 ? nsel : 1));
    long n = 0;
    for (int r = 0; r < count[u]; ++r)
      for (int p = offsets[lu[r]]; p < offsets[lu[r] + 1]; ++p) J[n++] = perm[p];
    double* s = (double*)malloc(sizeof(double) * (size_t)(nsel > 0 ? nsel : 1));
    for (long pos = qoffsets[u]; pos < qoffsets[u + 1]; ++pos) {
      long i = qperm[pos];
      double* Oi = O + (size_t)i * d;
      for (int a = 0; a < d; ++a) Oi[a] = 0.0;
      if (nsel == 0) {
        lse[i] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (long x = 0; x < nsel; ++x) {
        double dot = 0.0;
        for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)K[(size_t)J[x] * d + a];
        s[x] = scale * dot;
        if (s[x] > m) m = s[x];
      }
      double z = 0.0;
      for (long x = 0; x < nsel; ++x) {
        double e = exp(s[x] - m);
        z += e;
        for (int a = 0; a < d; ++a) Oi[a] += e * (double)V[(size_t)J[x] * d + a];
      }
      for (int a = 0; a < d; ++a) Oi[a] /= z;
      lse[i] = m + log(z);
    }
    free(s);
    free(J);
  }
}

/* M1 (Appendix A, "Attention-weight approximation error"): the total-variation distance of an
 * estimated block-importance map W^m from the exact one (Eq. (3)), weighted by the query-block
 * sizes:
 *   E_TV = sum_u (n_u / L) (1/2) sum_v |W^m_uv - W_uv|
 * (the printed formula lost its absolute-value bars; the TV distance is half the L1 distance). */
ORC_EXPORT double orc_tv(const double* West, const double* Wex, const long* nu, long nq, int nk, long L) {
  double e = 0.0;
  for (long u = 0; u < nq; ++u) {
    double t = 0.0;
    for (int v = 0; v < nk; ++v) t += fabs(West[(size_t)u * nk + v] - Wex[(size_t)u * nk + v]);
    e += (double)nu[u] / (double)L * 0.5 * t;
  }
  return e;
}

/* M2 (appendix B, "Centered log-mass approximation error"; section 4.2):
 *   S*_iv = log sum_{j in K_v} exp(scale q_i . k_j),   S_iv = log n_v + scale q_i . c_v,
 *   Delta_iv = S*_iv - S_iv over the non-empty blocks v, centred per query (minus its mean
 *   over v; the centring is not printed - a softmax over blocks ignores a per-query constant),
 *   RMSE = sqrt(mean over (i, v) of the centred Delta^2).
 * Queries `rows` (all if NULL).  Returns the RMSE. */
ORC_EXPORT double orc_logmass_rmse(const float* Q, const float* K, long L, int d, const int* labels,
                                   const float* cent, const int* counts, int nk, double scale,
                                   const long* rows, long nrows) {
  long nr = rows ? nrows : L;
  double ss = 0.0, np = 0.0;
#pragma omp parallel for schedule(dynamic) reduction(+ : ss, np)
  for (long r = 0; r < nr; ++r) {
    long i = rows ? rows[r] : r;
    double* mx = (double*)malloc(sizeof(double) * (size_t)nk);
    double* sm = (double*)malloc(sizeof(double) * (size_t)nk);
    double* dl = (double*)malloc(sizeof(double) * (size_t)nk);
    for (int v = 0; v < nk; ++v) { mx[v] = -INFINITY; sm[v] = 0.0; }
    for (long j = 0; j < L; ++j) {
      double dot = 0.0;
      for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)K[(size_t)j * d + a];
      double sc = scale * dot;
      int v = labels[j];
      if (sc > mx[v]) {
        sm[v] = sm[v] * exp(mx[v] - sc) + 1.0;
        mx[v] = sc;
      } else {
        sm[v] += exp(sc - mx[v]);
      }
    }
    double mean = 0.0;
    int n = 0;
    for (int v = 0; v < nk; ++v) {
      if (counts[v] <= 0) continue;
      double dot = 0.0;
      for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)cent[(size_t)v * d + a];
      dl[v] = (mx[v] + log(sm[v])) - (log((double)counts[v]) + scale * dot);
      mean += dl[v];
      ++n;
    }
    if (n > 0) {
      mean /= n;
      for (int v = 0; v < nk; ++v)
        if (counts[v] > 0) ss += (dl[v] - mean) * (dl[v] - mean);
      np += n;
    }
    free(mx); free(sm); free(dl);
  }
  return np > 0 ? sqrt(ss / np) : 0.0;
}

/* Dense attention (section 3.1, E1), textbook form, written independently of the sparse
 * routine above: A_i = softmax_j(scale q_i . k_j) over all L keys, O_i = sum_j A_ij v_j,
 * lse_i = log sum_j exp(scale q_i . k_j).  Rows listed in `rows` (all if NULL); outputs
 * are packed in the order of `rows`. */
ORC_EXPORT void orc_dense_attn(const float* Q, const float* K, const float* V, long L, int d,
                               double scale, const long* rows, long nrows, double* O, double* lse) {
  long nr = rows ? nrows : L;
#pragma omp parallel for schedule(dynamic)
  for (long r = 0; r < nr; ++r) {
    long i = rows ? rows[r] : r;
    double* logit = (double*)malloc(sizeof(double) * (size_t)L);
    double mx = -INFINITY;
    for (long j = 0; j < L; ++j) {
      double dot = 0.0;
      for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)K[(size_t)j * d + a];
      logit[j] = dot * scale;
      mx = logit[j] > mx ? logit[j] : mx;
    }
    double den = 0.0;
    for (long j = 0; j < L; ++j) den += exp(logit[j] - mx);
    for (int a = 0; a < d; ++a) {
      double num = 0.0;
      for (long j = 0; j < L; ++j) num += exp(logit[j] - mx) * (double)V[(size_t)j * d + a];
      O[(size_t)r * d + a] = num / den;
    }
    lse[r] = mx + log(den);
    free(logit);
  }
}

/* Exact block importance (section 3.2, Eq. (3)) from the dense attention matrix:
 *   W_uv = (1/n_u) sum_{i in Q_u} sum_{j in K_v} A_ij,  A = softmax(scale Q K^T).
 * Key blocks are given by labels[j] in [0, N_K).  Dense cost: tiny inputs only. */
ORC_EXPORT void orc_exact_block_importance(const float* Q, const float* K, long L, int d,
                                           const int* labels, int nk, int qb, double scale,
                                           double* W) {
  long nq = (L + qb - 1) / qb;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < nq; ++u) {
    double* A = (double*)malloc(sizeof(double) * (size_t)L);
    double* Wu = W + (size_t)u * nk;
    for (int v = 0; v < nk; ++v) Wu[v] = 0.0;
    long i0 = qblock_begin(u, qb), i1 = qblock_end(u, qb, L);
    for (long i = i0; i < i1; ++i) {
      double mx = -INFINITY;
      for (long j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int a = 0; a < d; ++a) dot += (double)Q[(size_t)i * d + a] * (double)K[(size_t)j * d + a];
        A[j] = dot * scale;
        if (A[j] > mx) mx = A[j];
      }
      double den = 0.0;
      for (long j = 0; j < L; ++j) den += exp(A[j] - mx);
      for (long j = 0; j < L; ++j) Wu[labels[j]] += exp(A[j] - mx) / den;
    }
    for (int v = 0; v < nk; ++v) Wu[v] /= (double)(i1 - i0);
    free(A);
  }
}
