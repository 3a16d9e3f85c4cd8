/*
 * CPU oracle for the MiniMax Sparse Attention (MSA) training hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP implementation, and the product path
 * never calls it.
 *
 * It is the plain definition of what the hot path computes, written as slow,
 * obviously correct loops:
 *
 *   Index Branch  (msa_oracle_select)
 *     One proxy head per KV group scores every query against every causal key;
 *     the scores are max-pooled over 128-key blocks and the top-k blocks of each
 *     query are kept as its block-index cache.  Sources: page "Flash-MSA:
 *     Open-Source Sparse Attention Kernels Debut", section "How MSA works"
 *     (128-key blocks chosen by max-pooling proxy scores; indices cached; one
 *     proxy head per group of heads) and page "flash-msa-sparse-attention-
 *     training" (ai-beat.github.io), paragraphs 1, 3 and 4 (Index Branch picks
 *     the KV blocks each query reads; 128-token blocks; group-specialised proxy
 *     heads).
 *
 *   Main Branch   (msa_oracle_fwd, msa_oracle_bwd*)
 *     Exact softmax GQA attention restricted to the keys of the cached blocks,
 *     and its gradients with respect to Q, K and V.  Sources: ai-beat page,
 *     paragraph 1 (exact softmax attention over only the selected blocks) and
 *     paragraph 2 (training needs a backward pass through the sparse pattern);
 *     xcelit page, section "How MSA works" (GQA main attention).
 *
 * Precision.  Main-branch arithmetic is IEEE fp64 throughout.  The Index
 * Branch takes its integer decision in fp32, the precision of the kernel that
 * produces the scores: each proxy dot product is accumulated in fp64 (exact for
 * bf16 inputs of the sizes used here) and rounded once to fp32; the block score
 * is the maximum of those fp32 values.
 *
 * Readings of points the pages leave open (each also listed with the design
 * notes of the project):
 *   - proxy score = plain dot product q_p . k_p, no scale or activation;
 *   - head h belongs to KV/proxy group g = h / (H/G);
 *   - candidates for query t are blocks 0..floor(t/128); inside a block only
 *     keys j <= t count, both for pooling and for attention;
 *   - the diagonal block is an ordinary candidate (not forced);
 *   - ties in the pooled score go to the lower block index; -0.0 counts as +0.0;
 *   - a NaN proxy score never wins a max (it is skipped);
 *   - the cache row lists the selected blocks in ascending order, padded with
 *     -1 up to topk; when topk >= number of causal blocks all are selected;
 *   - softmax scale is a parameter (the ABI default is 1/sqrt(d));
 *   - LSE is the natural-log log-sum-exp of the scaled scores;
 *   - D = dO . O uses the exact (fp64) O.
 *
 * Parity pins: tests/test_oracle_*.py check every function here against
 * dense masked attention, PyTorch's causal scaled-dot-product attention and
 * autograd, finite differences, closed forms and planted selections.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BLOCK 128

typedef struct {
  int64_t B, T, H, G, d, dp, topk;
  double scale;
} msa_oracle_dims;

enum { OR_OK = 0, OR_ERR_DIMS = 1, OR_ERR_INDEX = 2, OR_ERR_ALLOC = 3, OR_ERR_ROW = 4 };

static int dims_ok(const msa_oracle_dims* D, int need_main, int need_proxy) {
  if (!D || D->B < 1 || D->T < 1 || D->G < 1 || D->topk < 1) return 0;
  if (need_main && (D->H < 1 || D->H % D->G != 0 || D->d < 1)) return 0;
  if (need_proxy && D->dp < 1) return 0;
  return 1;
}

static int64_t n_blocks(const msa_oracle_dims* D) { return (D->T + OR_BLOCK - 1) / OR_BLOCK; }

int msa_oracle_max_threads(void) { return omp_get_max_threads(); }
void msa_oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* ------------------------------------------------------------------------ */
/* Index Branch                                                             */
/* ------------------------------------------------------------------------ */

/* Proxy score of query (b,t) against key (b,j) in group g, taken to fp32. */
static float proxy_score(const msa_oracle_dims* D, const double* qp, const double* kp,
                         int64_t b, int64_t t, int64_t j, int64_t g) {
  const double* x = qp + ((b * D->T + t) * D->G + g) * D->dp;
  const double* y = kp + ((b * D->T + j) * D->G + g) * D->dp;
  double s = 0.0;
  for (int64_t c = 0; c < D->dp; ++c) s += x[c] * y[c];
  return (float)s;
}

/* Does block a (score sa) rank before block b (score sb)?  Higher score first,
 * lower index on equal scores. */
static int ranks_before(float sa, int64_t a, float sb, int64_t b) {
  if (sa > sb) return 1;
  if (sa < sb) return 0;
  return a < b;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * For each listed token row (rows[r] = b*T + t; rows == NULL means every token
 * in order) and each group g:
 *   pooled[i] = max_{128 i <= j <= min(128 i + 127, t)} score(t, j),  i <= t/128
 *   the min(topk, t/128 + 1) blocks first in (score desc, index asc) order are
 *   written ascending to idx_out[r][g][0..), the rest of the row is -1.
 * idx_out: [n_rows][G][topk];  pooled_out (optional): [n_rows][G][ceil(T/128)]
 * with -inf past the causal blocks.
 */
int msa_oracle_select(const msa_oracle_dims* D, const double* qp, const double* kp,
                      int64_t n_rows, const int64_t* rows, int32_t* idx_out, float* pooled_out) {
  if (!dims_ok(D, 0, 1) || !qp || !kp || !idx_out || n_rows < 0) return OR_ERR_DIMS;
  const int64_t N = n_blocks(D), K = D->topk;
  int err = OR_OK;
#pragma omp parallel
  {
    float* pooled = (float*)malloc(sizeof(float) * (size_t)N);
    float* best_s = (float*)malloc(sizeof(float) * (size_t)(K + 1));
    int32_t* best_i = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
    if (!pooled || !best_s || !best_i) {
#pragma omp atomic write
      err = OR_ERR_ALLOC;
    }
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; ++r) {
      for (int64_t g = 0; g < D->G; ++g) {
        if (err != OR_OK) continue;
        const int64_t row = rows ? rows[r] : r;
        if (row < 0 || row >= D->B * D->T) {
#pragma omp atomic write
          err = OR_ERR_ROW;
          continue;
        }
        const int64_t b = row / D->T, t = row % D->T;
        const int64_t nc = t / OR_BLOCK + 1;
        for (int64_t i = 0; i < nc; ++i) {
          float m = -INFINITY;
          const int64_t j1 = (i + 1) * OR_BLOCK - 1 < t ? (i + 1) * OR_BLOCK - 1 : t;
          for (int64_t j = i * OR_BLOCK; j <= j1; ++j) {
            float s = proxy_score(D, qp, kp, b, t, j, g);
            if (s > m) m = s;           /* NaN never wins */
          }
          if (m == 0.0f) m = 0.0f;      /* -0.0 -> +0.0 */
          pooled[i] = m;
        }
        if (pooled_out) {
          float* po = pooled_out + (r * D->G + g) * N;
          for (int64_t i = 0; i < N; ++i) po[i] = i < nc ? pooled[i] : -INFINITY;
        }
        /* Keep the best n_sel blocks in a list ordered by rank (insertion). */
        const int64_t n_sel = K < nc ? K : nc;
        int64_t cnt = 0;
        for (int64_t i = 0; i < nc; ++i) {
          if (cnt == n_sel && !ranks_before(pooled[i], i, best_s[cnt - 1], best_i[cnt - 1])) continue;
          int64_t p = cnt < n_sel ? cnt : n_sel - 1;
          while (p > 0 && ranks_before(pooled[i], i, best_s[p - 1], best_i[p - 1])) {
            best_s[p] = best_s[p - 1];
            best_i[p] = best_i[p - 1];
            --p;
          }
          best_s[p] = pooled[i];
          best_i[p] = (int32_t)i;
          if (cnt < n_sel) ++cnt;
        }
        int32_t* out = idx_out + (r * D->G + g) * K;
        for (int64_t s = 0; s < K; ++s) out[s] = s < cnt ? best_i[s] : -1;
        qsort(out, (size_t)cnt, sizeof(int32_t), cmp_i32);
      }
    }
    free(pooled);
    free(best_s);
    free(best_i);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Main Branch                                                              */
/* ------------------------------------------------------------------------ */

/* Keys attended by query (b,t) in group g: every j <= t whose block is listed in
 * the cache row idx[b][g][t][:].  Negative entries are unused slots.  Returns
 * the number of keys, or -1 if the row names a block that is out of range,
 * non-causal or repeated. */
static int64_t row_keys(const msa_oracle_dims* D, const int32_t* idx, int64_t b, int64_t g,
                        int64_t t, int64_t* J) {
  const int32_t* row = idx + ((b * D->G + g) * D->T + t) * D->topk;
  const int64_t last = t / OR_BLOCK;
  int64_t n = 0;
  for (int64_t s = 0; s < D->topk; ++s) {
    const int64_t blk = row[s];
    if (blk < 0) continue;
    if (blk > last) return -1;
    for (int64_t u = 0; u < s; ++u)
      if (row[u] == blk) return -1;
    const int64_t j1 = (blk + 1) * OR_BLOCK - 1 < t ? (blk + 1) * OR_BLOCK - 1 : t;
    for (int64_t j = blk * OR_BLOCK; j <= j1; ++j) J[n++] = j;
  }
  return n;
}

static const double* qrow(const msa_oracle_dims* D, const double* q, int64_t b, int64_t t, int64_t h) {
  return q + ((b * D->T + t) * D->H + h) * D->d;
}
static const double* krow(const msa_oracle_dims* D, const double* k, int64_t b, int64_t j, int64_t g) {
  return k + ((b * D->T + j) * D->G + g) * D->d;
}
static double dot(const double* x, const double* y, int64_t n) {
  double s = 0.0;
  for (int64_t c = 0; c < n; ++c) s += x[c] * y[c];
  return s;
}

/* Softmax attention of one query row over the key list J:
 *   s_j = scale * q . k_j,  m = max s_j,  l = sum exp(s_j - m)
 *   p_j = exp(s_j - m) / l,  o = sum p_j v_j,  lse = m + ln l.
 * p (length nJ) and o (length d) are outputs; returns lse. */
static double row_attention(const msa_oracle_dims* D, const double* q, const double* k,
                            const double* v, int64_t b, int64_t t, int64_t h,
                            const int64_t* J, int64_t nJ, double* p, double* o) {
  const int64_t g = h / (D->H / D->G);
  const double* qr = qrow(D, q, b, t, h);
  double m = -INFINITY;
  for (int64_t n = 0; n < nJ; ++n) {
    p[n] = D->scale * dot(qr, krow(D, k, b, J[n], g), D->d);
    if (p[n] > m) m = p[n];
  }
  double l = 0.0;
  for (int64_t n = 0; n < nJ; ++n) {
    p[n] = exp(p[n] - m);
    l += p[n];
  }
  for (int64_t c = 0; c < D->d; ++c) o[c] = 0.0;
  for (int64_t n = 0; n < nJ; ++n) {
    p[n] /= l;
    const double* vr = krow(D, v, b, J[n], g);
    for (int64_t c = 0; c < D->d; ++c) o[c] += p[n] * vr[c];
  }
  return m + log(l);
}

/*
 * Forward of the Main Branch for the listed token rows (rows == NULL: all).
 * o_out: [n_rows][H][d], lse_out: [n_rows][H].  idx: [B][G][T][topk].
 */
int msa_oracle_fwd(const msa_oracle_dims* D, const double* q, const double* k, const double* v,
                   const int32_t* idx, int64_t n_rows, const int64_t* rows, double* o_out,
                   double* lse_out) {
  if (!dims_ok(D, 1, 0) || !q || !k || !v || !idx || !o_out || !lse_out || n_rows < 0) return OR_ERR_DIMS;
  const int64_t maxJ = D->topk * OR_BLOCK;
  int err = OR_OK;
#pragma omp parallel
  {
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxJ);
    double* p = (double*)malloc(sizeof(double) * (size_t)maxJ);
    if (!J || !p) {
#pragma omp atomic write
      err = OR_ERR_ALLOC;
    }
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; ++r) {
      for (int64_t h = 0; h < D->H; ++h) {
        if (err != OR_OK) continue;
        const int64_t row = rows ? rows[r] : r;
        if (row < 0 || row >= D->B * D->T) {
#pragma omp atomic write
          err = OR_ERR_ROW;
          continue;
        }
        const int64_t b = row / D->T, t = row % D->T, g = h / (D->H / D->G);
        const int64_t nJ = row_keys(D, idx, b, g, t, J);
        if (nJ < 0) {
#pragma omp atomic write
          err = OR_ERR_INDEX;
          continue;
        }
        double* o = o_out + (r * D->H + h) * D->d;
        if (nJ == 0) { /* empty row: no keys, defined as O = 0, LSE = -inf */
          for (int64_t c = 0; c < D->d; ++c) o[c] = 0.0;
          lse_out[r * D->H + h] = -INFINITY;
          continue;
        }
        lse_out[r * D->H + h] = row_attention(D, q, k, v, b, t, h, J, nJ, p, o);
      }
    }
    free(J);
    free(p);
  }
  return err;
}

/* Backward quantities of one query row (b,t,h) over its key list J:
 *   P_j = softmax weights, O = sum P_j v_j, Dd = dO . O,
 *   dP_j = dO . v_j,  dS_j = P_j (dP_j - Dd).
 * Writes dS into ds[0..nJ). */
static void row_dscores(const msa_oracle_dims* D, const double* q, const double* k,
                        const double* v, const double* dout, int64_t b, int64_t t, int64_t h,
                        const int64_t* J, int64_t nJ, double* p, double* o, double* ds) {
  const int64_t g = h / (D->H / D->G);
  row_attention(D, q, k, v, b, t, h, J, nJ, p, o);
  const double* dor = qrow(D, dout, b, t, h);
  const double Dd = dot(dor, o, D->d);
  for (int64_t n = 0; n < nJ; ++n) {
    const double dP = dot(dor, krow(D, v, b, J[n], g), D->d);
    ds[n] = p[n] * (dP - Dd);
  }
}

/*
 * dQ rows of the Main Branch backward for the listed tokens (rows == NULL: all):
 *   dQ[t,h] = scale * sum_j dS_j k_j.     dq_out: [n_rows][H][d]
 * The loss is L = sum O * dO, so dO is the incoming gradient.
 */
int msa_oracle_bwd_rows(const msa_oracle_dims* D, const double* q, const double* k, const double* v,
                        const double* dout, const int32_t* idx, int64_t n_rows, const int64_t* rows,
                        double* dq_out) {
  if (!dims_ok(D, 1, 0) || !q || !k || !v || !dout || !idx || !dq_out || n_rows < 0) return OR_ERR_DIMS;
  const int64_t maxJ = D->topk * OR_BLOCK;
  int err = OR_OK;
#pragma omp parallel
  {
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxJ);
    double* p = (double*)malloc(sizeof(double) * (size_t)maxJ);
    double* ds = (double*)malloc(sizeof(double) * (size_t)maxJ);
    double* o = (double*)malloc(sizeof(double) * (size_t)D->d);
    if (!J || !p || !ds || !o) {
#pragma omp atomic write
      err = OR_ERR_ALLOC;
    }
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; ++r) {
      for (int64_t h = 0; h < D->H; ++h) {
        if (err != OR_OK) continue;
        const int64_t row = rows ? rows[r] : r;
        if (row < 0 || row >= D->B * D->T) {
#pragma omp atomic write
          err = OR_ERR_ROW;
          continue;
        }
        const int64_t b = row / D->T, t = row % D->T, g = h / (D->H / D->G);
        const int64_t nJ = row_keys(D, idx, b, g, t, J);
        if (nJ < 0) {
#pragma omp atomic write
          err = OR_ERR_INDEX;
          continue;
        }
        double* dq = dq_out + (r * D->H + h) * D->d;
        for (int64_t c = 0; c < D->d; ++c) dq[c] = 0.0;
        if (nJ == 0) continue;
        row_dscores(D, q, k, v, dout, b, t, h, J, nJ, p, o, ds);
        for (int64_t n = 0; n < nJ; ++n) {
          const double* kr = krow(D, k, b, J[n], g);
          for (int64_t c = 0; c < D->d; ++c) dq[c] += D->scale * ds[n] * kr[c];
        }
      }
    }
    free(J);
    free(p);
    free(ds);
    free(o);
  }
  return err;
}

/*
 * dK and dV of the listed key blocks (blocks[i] = (b*G + g)*N + blk):
 *   dK[j] = scale * sum_{t,h in g : j in J(t)} dS_{t,h,j} q[t,h]
 *   dV[j] =         sum_{t,h in g : j in J(t)} P_{t,h,j} dO[t,h]
 * for the 128 keys j of each block (rows past T stay zero).
 * dk_out, dv_out: [n_blocks][128][d].  Each contributing query row is
 * recomputed in full, so the cost grows with the number of tokens that
 * selected the block.
 */
int msa_oracle_bwd_blocks(const msa_oracle_dims* D, const double* q, const double* k,
                          const double* v, const double* dout, const int32_t* idx,
                          int64_t n_blk, const int64_t* blocks, double* dk_out, double* dv_out) {
  if (!dims_ok(D, 1, 0) || !q || !k || !v || !dout || !idx || !blocks || !dk_out || !dv_out || n_blk < 0)
    return OR_ERR_DIMS;
  const int64_t N = n_blocks(D), maxJ = D->topk * OR_BLOCK, R = D->H / D->G, d = D->d;
  const size_t blk_elems = (size_t)OR_BLOCK * (size_t)d;
  memset(dk_out, 0, sizeof(double) * blk_elems * (size_t)n_blk);
  memset(dv_out, 0, sizeof(double) * blk_elems * (size_t)n_blk);
  int err = OR_OK;
  for (int64_t ib = 0; ib < n_blk && err == OR_OK; ++ib) {
    const int64_t bg = blocks[ib] / N, blk = blocks[ib] % N;
    if (blocks[ib] < 0 || bg >= D->B * D->G) return OR_ERR_ROW;
    const int64_t b = bg / D->G, g = bg % D->G;
    double* dk_blk = dk_out + (size_t)ib * blk_elems;
    double* dv_blk = dv_out + (size_t)ib * blk_elems;
#pragma omp parallel
    {
      int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxJ);
      double* p = (double*)malloc(sizeof(double) * (size_t)maxJ);
      double* ds = (double*)malloc(sizeof(double) * (size_t)maxJ);
      double* o = (double*)malloc(sizeof(double) * (size_t)d);
      double* dk_loc = (double*)calloc(blk_elems, sizeof(double));
      double* dv_loc = (double*)calloc(blk_elems, sizeof(double));
      if (!J || !p || !ds || !o || !dk_loc || !dv_loc) {
#pragma omp atomic write
        err = OR_ERR_ALLOC;
      }
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = blk * OR_BLOCK; t < D->T; ++t) {
        if (err != OR_OK) continue;
        const int32_t* row = idx + ((b * D->G + g) * D->T + t) * D->topk;
        int sel = 0;
        for (int64_t s = 0; s < D->topk; ++s) sel |= (row[s] == blk);
        if (!sel) continue;
        const int64_t nJ = row_keys(D, idx, b, g, t, J);
        if (nJ < 0) {
#pragma omp atomic write
          err = OR_ERR_INDEX;
          continue;
        }
        for (int64_t h = g * R; h < (g + 1) * R; ++h) {
          row_dscores(D, q, k, v, dout, b, t, h, J, nJ, p, o, ds);
          const double* qr = qrow(D, q, b, t, h);
          const double* dor = qrow(D, dout, b, t, h);
          for (int64_t n = 0; n < nJ; ++n) {
            if (J[n] / OR_BLOCK != blk) continue;
            const int64_t jj = J[n] - blk * OR_BLOCK;
            for (int64_t c = 0; c < d; ++c) {
              dk_loc[jj * d + c] += D->scale * ds[n] * qr[c];
              dv_loc[jj * d + c] += p[n] * dor[c];
            }
          }
        }
      }
#pragma omp critical
      {
        if (dk_loc && dv_loc)
          for (size_t e = 0; e < blk_elems; ++e) {
            dk_blk[e] += dk_loc[e];
            dv_blk[e] += dv_loc[e];
          }
      }
      free(J);
      free(p);
      free(ds);
      free(o);
      free(dk_loc);
      free(dv_loc);
    }
  }
  return err;
}

/*
 * Full Main Branch backward: dq [B][T][H][d], dk and dv [B][T][G][d].
 * dQ rows come from msa_oracle_bwd_rows; dK/dV accumulate every query row's
 * contribution into per-thread copies that are summed at the end.
 */
int msa_oracle_bwd(const msa_oracle_dims* D, const double* q, const double* k, const double* v,
                   const double* dout, const int32_t* idx, double* dq, double* dk, double* dv) {
  if (!dims_ok(D, 1, 0) || !q || !k || !v || !dout || !idx || !dq || !dk || !dv) return OR_ERR_DIMS;
  int err = msa_oracle_bwd_rows(D, q, k, v, dout, idx, D->B * D->T, NULL, dq);
  if (err != OR_OK) return err;
  const int64_t maxJ = D->topk * OR_BLOCK, R = D->H / D->G, d = D->d;
  const size_t kv_elems = (size_t)(D->B * D->T * D->G * d);
  memset(dk, 0, sizeof(double) * kv_elems);
  memset(dv, 0, sizeof(double) * kv_elems);
#pragma omp parallel
  {
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxJ);
    double* p = (double*)malloc(sizeof(double) * (size_t)maxJ);
    double* ds = (double*)malloc(sizeof(double) * (size_t)maxJ);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    double* dk_loc = (double*)calloc(kv_elems, sizeof(double));
    double* dv_loc = (double*)calloc(kv_elems, sizeof(double));
    if (!J || !p || !ds || !o || !dk_loc || !dv_loc) {
#pragma omp atomic write
      err = OR_ERR_ALLOC;
    }
#pragma omp for schedule(dynamic, 4) collapse(2)
    for (int64_t bt = 0; bt < D->B * D->T; ++bt) {
      for (int64_t h = 0; h < D->H; ++h) {
        if (err != OR_OK) continue;
        const int64_t b = bt / D->T, t = bt % D->T, g = h / R;
        const int64_t nJ = row_keys(D, idx, b, g, t, J);
        if (nJ < 0) {
#pragma omp atomic write
          err = OR_ERR_INDEX;
          continue;
        }
        if (nJ == 0) continue;
        row_dscores(D, q, k, v, dout, b, t, h, J, nJ, p, o, ds);
        const double* qr = qrow(D, q, b, t, h);
        const double* dor = qrow(D, dout, b, t, h);
        for (int64_t n = 0; n < nJ; ++n) {
          double* dkr = dk_loc + ((b * D->T + J[n]) * D->G + g) * d;
          double* dvr = dv_loc + ((b * D->T + J[n]) * D->G + g) * d;
          for (int64_t c = 0; c < d; ++c) {
            dkr[c] += D->scale * ds[n] * qr[c];
            dvr[c] += p[n] * dor[c];
          }
        }
      }
    }
#pragma omp critical
    {
      if (dk_loc && dv_loc)
        for (size_t e = 0; e < kv_elems; ++e) {
          dk[e] += dk_loc[e];
          dv[e] += dv_loc[e];
        }
    }
    free(J);
    free(p);
    free(ds);
    free(o);
    free(dk_loc);
    free(dv_loc);
  }
  return err;
}
