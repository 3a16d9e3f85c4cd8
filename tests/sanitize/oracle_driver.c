/* Drives every oracle entry point on small ragged inputs, plus the argument
 * checks, so that a build of the oracle with AddressSanitizer and
 * UndefinedBehaviorSanitizer can watch each memory access (test
 * infrastructure: built and run by tests/test_sanitizers.py).  Exit status 0
 * when every call returns the expected code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
  int64_t B, T, H, G, d, dp, topk;
  double scale;
} msa_oracle_dims;

int msa_oracle_select(const msa_oracle_dims*, const double*, const double*, int64_t, const int64_t*, int32_t*,
                      float*);
int msa_oracle_fwd(const msa_oracle_dims*, const double*, const double*, const double*, const int32_t*, int64_t,
                   const int64_t*, double*, double*);
int msa_oracle_bwd_rows(const msa_oracle_dims*, const double*, const double*, const double*, const double*,
                        const int32_t*, int64_t, const int64_t*, double*);
int msa_oracle_bwd_blocks(const msa_oracle_dims*, const double*, const double*, const double*, const double*,
                          const int32_t*, int64_t, const int64_t*, double*, double*);
int msa_oracle_bwd(const msa_oracle_dims*, const double*, const double*, const double*, const double*,
                   const int32_t*, double*, double*, double*);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double unit(void) { /* xorshift64*, mapped to [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static double* fill(size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = unit();
  return p;
}

#define EXPECT(call, code)                                                  \
  do {                                                                      \
    const int rc_ = (call);                                                 \
    if (rc_ != (code)) {                                                    \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, rc_, (code)); \
      return 1;                                                             \
    }                                                                       \
  } while (0)

int main(void) {
  /* T = 300: two full blocks and a ragged third; topk 2 < 3 blocks */
  const msa_oracle_dims D = {2, 300, 4, 2, 16, 8, 2, 0.25};
  const int64_t N = (D.T + 127) / 128, BT = D.B * D.T;
  double* qp = fill((size_t)BT * D.G * D.dp);
  double* kp = fill((size_t)BT * D.G * D.dp);
  double* q = fill((size_t)BT * D.H * D.d);
  double* k = fill((size_t)BT * D.G * D.d);
  double* v = fill((size_t)BT * D.G * D.d);
  double* dout = fill((size_t)BT * D.H * D.d);
  int32_t* idx_rows = (int32_t*)malloc(sizeof(int32_t) * BT * D.G * D.topk);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * BT * D.G * D.topk);
  float* pooled = (float*)malloc(sizeof(float) * BT * D.G * N);
  double* o = (double*)malloc(sizeof(double) * BT * D.H * D.d);
  double* lse = (double*)malloc(sizeof(double) * BT * D.H);
  double* dq = (double*)malloc(sizeof(double) * BT * D.H * D.d);
  double* dk = (double*)malloc(sizeof(double) * BT * D.G * D.d);
  double* dv = (double*)malloc(sizeof(double) * BT * D.G * D.d);
  double* dkb = (double*)malloc(sizeof(double) * 3 * 128 * D.d);
  double* dvb = (double*)malloc(sizeof(double) * 3 * 128 * D.d);

  /* all rows, token-major output [B*T][G][topk] */
  EXPECT(msa_oracle_select(&D, qp, kp, BT, NULL, idx_rows, pooled), 0);
  for (int64_t r = 0; r < BT; ++r)
    for (int64_t g = 0; g < D.G; ++g)
      for (int64_t s = 0; s < D.topk; ++s)
        idx[(((r / D.T) * D.G + g) * D.T + r % D.T) * D.topk + s] = idx_rows[(r * D.G + g) * D.topk + s];
  const int64_t rows[4] = {0, 127, 299, 599};
  EXPECT(msa_oracle_select(&D, qp, kp, 4, rows, idx_rows, pooled), 0);
  EXPECT(msa_oracle_fwd(&D, q, k, v, idx, BT, NULL, o, lse), 0);
  EXPECT(msa_oracle_fwd(&D, q, k, v, idx, 4, rows, o, lse), 0);
  EXPECT(msa_oracle_bwd_rows(&D, q, k, v, dout, idx, 4, rows, dq), 0);
  const int64_t blocks[3] = {0, 2, 2 * D.G * N - 1};  /* first, ragged last of (b0, g0), last of all */
  EXPECT(msa_oracle_bwd_blocks(&D, q, k, v, dout, idx, 3, blocks, dkb, dvb), 0);
  EXPECT(msa_oracle_bwd(&D, q, k, v, dout, idx, dq, dk, dv), 0);
  for (int64_t i = 0; i < BT * D.H; ++i)
    if (!isfinite(lse[i])) {
      fprintf(stderr, "non-finite lse at %lld\n", (long long)i);
      return 1;
    }

  /* argument checks */
  msa_oracle_dims bad = D;
  bad.H = 3; /* not a multiple of G */
  EXPECT(msa_oracle_fwd(&bad, q, k, v, idx, BT, NULL, o, lse), 1);
  EXPECT(msa_oracle_select(&D, NULL, kp, BT, NULL, idx_rows, pooled), 1);
  const int64_t out_of_range[1] = {BT};
  EXPECT(msa_oracle_fwd(&D, q, k, v, idx, 1, out_of_range, o, lse), 4);
  const int64_t bad_block[1] = {2 * D.G * N};
  EXPECT(msa_oracle_bwd_blocks(&D, q, k, v, dout, idx, 1, bad_block, dkb, dvb), 4);
  idx[5 * D.topk] = 2; /* row t = 5 of (b0, g0) names a future block */
  EXPECT(msa_oracle_fwd(&D, q, k, v, idx, BT, NULL, o, lse), 2);

  free(qp); free(kp); free(q); free(k); free(v); free(dout); free(idx_rows); free(idx); free(pooled);
  free(o); free(lse); free(dq); free(dk); free(dv); free(dkb); free(dvb);
  puts("oracle driver ok");
  return 0;
}
