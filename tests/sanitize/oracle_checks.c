/* Runs every entry point of oracle/oracle.c on small inputs (segments,
 * positions, row subsets, key-column windows, ring order, odd sizes) so that
 * the oracle can be built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer and checked for out-of-bounds accesses, leaks and undefined
 * arithmetic.  Also checks that the blocked forward equals the plain one.
 * Prints "oracle checks ok" and exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_rope(int B, int H, int S, int D, const double* x, const int32_t* pos, double theta, int inverse,
                double* y);
int oracle_attn_fwd(int B, int H, int S, int D, const double* q, const double* k, const double* v,
                    const int32_t* seg, const int32_t* pos, double theta, double scale, int causal,
                    const int64_t* rows, int64_t n_rows, double* o, double* lse);
int oracle_attn_fwd_blocked(int B, int H, int S, int D, const double* q, const double* k, const double* v,
                            const int32_t* seg, const int32_t* pos, double theta, double scale, int causal,
                            int block_k, int kv_chunk, double* o, double* lse);
int oracle_attn_bwd(int B, int H, int S, int D, const double* q, const double* k, const double* v,
                    const double* dout, const int32_t* seg, const int32_t* pos, double theta, double scale,
                    int causal, const int64_t* rows, int64_t n_rows, int col_begin, int col_end, double* dq,
                    double* dk, double* dv);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double* fill(size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = uniform();
  return p;
}

static int run_case(int B, int H, int S, int D, int packed, int causal, double theta, int kv_chunk) {
  const size_t n = (size_t)B * H * S * D;
  double *q = fill(n), *k = fill(n), *v = fill(n), *d = fill(n);
  int32_t* seg = NULL;
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * S);
  if (packed) seg = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * S);
  for (int b = 0; b < B; ++b) {
    int doc = 0, start = 0;
    for (int s = 0; s < S; ++s) {
      if (packed && s > 0 && (s * 7 + b) % 23 == 0) { ++doc; start = s; }
      if (seg) seg[b * S + s] = doc;
      pos[b * S + s] = packed ? s - start : s;
    }
  }
  /* outputs sized for max(S, 3) rows: the row-subset calls below list 3 rows */
  const size_t rows_max = (size_t)(S > 3 ? S : 3), no = (size_t)B * H * rows_max * D;
  double *o = calloc(no, sizeof(double)), *o2 = calloc(n, sizeof(double)), *y = calloc(n, sizeof(double));
  double *lse = calloc((size_t)B * H * rows_max, sizeof(double)), *lse2 = calloc((size_t)B * H * S, sizeof(double));
  double *dq = calloc(no, sizeof(double)), *dk = calloc(n, sizeof(double)), *dv = calloc(n, sizeof(double));
  int rc = 0;
  rc |= oracle_rope(B, H, S, D, q, pos, theta > 0 ? theta : 1e4, 0, y);
  rc |= oracle_rope(B, H, S, D, y, pos, theta > 0 ? theta : 1e4, 1, y);
  rc |= oracle_attn_fwd(B, H, S, D, q, k, v, seg, pos, theta, 0.0, causal, NULL, 0, o, lse);
  rc |= oracle_attn_fwd_blocked(B, H, S, D, q, k, v, seg, pos, theta, 0.0, causal, 3, kv_chunk, o2, lse2);
  double worst = 0.0;
  for (size_t i = 0; i < n; ++i) worst = fmax(worst, fabs(o[i] - o2[i]));
  for (size_t i = 0; i < (size_t)B * H * S; ++i) worst = fmax(worst, fabs(lse[i] - lse2[i]));
  if (worst > 1e-12) { fprintf(stderr, "blocked forward differs by %g\n", worst); rc |= 1; }
  /* a subset of rows, and a window of key columns */
  int64_t rows[3] = {0, S / 2, S - 1};
  rc |= oracle_attn_fwd(B, H, S, D, q, k, v, seg, pos, theta, 0.3, causal, rows, 3, o, lse);
  rc |= oracle_attn_bwd(B, H, S, D, q, k, v, d, seg, pos, theta, 0.0, causal, NULL, 0, 0, S, dq, dk, dv);
  rc |= oracle_attn_bwd(B, H, S, D, q, k, v, d, seg, pos, theta, 0.0, causal, rows, 3, S / 3, S, dq, dk, dv);
  /* argument errors are refused */
  if (oracle_attn_bwd(B, H, S, D, q, k, v, d, seg, pos, theta, 0.0, causal, NULL, 0, 2, 1, dq, dk, dv) == 0) rc |= 1;
  if (oracle_attn_fwd(B, H, S, 3, q, k, v, seg, pos, theta, 0.0, causal, NULL, 0, o, lse) == 0) rc |= 1;
  free(q); free(k); free(v); free(d); free(seg); free(pos); free(o); free(o2); free(y);
  free(lse); free(lse2); free(dq); free(dk); free(dv);
  return rc;
}

int main(void) {
  int rc = 0;
  rc |= run_case(1, 2, 97, 16, 0, 1, 1e6, 0);
  rc |= run_case(2, 1, 130, 8, 1, 1, 5e7, 32);
  rc |= run_case(1, 1, 64, 6, 1, 0, 0.0, 0);
  rc |= run_case(1, 1, 1, 4, 0, 1, 1e4, 0);
  if (rc) {
    fprintf(stderr, "oracle checks failed\n");
    return 1;
  }
  printf("oracle checks ok\n");
  return 0;
}
