/*
 * Oracle for blockwise causal attention with RoPE and a packing mask.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain CPU definition that
 * the GPU library is checked against.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Everything is double precision.  The caller passes the values the GPU sees
 * (bf16 inputs widened exactly to double).
 *
 * What is computed, and where the pages fix it (arXiv 2402.08268, "World Model
 * on Million-Length Video And Language With Blockwise RingAttention"; the
 * zhao9797 page "LWM (Large World Model)", sections 模型架构 / 训练方法 / 数据):
 *
 *  - Exact softmax attention: the blockwise ring method of the paper is stated
 *    to work "without approximation" (elamur.ai summary page, Summary), so
 *    the oracle is the plain definition, not the blockwise algorithm.
 *  - Causal mask: the model is a decoder-only autoregressive transformer
 *    (zhao9797 page, 模型架构), so query i sees keys j <= i (sequence index).
 *  - Packing mask: under masked sequence packing each packed example attends
 *    only to itself (zhao9797 page, 训练方法, "Masked Sequence Packing"), so a
 *    key is visible only when its segment id equals the query's.
 *  - RoPE: "standard RoPE" with a context-scaled base theta (zhao9797 page,
 *    模型架构 and the Stage I table in 训练方法).  Read as RoFormer's rotation
 *    of adjacent pairs (x[2i], x[2i+1]) by angle pos * theta^(-2i/D).
 *  - Softmax scale: not stated on the pages; taken as 1/sqrt(D) unless the
 *    caller passes another value.
 *  - Backward: the exact gradient of the forward (training needs gradient
 *    steps, zhao9797 page 训练方法).
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* RoPE.  For pair index i in [0, D/2): w_i = theta^(-2i/D), a = pos * w_i,  */
/*   y[2i]   = x[2i] cos a - x[2i+1] sin a                                    */
/*   y[2i+1] = x[2i] sin a + x[2i+1] cos a                                    */
/* inverse != 0 rotates by -a (the transpose, since the rotation is           */
/* orthogonal).  x, y: [B,H,S,D]; pos: [B,S] (NULL means pos = s).            */
/* ------------------------------------------------------------------------ */
static void rotate_row(const double* x, double* y, int D, double pos, double theta, int inverse) {
  for (int i = 0; i < D / 2; ++i) {
    double w = pow(theta, -2.0 * (double)i / (double)D);
    double a = pos * w;
    if (inverse) a = -a;
    double c = cos(a), s = sin(a);
    double x0 = x[2 * i], x1 = x[2 * i + 1];
    y[2 * i] = x0 * c - x1 * s;
    y[2 * i + 1] = x0 * s + x1 * c;
  }
}

static double position_of(const int32_t* pos, int S, int b, int s) {
  return pos ? (double)pos[(int64_t)b * S + s] : (double)s;
}

int oracle_rope(int B, int H, int S, int D, const double* x, const int32_t* pos, double theta,
                int inverse, double* y) {
  if (B < 0 || H < 0 || S < 0 || D <= 0 || (D & 1)) return 1;
  int64_t n = (int64_t)B * H * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    int s = (int)(r % S);
    int b = (int)(r / ((int64_t)H * S));
    rotate_row(x + r * D, y + r * D, D, position_of(pos, S, b, s), theta, inverse);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention helpers                                                          */
/* ------------------------------------------------------------------------ */

/* M_ij: key j is visible to query i. */
static int visible(const int32_t* seg_b, int causal, int i, int j) {
  if (causal && j > i) return 0;
  if (seg_b && seg_b[i] != seg_b[j]) return 0;
  return 1;
}

static double dot(const double* a, const double* b, int D) {
  double acc = 0.0;
  for (int d = 0; d < D; ++d) acc += a[d] * b[d];
  return acc;
}

/* Rotate all S rows of one (b,h) slice; theta <= 0 means no RoPE. */
static void rotate_slice(const double* x, double* y, int S, int D, const int32_t* pos, int b,
                         double theta) {
  for (int s = 0; s < S; ++s) {
    if (theta > 0.0)
      rotate_row(x + (int64_t)s * D, y + (int64_t)s * D, D, position_of(pos, S, b, s), theta, 0);
    else
      memcpy(y + (int64_t)s * D, x + (int64_t)s * D, sizeof(double) * D);
  }
}

/* Forward of one query row i against rotated keys kr (S x D) and values v.
 * qr: the rotated query row.  Writes o_row (D) and returns the natural-log
 * LSE.  p (length S) receives P_ij for visible j and 0 elsewhere. */
static double row_forward(const double* qr, const double* kr, const double* v, const int32_t* seg_b,
                          int causal, int S, int D, double scale, int i, double* p, double* o_row) {
  double mu = -INFINITY;
  for (int j = 0; j < S; ++j) {
    if (visible(seg_b, causal, i, j)) {
      p[j] = scale * dot(qr, kr + (int64_t)j * D, D);
      if (p[j] > mu) mu = p[j];
    } else {
      p[j] = 0.0;
    }
  }
  double z = 0.0;
  for (int j = 0; j < S; ++j)
    if (visible(seg_b, causal, i, j)) z += exp(p[j] - mu);
  for (int j = 0; j < S; ++j) p[j] = visible(seg_b, causal, i, j) ? exp(p[j] - mu) / z : 0.0;
  for (int d = 0; d < D; ++d) o_row[d] = 0.0;
  for (int j = 0; j < S; ++j) {
    if (p[j] == 0.0) continue;
    const double* vj = v + (int64_t)j * D;
    for (int d = 0; d < D; ++d) o_row[d] += p[j] * vj[d];
  }
  return mu + log(z);
}

static double default_scale(double scale, int D) { return scale > 0.0 ? scale : 1.0 / sqrt((double)D); }

/* ------------------------------------------------------------------------ */
/* Forward.  q,k,v: [B,H,S,D] un-rotated.  seg, pos: [B,S] or NULL.           */
/* rows: list of n_rows query indices evaluated in every (b,h) (NULL: all S   */
/* rows, n_rows ignored).  o: [B,H,n,D], lse: [B,H,n] with n = number of rows. */
/* ------------------------------------------------------------------------ */
int oracle_attn_fwd(int B, int H, int S, int D, const double* q, const double* k, const double* v,
                    const int32_t* seg, const int32_t* pos, double theta, double scale, int causal,
                    const int64_t* rows, int64_t n_rows, double* o, double* lse) {
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || (D & 1)) return 1;
  scale = default_scale(scale, D);
  int64_t n = rows ? n_rows : S;
  for (int b = 0; b < B; ++b) {
    const int32_t* seg_b = seg ? seg + (int64_t)b * S : NULL;
    for (int h = 0; h < H; ++h) {
      int64_t base = ((int64_t)b * H + h) * S * D;
      double* kr = (double*)malloc(sizeof(double) * (size_t)S * D);
      if (!kr) return 2;
      rotate_slice(k + base, kr, S, D, pos, b, theta);
#pragma omp parallel
      {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        double* qr = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n; ++r) {
          int i = rows ? (int)rows[r] : (int)r;
          const double* qi = q + base + (int64_t)i * D;
          if (theta > 0.0)
            rotate_row(qi, qr, D, position_of(pos, S, b, i), theta, 0);
          else
            memcpy(qr, qi, sizeof(double) * D);
          int64_t out = ((int64_t)b * H + h) * n + r;
          lse[out] = row_forward(qr, kr, v + base, seg_b, causal, S, D, scale, i, p, o + out * D);
        }
        free(p);
        free(qr);
      }
      free(kr);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Blocked forward: the blockwise algorithm of the paper (query rows visit K/V */
/* blocks of block_k keys, merging each block into a running max m, running   */
/* sum l and running output acc).  It exists only so that tests can check     */
/* that the blockwise result does not depend on the block size or on the      */
/* order the blocks are visited in.                                           */
/*                                                                            */
/* kv_chunk > 0 selects ring order: the sequence is cut into chunks of        */
/* kv_chunk keys; the query in chunk r visits chunk r, r-1, ..., 0, then      */
/* C-1, ..., r+1 (C chunks), as one device of a ring sees the K/V blocks of   */
/* its predecessors arrive.  Inside a chunk, blocks go in natural order.      */
/* ------------------------------------------------------------------------ */
int oracle_attn_fwd_blocked(int B, int H, int S, int D, const double* q, const double* k,
                            const double* v, const int32_t* seg, const int32_t* pos, double theta,
                            double scale, int causal, int block_k, int kv_chunk, double* o,
                            double* lse) {
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || (D & 1) || block_k <= 0) return 1;
  scale = default_scale(scale, D);
  int chunk = kv_chunk > 0 ? kv_chunk : S;
  int n_chunks = (S + chunk - 1) / chunk;
  for (int b = 0; b < B; ++b) {
    const int32_t* seg_b = seg ? seg + (int64_t)b * S : NULL;
    for (int h = 0; h < H; ++h) {
      int64_t base = ((int64_t)b * H + h) * S * D;
      double* kr = (double*)malloc(sizeof(double) * (size_t)S * D);
      if (!kr) return 2;
      rotate_slice(k + base, kr, S, D, pos, b, theta);
#pragma omp parallel
      {
        double* qr = (double*)malloc(sizeof(double) * (size_t)D);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        double* sblk = (double*)malloc(sizeof(double) * (size_t)block_k);
#pragma omp for schedule(dynamic, 16)
        for (int i = 0; i < S; ++i) {
          const double* qi = q + base + (int64_t)i * D;
          if (theta > 0.0)
            rotate_row(qi, qr, D, position_of(pos, S, b, i), theta, 0);
          else
            memcpy(qr, qi, sizeof(double) * D);
          double m = -INFINITY, l = 0.0;
          for (int d = 0; d < D; ++d) acc[d] = 0.0;
          int r = i / chunk;
          for (int t = 0; t < n_chunks; ++t) {
            int c = ((r - t) % n_chunks + n_chunks) % n_chunks;
            int c0 = c * chunk, c1 = c0 + chunk < S ? c0 + chunk : S;
            for (int j0 = c0; j0 < c1; j0 += block_k) {
              int j1 = j0 + block_k < c1 ? j0 + block_k : c1;
              /* scores of this block, masked entries at -inf */
              double bmax = -INFINITY;
              for (int j = j0; j < j1; ++j) {
                double s = visible(seg_b, causal, i, j) ? scale * dot(qr, kr + (int64_t)j * D, D)
                                                        : -INFINITY;
                sblk[j - j0] = s;
                if (s > bmax) bmax = s;
              }
              if (bmax == -INFINITY) continue; /* nothing visible in this block */
              double m_new = m > bmax ? m : bmax;
              double alpha = exp(m - m_new); /* exp(-inf) = 0 on the first block */
              l *= alpha;
              for (int d = 0; d < D; ++d) acc[d] *= alpha;
              for (int j = j0; j < j1; ++j) {
                if (sblk[j - j0] == -INFINITY) continue;
                double p = exp(sblk[j - j0] - m_new);
                l += p;
                const double* vj = v + base + (int64_t)j * D;
                for (int d = 0; d < D; ++d) acc[d] += p * vj[d];
              }
              m = m_new;
            }
          }
          int64_t out = ((int64_t)b * H + h) * S + i;
          for (int d = 0; d < D; ++d) o[out * D + d] = acc[d] / l;
          lse[out] = m + log(l);
        }
        free(qr);
        free(acc);
        free(sblk);
      }
      free(kr);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward.  With the forward's P_ij and O_i, and dO given:                  */
/*   Delta_i = <dO_i, O_i>                                                    */
/*   dP_ij   = <dO_i, v_j>                                                    */
/*   dS_ij   = P_ij (dP_ij - Delta_i)                                         */
/*   dv_j   += P_ij dO_i                                                      */
/*   dq'_i   = scale * sum_j dS_ij k'_j                                       */
/*   dk'_j  += scale * dS_ij q'_i                                             */
/* and the RoPE backward dq = R(-a) dq', dk = R(-a) dk'.                      */
/*                                                                            */
/* Only the query rows listed in rows (NULL: all) contribute.  dq has one row */
/* per listed query: [B,H,n,D].  dk and dv hold the contributions of those    */
/* rows to the key columns [col_begin, col_end): [B,H,col_end-col_begin,D].   */
/* A column is exact when every row that sees it is listed.                   */
/* ------------------------------------------------------------------------ */
int oracle_attn_bwd(int B, int H, int S, int D, const double* q, const double* k, const double* v,
                    const double* dout, const int32_t* seg, const int32_t* pos, double theta,
                    double scale, int causal, const int64_t* rows, int64_t n_rows, int col_begin,
                    int col_end, double* dq, double* dk, double* dv) {
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || (D & 1)) return 1;
  if (col_begin < 0 || col_end > S || col_begin > col_end) return 1;
  scale = default_scale(scale, D);
  int64_t n = rows ? n_rows : S;
  int ncol = col_end - col_begin;
  for (int b = 0; b < B; ++b) {
    const int32_t* seg_b = seg ? seg + (int64_t)b * S : NULL;
    for (int h = 0; h < H; ++h) {
      int64_t base = ((int64_t)b * H + h) * S * D;
      int64_t bh = (int64_t)b * H + h;
      double* kr = (double*)malloc(sizeof(double) * (size_t)S * D);
      if (!kr) return 2;
      rotate_slice(k + base, kr, S, D, pos, b, theta);
      double* dkr_out = dk + bh * (int64_t)ncol * D; /* accumulates dk' (rotated frame) */
      double* dv_out = dv + bh * (int64_t)ncol * D;
      memset(dkr_out, 0, sizeof(double) * (size_t)ncol * D);
      memset(dv_out, 0, sizeof(double) * (size_t)ncol * D);
#pragma omp parallel
      {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        double* qr = (double*)malloc(sizeof(double) * (size_t)D);
        double* o_row = (double*)malloc(sizeof(double) * (size_t)D);
        double* dqr = (double*)malloc(sizeof(double) * (size_t)D);
        double* dk_loc = (double*)calloc((size_t)ncol * D, sizeof(double));
        double* dv_loc = (double*)calloc((size_t)ncol * D, sizeof(double));
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < n; ++r) {
          int i = rows ? (int)rows[r] : (int)r;
          const double* qi = q + base + (int64_t)i * D;
          double pos_i = position_of(pos, S, b, i);
          if (theta > 0.0)
            rotate_row(qi, qr, D, pos_i, theta, 0);
          else
            memcpy(qr, qi, sizeof(double) * D);
          row_forward(qr, kr, v + base, seg_b, causal, S, D, scale, i, p, o_row);
          const double* doi = dout + base + (int64_t)i * D;
          double delta = dot(doi, o_row, D);
          for (int d = 0; d < D; ++d) dqr[d] = 0.0;
          for (int j = 0; j < S; ++j) {
            if (!visible(seg_b, causal, i, j)) continue;
            const double* vj = v + base + (int64_t)j * D;
            double dp = dot(doi, vj, D);
            double ds = p[j] * (dp - delta);
            const double* kj = kr + (int64_t)j * D;
            for (int d = 0; d < D; ++d) dqr[d] += scale * ds * kj[d];
            if (j >= col_begin && j < col_end) {
              double* dkj = dk_loc + (int64_t)(j - col_begin) * D;
              double* dvj = dv_loc + (int64_t)(j - col_begin) * D;
              for (int d = 0; d < D; ++d) {
                dkj[d] += scale * ds * qr[d];
                dvj[d] += p[j] * doi[d];
              }
            }
          }
          double* dq_out = dq + (bh * n + r) * D;
          if (theta > 0.0)
            rotate_row(dqr, dq_out, D, pos_i, theta, 1);
          else
            memcpy(dq_out, dqr, sizeof(double) * D);
        }
#pragma omp critical
        {
          for (int64_t e = 0; e < (int64_t)ncol * D; ++e) {
            dkr_out[e] += dk_loc[e];
            dv_out[e] += dv_loc[e];
          }
        }
        free(p);
        free(qr);
        free(o_row);
        free(dqr);
        free(dk_loc);
        free(dv_loc);
      }
      /* RoPE backward on the key gradients */
      if (theta > 0.0) {
        double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
        for (int c = 0; c < ncol; ++c) {
          double* row = dkr_out + (int64_t)c * D;
          rotate_row(row, tmp, D, position_of(pos, S, b, col_begin + c), theta, 1);
          memcpy(row, tmp, sizeof(double) * D);
        }
        free(tmp);
      }
      free(kr);
    }
  }
  return 0;
}
