/*
 * segquant_oracle.c -- plain CPU oracle for the DualScale x SegLinear W8A8
 * linear layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark load this library; the product path
 * (libsegquant) never links, loads or calls it, and shares no code with it.
 *
 * It is written to be read against the pages, not to be fast: loops follow
 * the definitions, floating point follows the stated precision, integer sums
 * are exact.  The only concession to speed is OpenMP over independent output
 * rows (results do not depend on it: integer sums are exact and each fp64 sum
 * is taken in a fixed order inside one thread).
 *
 * Sources cited below:
 *   [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization
 *        Framework for Diffusion Models", paper notes (papernotes.org,
 *        CVPR 2026).
 *   [P2] "SegQuant", project page (hliangzhao.me/works/segquant.html).
 *
 * Readings taken where the pages leave a step open (the reason for each is
 * that it is the plainest reading the rest of the pages support, or the one
 * that keeps the codes in int8; each is pinned by a test):
 *   R1  q_max = 127 and q_min = 128 (a magnitude): s+ = max/127,
 *       s- = |min|/128, so the negative half lives in [-128, 0].
 *   R2  "round" is round-half-to-even.
 *   R3  x/s is taken as one IEEE fp32 product x*inv with the fp32 inverse
 *       inv passed in, then rounded to an integer; never fused.
 *   R4  clamps: positive half [0,127], negative half [-128,0], weights
 *       [-127,127].
 *   R5  a zero range gives s = 0 and inv = 0, so that half is all zeros.
 *   R8  input-segmented: one (s+, s-) pair per K-segment; output-segmented
 *       (or unsegmented) input: one pair for the whole K.
 *   R9  weight scale group: the whole sub-matrix of a segment (K-segment x
 *       N-segment block), or one column per K-segment when per_column is set.
 *   R10 dequantisation sums in fp64 here.
 *
 * Parity pins for every function are in tests/test_oracle.py; none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(_OPENMP)
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_OVERFLOW (-2)

/* bf16 is the top half of an IEEE binary32: widening is exact. */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int oracle_num_threads(void) {
#if defined(_OPENMP)
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Segment list check: offsets start at 0, are contiguous, widths positive,
 * and the list covers exactly `dim`. */
static int segs_ok(int32_t n, const int32_t *off, const int32_t *wid, int64_t dim) {
  if (n < 1 || !off || !wid) return 0;
  int64_t at = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (off[i] != at || wid[i] <= 0) return 0;
    at += wid[i];
  }
  return at == dim;
}

/* Index of the segment that holds position k. */
static int32_t seg_of(int64_t k, int32_t n, const int32_t *off, const int32_t *wid) {
  for (int32_t i = 0; i < n; ++i)
    if (k >= off[i] && k < (int64_t)off[i] + wid[i]) return i;
  return -1;
}

/* ------------------------------------------------------------------------
 * Polarity split  [P1 "DualScale" section, split equation; P2 section 3]:
 *   X+ = max(X, 0),  X- = min(X, 0)   (elementwise, exact in fp32).
 * ---------------------------------------------------------------------- */
void oracle_polarity_split(const uint16_t *x_bf16, int64_t n, float *x_pos, float *x_neg) {
  for (int64_t i = 0; i < n; ++i) {
    float x = bf16_to_f32(x_bf16[i]);
    x_pos[i] = x > 0.0f ? x : 0.0f;
    x_neg[i] = x < 0.0f ? x : 0.0f;
  }
}

/* Scale and inverse of a range a >= 0 spread over `levels` steps:
 * s = a/levels and inv = levels/a, each formed in fp64 and rounded once to
 * fp32.  A zero range, or one so small that levels/a overflows fp32 (a below
 * about 3.7e-37), counts as zero: s = inv = 0 (R5). */
static void range_scale(double a, double levels, float *s, float *inv) {
  float iv = a > 0.0 ? (float)(levels / a) : 0.0f;
  if (isinf(iv)) iv = 0.0f;
  *inv = iv;
  *s = iv == 0.0f ? 0.0f : (float)(a / levels);
}

/* ------------------------------------------------------------------------
 * AMax activation calibration  [P1 framework table, AMax calibrator;
 * P1 "DualScale" scale equation; P2 section 3, s- and s+ definitions]
 * per K-segment i (R1, R5, R8):
 *   mx = max(0, max x),  mn = min(0, min x)   over X[:, segment i]
 *   s+ = mx / 127,   inv+ = 127 / mx
 *   s- = |mn| / 128, inv- = 128 / |mn|
 * through range_scale (fp64 quotients rounded once; zero ranges give 0).
 * ---------------------------------------------------------------------- */
int oracle_calibrate_amax(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                          int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                          float *s_pos, float *s_neg, float *inv_pos, float *inv_neg) {
  if (M < 0 || K < 1 || ld < K || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
  for (int32_t i = 0; i < n_kseg; ++i) {
    float mx = 0.0f, mn = 0.0f;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = koff[i]; k < (int64_t)koff[i] + kwid[i]; ++k) {
        float v = bf16_to_f32(x[m * ld + k]);
        if (v > mx) mx = v;
        if (v < mn) mn = v;
      }
    range_scale((double)mx, 127.0, &s_pos[i], &inv_pos[i]);
    range_scale(-(double)mn, 128.0, &s_neg[i], &inv_neg[i]);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * The producers of the activation [P1 DualScale motivation; P2 section 3:
 * SiLU and GELU leave a wide positive and a narrow negative range], in fp64
 * from a bf16 pre-activation z:
 *   kind 1  SiLU  z / (1 + exp(-z))
 *   kind 2  GELU  z/2 (1 + erf(z / sqrt 2))   (the exact form)
 * The kernels evaluate these in fp32 and round to bf16; the tests accept
 * any bf16 value (and code) between those of act(z) -/+ a stated bound.
 * ---------------------------------------------------------------------- */
int oracle_activation(const uint16_t *z, int64_t n, int32_t kind, double *out) {
  if (n < 0 || (kind != 1 && kind != 2)) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)bf16_to_f32(z[i]);
    /* GELU through erfc(-z / sqrt 2) = 1 + erf(z / sqrt 2): no cancellation
       for negative z, where 1 + erf would lose every digit in fp64 too */
    out[i] = kind == 1 ? v / (1.0 + exp(-v)) : 0.5 * v * erfc(-v / sqrt(2.0));
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Single-scale calibration, the plain W8A8 baseline that DualScale is
 * measured against  [P2 deployment-cost table, INT8 baseline row; P1
 * limitations section: DualScale could be enabled per layer only where the
 * polarity asymmetry is strong].  Per K-segment i one symmetric range:
 *   a = max(max x, -min x)   over X[:, segment i]
 *   s = a / 127, inv = 127 / a   (range_scale; zero range gives 0)
 * stored in both halves (s+ = s- = s, inv+ = inv- = inv), so that the
 * dual-scale quantisation below produces clamp(rne(fp32(x * inv)),
 * -127, 127) and the dequantisation the single-scale sum.
 * ---------------------------------------------------------------------- */
int oracle_calibrate_amax_single(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                                 int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                                 float *s_pos, float *s_neg, float *inv_pos, float *inv_neg) {
  if (M < 0 || K < 1 || ld < K || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
  for (int32_t i = 0; i < n_kseg; ++i) {
    double a = 0.0;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = koff[i]; k < (int64_t)koff[i] + kwid[i]; ++k) {
        double v = fabs((double)bf16_to_f32(x[m * ld + k]));
        if (v > a) a = v;
      }
    range_scale(a, 127.0, &s_pos[i], &inv_pos[i]);
    s_neg[i] = s_pos[i];
    inv_neg[i] = inv_pos[i];
  }
  return ORACLE_OK;
}

/* One half's code: rne of the fp32 product (R2, R3), then clamp (R4).
 * A zero inverse means a zero range: that half is all zeros (R5). */
static int32_t quant_code(float v_half, float inv, int32_t lo, int32_t hi) {
  if (inv == 0.0f) return 0;
  float p = v_half * inv;          /* one IEEE binary32 multiply */
  float r = nearbyintf(p);         /* default mode: round half to even */
  if (r < (float)lo) return lo;    /* +-Inf saturate here */
  if (r > (float)hi) return hi;
  return (int32_t)r;
}

/* ------------------------------------------------------------------------
 * Dual-scale activation quantisation  [P2 section 3, Q_dual equation;
 * P1 "DualScale" quantisation scheme] for k in K-segment i:
 *   q+[m][k] = clamp(rne(x+ * inv+_i), 0, 127)
 *   q-[m][k] = clamp(rne(x- * inv-_i), -128, 0)
 * Output: two int8 planes, row-major [M][K].
 * ---------------------------------------------------------------------- */
int oracle_quantize_dualscale(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                              int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                              const float *inv_pos, const float *inv_neg,
                              int8_t *q_pos, int8_t *q_neg) {
  if (M < 0 || K < 1 || ld < K || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    float xp[1], xn[1];
    for (int64_t k = 0; k < K; ++k) {
      int32_t i = seg_of(k, n_kseg, koff, kwid);
      oracle_polarity_split(&x[m * ld + k], 1, xp, xn);
      q_pos[m * K + k] = (int8_t)quant_code(xp[0], inv_pos[i], 0, 127);
      q_neg[m * K + k] = (int8_t)quant_code(xn[0], inv_neg[i], -128, 0);
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Symmetric int8 weight quantisation per group  [P1 SegLinear section,
 * output-segmented and input-segmented patterns: each segment of W is
 * quantised on its own; P2 section 2, same two equations] (R4, R5, R9).
 * W is fp32 row-major [K][ldw] (Y = X W, W in R^{k x n}).  The group of
 * (k, n) is (K-segment of k) x (N-segment of n), or (K-segment of k) x
 * {column n} when per_column != 0.  Per group:
 *   a = max |w|;  s_w = a / 127;  inv_w = 127 / a   (range_scale)
 *   w_q = clamp(rne(w * inv_w), -127, 127)
 * Outputs: w_q int8 [K][N] and w_scale fp32 [n_kseg][N] (the s_w of the
 * group holding (segment i, column n)).
 * ---------------------------------------------------------------------- */
/* levels: 127 (int8) or 7 (the 4-bit weights of W4A8 [P2 deployment-cost
 * table, SegQuant-4; P1 experiments, W4A8]; reading: the same groups,
 * symmetric codes in [-7, 7]). */
static int quantize_weight_levels(const float *w, int64_t K, int64_t N, int64_t ldw,
                                  int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                                  int32_t n_nseg, const int32_t *noff, const int32_t *nwid,
                                  int32_t per_column, int8_t *w_q, float *w_scale,
                                  int32_t levels) {
  if (K < 1 || N < 1 || ldw < N || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
  if (!per_column && !segs_ok(n_nseg, noff, nwid, N)) return ORACLE_ERR_ARG;
  int32_t ng = per_column ? (int32_t)N : n_nseg;
  for (int32_t i = 0; i < n_kseg; ++i) {
    for (int32_t j = 0; j < ng; ++j) {
      int64_t n0 = per_column ? j : noff[j];
      int64_t n1 = per_column ? j + 1 : (int64_t)noff[j] + nwid[j];
      float a = 0.0f;
      for (int64_t k = koff[i]; k < (int64_t)koff[i] + kwid[i]; ++k)
        for (int64_t n = n0; n < n1; ++n) {
          float v = fabsf(w[k * ldw + n]);
          if (v > a) a = v;
        }
      float s_w, inv_w;
      range_scale((double)a, (double)levels, &s_w, &inv_w);
      for (int64_t n = n0; n < n1; ++n) w_scale[(int64_t)i * N + n] = s_w;
      for (int64_t k = koff[i]; k < (int64_t)koff[i] + kwid[i]; ++k)
        for (int64_t n = n0; n < n1; ++n)
          w_q[k * N + n] = (int8_t)quant_code(w[k * ldw + n], inv_w, -levels, levels);
    }
  }
  return ORACLE_OK;
}

int oracle_quantize_weight(const float *w, int64_t K, int64_t N, int64_t ldw,
                           int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                           int32_t n_nseg, const int32_t *noff, const int32_t *nwid,
                           int32_t per_column, int8_t *w_q, float *w_scale) {
  return quantize_weight_levels(w, K, N, ldw, n_kseg, koff, kwid, n_nseg, noff, nwid,
                                per_column, w_q, w_scale, 127);
}

int oracle_quantize_weight_w4(const float *w, int64_t K, int64_t N, int64_t ldw,
                              int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                              int32_t n_nseg, const int32_t *noff, const int32_t *nwid,
                              int32_t per_column, int8_t *w_q, float *w_scale) {
  return quantize_weight_levels(w, K, N, ldw, n_kseg, koff, kwid, n_nseg, noff, nwid,
                                per_column, w_q, w_scale, 7);
}

/* ------------------------------------------------------------------------
 * Per-segment integer products  [P1 input-segmented equation: Y is the sum
 * over segments of X_i W_i; P1 "DualScale" reconstruction: one product per
 * polarity half; P2 sections 2 and 3]:
 *   A+_i[m][n] = sum_{k in segment i} q+[m][k] * w_q[k][n]
 *   A-_i[m][n] = sum_{k in segment i} q-[m][k] * w_q[k][n]
 * Exact: accumulated in int64, checked to fit int32, stored int32 as
 * acc[h][i][m][n] with h = 0 for the + half and 1 for the - half.
 * ---------------------------------------------------------------------- */
int oracle_segment_acc(const int8_t *q_pos, const int8_t *q_neg, const int8_t *w_q,
                       int64_t M, int64_t K, int64_t N,
                       int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                       int32_t *acc) {
  if (M < 0 || K < 1 || N < 1 || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
  int overflow = 0;
  const int8_t *halves[2] = {q_pos, q_neg};
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t m = 0; m < M; ++m) {
    int64_t *row = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    for (int h = 0; h < 2; ++h)
      for (int32_t i = 0; i < n_kseg; ++i) {
        for (int64_t n = 0; n < N; ++n) row[n] = 0;
        for (int64_t k = koff[i]; k < (int64_t)koff[i] + kwid[i]; ++k) {
          int64_t a = halves[h][m * K + k];
          for (int64_t n = 0; n < N; ++n) row[n] += a * (int64_t)w_q[k * N + n];
        }
        int32_t *out = acc + (((int64_t)h * n_kseg + i) * M + m) * N;
        for (int64_t n = 0; n < N; ++n) {
          if (row[n] > INT32_MAX || row[n] < INT32_MIN) overflow = 1;
          out[n] = (int32_t)row[n];
        }
      }
    free(row);
  }
  return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Dequantisation  [P1 "DualScale" reconstruction equation; P2 section 3,
 * reconstruction equation; P1/P2 input-segmented sum] (R10):
 *   y[m][n] = sum_i w_scale[i][n] * (s+_i * A+_i[m][n] + s-_i * A-_i[m][n])
 * in fp64, segments summed in index order.
 * ---------------------------------------------------------------------- */
int oracle_dequantize(const int32_t *acc, int64_t M, int64_t N, int32_t n_kseg,
                      const float *s_pos, const float *s_neg, const float *w_scale,
                      double *y) {
  if (M < 0 || N < 1 || n_kseg < 1) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0;
      for (int32_t i = 0; i < n_kseg; ++i) {
        double ap = (double)acc[((int64_t)0 * n_kseg + i) * M * N + m * N + n];
        double an = (double)acc[((int64_t)1 * n_kseg + i) * M * N + m * N + n];
        sum += (double)w_scale[(int64_t)i * N + n] *
               ((double)s_pos[i] * ap + (double)s_neg[i] * an);
      }
      y[m * N + n] = sum;
    }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * The whole layer, one output row at a time: quantise the row, form both
 * halves' per-segment integer sums, dequantise.  Same arithmetic as the
 * three functions above composed (rows of Y depend only on the same row
 * of X), without materialising [2][S][M][N]; used for large inputs and as
 * the timed CPU baseline.
 * ---------------------------------------------------------------------- */
int oracle_dualscale_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                            const int8_t *w_q, const float *w_scale, int64_t N,
                            int32_t n_kseg, const int32_t *koff, const int32_t *kwid,
                            const float *s_pos, const float *s_neg,
                            const float *inv_pos, const float *inv_neg, double *y) {
  if (M < 0 || K < 1 || N < 1 || ld < K || !segs_ok(n_kseg, koff, kwid, K)) return ORACLE_ERR_ARG;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t m = 0; m < M; ++m) {
    int8_t *qp = (int8_t *)malloc((size_t)K);
    int8_t *qn = (int8_t *)malloc((size_t)K);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * 2 * (size_t)n_kseg * (size_t)N);
    double *yr = (double *)malloc(sizeof(double) * (size_t)N);
    if (oracle_quantize_dualscale(x + m * ld, 1, K, ld, n_kseg, koff, kwid, inv_pos, inv_neg,
                                  qp, qn) != ORACLE_OK ||
        oracle_segment_acc(qp, qn, w_q, 1, K, N, n_kseg, koff, kwid, acc) != ORACLE_OK ||
        oracle_dequantize(acc, 1, N, n_kseg, s_pos, s_neg, w_scale, yr) != ORACLE_OK)
      bad = 1;
    for (int64_t n = 0; n < N; ++n) y[m * N + n] = yr[n];
    free(qp); free(qn); free(acc); free(yr);
  }
  return bad ? ORACLE_ERR_ARG : ORACLE_OK;
}
