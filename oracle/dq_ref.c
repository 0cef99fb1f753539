/*
 * dq_ref.c -- CPU oracle for the DualQuant dual-scale weight-reconstruction solver.
 *
 * TEST INFRASTRUCTURE, not product code: only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg load this library. It is a plain,
 * slow, obviously-correct reading of the method in double precision, written
 * independently of the HIP library (no shared source, header or table).
 *
 * Sources (DualQuant pages):
 *  - daiwk reproduction notes, "核心公式": eq. 1 (W ~= D_alpha^-1 Q(D_alpha W D_beta) D_beta^-1),
 *    eq. 2 (closed-form row / column inverse-scale updates with R = Qhat D_b, S = D_a Qhat),
 *    and the conventions under it (re-quantize after the row update, then solve the
 *    columns and re-quantize; an all-zero-code slice takes scale 1; the projection acts
 *    on the inverse scale).
 *  - daiwk notes, "原始论文总结" (variable splitting: inner copies decide the grid
 *    assignment, outer copies the reconstruction; Q is a black box) and its flowchart.
 *  - daiwk notes, "本地复现" (INT4 codebook [-8, 7] with BF16 scales; MXINT4 with E8M0
 *    power-of-two scales, exponent in [-126, 126]).
 *  - trove summary, "How it works" (the update order and the flowchart) and the
 *    news article's block-format paragraph (MXFP4: 32-element blocks, E2M1 elements,
 *    E8M0 shared scale; NVFP4: 16-element blocks with an E4M3 scale).
 * Where the pages leave a step open, the reading taken is stated at that step.
 *
 * Arithmetic conventions:
 *  - every "fl32(.)" step is one IEEE round-to-nearest-even binary32 operation; it is
 *    written as (float) of one double operation on float operands, which gives the same
 *    result (the double result of +, *, / of two floats rounds innocuously, 53 >= 2*24+2);
 *  - a code rounds the exact real quotient x/d: the double quotient of two floats lies on
 *    the same side of every rounding boundary (half-integers, E2M1 midpoints) as the exact
 *    quotient, and equals a boundary only when the exact quotient does, because a quotient
 *    of two 24-bit numbers that is not a boundary stays more than 2^-30 (relative) away
 *    from any boundary with at most 3 significant bits, far above the 2^-53 division error;
 *  - sums are plain double sums in ascending index order; subnormals are kept; this file
 *    is compiled with -ffp-contract=off so no multiply-add is fused.
 */
#include "dq_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

int dq_ref_set_threads(int n) {
  if (n < 1) n = 1;
#ifdef _OPENMP
  g_threads = n;
#else
  g_threads = 1;
#endif
  return g_threads;
}

/* ------------------------------------------------------------------ scalar helpers */

static float fl32_mul(float x, float y) { return (float)((double)x * (double)y); }
static float fl32_div(float x, float y) { return (float)((double)x / (double)y); }

/* nearest integer, ties to even, independent of the FP environment (|v| < 2^52) */
static double rne_int(double v) {
  double f = floor(v);
  double frac = v - f; /* exact */
  if (frac > 0.5) return f + 1.0;
  if (frac < 0.5) return f;
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* E2M1 magnitudes, index 0..7 (sign is a separate bit) */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Nearest E2M1 value to v; a tie between two neighbours goes to the even index.
 * Values beyond 6 in magnitude map to +-6 (the nearest grid value). -0 becomes +0. */
double dq_ref_e2m1_round(double v) {
  double av = fabs(v);
  int best = 0;
  double bd = av;
  for (int k = 1; k < 8; k++) {
    double dd = fabs(av - E2M1_GRID[k]);
    /* ties occur only between neighbours k-1 and k; keep the even one */
    if (dd < bd || (dd == bd && (k % 2) == 0)) {
      best = k;
      bd = dd;
    }
  }
  if (best == 0) return 0.0;
  return v < 0 ? -E2M1_GRID[best] : E2M1_GRID[best];
}

/* Nearest bf16 value to v >= 0 (8 significant bits; below 2^-126 the bf16 grid is
 * uniform with spacing 2^-133), ties to even. Inputs here never reach bf16 overflow. */
double dq_ref_bf16_rne(double v) {
  if (v == 0.0) return 0.0;
  if (v < ldexp(1.0, -126)) return ldexp(rne_int(ldexp(v, 133)), -133);
  int e;
  double f = frexp(v, &e); /* v = f * 2^e, f in [0.5, 1) */
  return ldexp(rne_int(ldexp(f, 8)), e - 8);
}

/* Nearest E4M3FN value to v >= 0, ties to even mantissa, saturating at 448.
 * E4M3FN: bias 7, 3 mantissa bits, normals from 2^-6, subnormals k * 2^-9. */
double dq_ref_e4m3_rne_sat(double v) {
  if (v >= 448.0) return 448.0;
  double r;
  if (v < ldexp(1.0, -6)) {
    r = ldexp(rne_int(ldexp(v, 9)), -9);
  } else {
    int e;
    double f = frexp(v, &e);
    r = ldexp(rne_int(ldexp(f, 4)), e - 4);
  }
  return r > 448.0 ? 448.0 : r;
}

/* --------------------------------------------------------- projections Pi_F (eq. 2) */
/* Pi_F maps a positive closed-form value to the nearest value of the format's scale
 * set. For fixed codes the row objective is D_i (a - N_i/D_i)^2 + const, so the
 * nearest feasible point is the constrained minimiser. */

#define BF16_MAX_FINITE (255.0 * 0x1p120) /* (2 - 2^-7) * 2^127 */

static double proj_bf16(double v) {
  /* reading: outer BF16 scales stay normal, in [2^-126, max finite bf16] */
  double lo = ldexp(1.0, -126);
  if (!(v > lo)) return lo;
  int e;
  double f = frexp(v, &e);
  double r = ldexp(rne_int(ldexp(f, 8)), e - 8);
  return r > BF16_MAX_FINITE ? BF16_MAX_FINITE : r;
}

static double proj_e8m0(double v) {
  /* powers of two 2^k, k in [-126, 126] (daiwk notes, "本地复现"); nearest in value,
   * so between p and 2p the midpoint 1.5p decides; reading: the midpoint goes up */
  int e;
  frexp(v, &e); /* v in [2^(e-1), 2^e) */
  int k = e - 1;
  double p = ldexp(1.0, k);
  if (v >= 1.5 * p) k += 1;
  if (k < -126) k = -126;
  if (k > 126) k = 126;
  return ldexp(1.0, k);
}

static double proj_e4m3(double v) {
  /* E4M3FN values; reading: never 0 (floor 2^-9), saturate at 448 */
  double r = dq_ref_e4m3_rne_sat(v);
  double lo = ldexp(1.0, -9);
  return r < lo ? lo : r;
}

double dq_ref_project(int fmt, double v) {
  switch (fmt) {
    case DQR_FMT_INT4_BF16: return proj_bf16(v);
    case DQR_FMT_MXINT4:
    case DQR_FMT_MXFP4: return proj_e8m0(v);
    case DQR_FMT_NVFP4: return proj_e4m3(v);
    default: return NAN;
  }
}

/* sorted positive E4M3FN values, for neighbour lookups in the margin diagnostic */
static double e4m3_table[126];
static int e4m3_table_ready = 0;
static void e4m3_table_init(void) {
  if (e4m3_table_ready) return;
  int n = 0;
  for (int code = 1; code <= 0x7E; code++) {
    int ef = code >> 3, mf = code & 7;
    e4m3_table[n++] = ef == 0 ? ldexp((double)mf, -9) : ldexp(1.0 + mf / 8.0, ef - 7);
  }
  e4m3_table_ready = 1;
}

/* relative distance from v to the nearest decision boundary of Pi_F: |v - t| / v for the
 * nearest midpoint t between two neighbouring values of the scale set (infinite where the
 * set has a single value on each side, which never happens) */
double dq_ref_proj_margin(int fmt, double v) {
  double p = dq_ref_project(fmt, v), prev = 0, next = 0;
  int has_prev = 1, has_next = 1;
  if (fmt == DQR_FMT_INT4_BF16) {
    int e = ilogb(p);
    next = p + ldexp(1.0, e - 7);
    prev = (p == ldexp(1.0, e)) ? p - ldexp(1.0, e - 8) : p - ldexp(1.0, e - 7);
    if (p <= ldexp(1.0, -126)) has_prev = 0;
    if (p >= BF16_MAX_FINITE) has_next = 0;
  } else if (fmt == DQR_FMT_NVFP4) {
    e4m3_table_init();
    int k = 0;
    while (k < 126 && e4m3_table[k] != p) k++;
    has_prev = k > 0;
    has_next = k < 125;
    if (has_prev) prev = e4m3_table[k - 1];
    if (has_next) next = e4m3_table[k + 1];
  } else {
    next = 2 * p;
    prev = p / 2;
    if (p <= ldexp(1.0, -126)) has_prev = 0;
    if (p >= ldexp(1.0, 126)) has_next = 0;
  }
  double m = INFINITY;
  if (has_prev) m = fmin(m, fabs(v - 0.5 * (prev + p)) / v);
  if (has_next) m = fmin(m, fabs(v - 0.5 * (p + next)) / v);
  return m;
}

/* ------------------------------------------------------------------ the quantizer Q */

typedef struct {
  const void* W;
  int wt;
  int64_t m, n;
  int fmt, G;
  int64_t ng;     /* groups per row */
  float g, sixg;  /* NVFP4 tensor scale and fl32(6 g) */
} ctx_t;

static float w_at(const ctx_t* c, int64_t i, int64_t j) {
  int64_t idx = i * c->n + j;
  if (c->wt == DQR_F32) return ((const float*)c->W)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)c->W)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint16_t bf16_bits(double s) {
  float f = (float)s; /* s is an exact bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static uint8_t e4m3_bits(double s) { /* s is an exact positive E4M3FN value */
  if (s < ldexp(1.0, -6)) return (uint8_t)ldexp(s, 9);
  int e;
  double f = frexp(s, &e); /* s = (2f) 2^(e-1), 2f in [1, 2) */
  int ef = (e - 1) + 7;
  int mf = (int)((2.0 * f - 1.0) * 8.0);
  return (uint8_t)((ef << 3) | mf);
}

/* Q on one group of G scaled values x (reading of the black-box quantizer, one rule per
 * format, chosen so that Q is idempotent):
 *   INT4_BF16: s = bf16(fl32(m/7)) (never below 2^-133), codes nearest integer in [-8, 7];
 *   MXINT4:    s = 2^clamp(floor(log2 m) - 2, -126, 126) (OCP shared-exponent rule with the
 *              INT4 element read as 1.2 fixed point), codes nearest integer in [-7, 7];
 *   MXFP4:     same scale rule (E2M1 emax = 2), codes nearest E2M1;
 *   NVFP4:     u = fl32(m / fl32(6 g)), s = max(E4M3(u), 2^-9), divisor d = fl32(s g),
 *              codes nearest E2M1;
 * with m = max |x| and s = 1 (E8M0 exponent 0) for an all-zero group.
 * Outputs twice the code value (an exact small integer), the divisor d and the stored
 * scale encoding. */
static void quant_group(const ctx_t* c, const float* x, int8_t* q2, double* d_out,
                        uint16_t* scode_out) {
  const int G = c->G;
  float m = 0.0f;
  for (int k = 0; k < G; k++) m = fmaxf(m, fabsf(x[k]));
  double d;
  uint16_t scode;
  switch (c->fmt) {
    case DQR_FMT_INT4_BF16: {
      double s = 1.0;
      if (m > 0) {
        s = dq_ref_bf16_rne((double)fl32_div(m, 7.0f));
        if (s < ldexp(1.0, -133)) s = ldexp(1.0, -133);
      }
      d = s;
      scode = bf16_bits(s);
      for (int k = 0; k < G; k++) {
        double q = rne_int((double)x[k] / d);
        if (q < -8) q = -8;
        if (q > 7) q = 7;
        q2[k] = (int8_t)(2.0 * q);
      }
      break;
    }
    case DQR_FMT_MXINT4:
    case DQR_FMT_MXFP4: {
      int e = 0;
      if (m > 0) {
        int ex;
        frexp((double)m, &ex); /* floor(log2 m) = ex - 1 */
        e = (ex - 1) - 2;
        if (e < -126) e = -126;
        if (e > 126) e = 126;
      }
      d = ldexp(1.0, e);
      scode = (uint16_t)(e + 127);
      for (int k = 0; k < G; k++) {
        double v = (double)x[k] / d;
        double q;
        if (c->fmt == DQR_FMT_MXINT4) {
          q = rne_int(v);
          if (q < -7) q = -7;
          if (q > 7) q = 7;
        } else {
          q = dq_ref_e2m1_round(v);
        }
        q2[k] = (int8_t)(2.0 * q);
      }
      break;
    }
    default: { /* NVFP4 */
      double s = 1.0;
      if (m > 0) {
        float u = fl32_div(m, c->sixg);
        s = dq_ref_e4m3_rne_sat((double)u);
        if (s < ldexp(1.0, -9)) s = ldexp(1.0, -9);
      }
      d = (double)fl32_mul((float)s, c->g);
      scode = e4m3_bits(s);
      for (int k = 0; k < G; k++) q2[k] = (int8_t)(2.0 * dq_ref_e2m1_round((double)x[k] / d));
      break;
    }
  }
  *d_out = d; /* codes are held as integers, so no negative zero survives */
  *scode_out = scode;
}

/* One pass of Q over X = fl32(fl32(W * rb) * ra) (column scale first, then row scale).
 * Returns DQR_ERR_RANGE if a scaled value is not finite. */
static int q_pass(const ctx_t* c, const float* ra, const float* rb, int8_t* q2, double* dv,
                  uint16_t* sc) {
  int bad = 0;
  const int64_t m = c->m, n = c->n, ng = c->ng;
  const int G = c->G;
#pragma omp parallel for num_threads(g_threads) schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < m; i++) {
    float x[64];
    for (int64_t gi = 0; gi < ng; gi++) {
      int row_bad = 0;
      for (int k = 0; k < G; k++) {
        int64_t j = gi * G + k;
        x[k] = fl32_mul(fl32_mul(w_at(c, i, j), rb[j]), ra[i]);
        if (!isfinite(x[k])) row_bad = 1;
      }
      if (row_bad) {
        bad = 1;
        break;
      }
      quant_group(c, x, q2 + i * n + gi * G, dv + i * ng + gi, sc + i * ng + gi);
    }
  }
  return bad ? DQR_ERR_RANGE : DQR_OK;
}

/* mean squared error of the synced state: sum_ij (W - a_i d_ig q_ij b_j)^2 / (m n) */
static double mse_of(const ctx_t* c, const float* a, const float* b, const int8_t* q2,
                     const double* dv, double* row_err) {
  const int64_t m = c->m, n = c->n, ng = c->ng;
  const int G = c->G;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t i = 0; i < m; i++) {
    double s = 0.0;
    for (int64_t j = 0; j < n; j++) {
      double rec = (double)a[i] * dv[i * ng + j / G] * (0.5 * q2[i * n + j]) * (double)b[j];
      double r = (double)w_at(c, i, j) - rec;
      s += r * r;
    }
    row_err[i] = s;
  }
  double tot = 0.0;
  for (int64_t i = 0; i < m; i++) tot += row_err[i];
  return tot / ((double)m * (double)n);
}

static void fill_reciprocals(const float* v, float* rv, int64_t len) {
  for (int64_t k = 0; k < len; k++) rv[k] = (float)(1.0 / (double)v[k]); /* fl32(1/v) */
}

static int64_t count_diff_i8(const int8_t* x, const int8_t* y, int64_t len) {
  int64_t c = 0;
  for (int64_t k = 0; k < len; k++) c += x[k] != y[k];
  return c;
}
static int64_t count_diff_u16(const uint16_t* x, const uint16_t* y, int64_t len) {
  int64_t c = 0;
  for (int64_t k = 0; k < len; k++) c += x[k] != y[k];
  return c;
}

/* ------------------------------------------------------------------- argument checks */

static int check_common(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group) {
  if (fmt < 0 || fmt > 3 || (wt != DQR_F32 && wt != DQR_BF16)) return DQR_ERR_UNSUPPORTED;
  if (!W || rows <= 0 || cols <= 0) return DQR_ERR_ARG;
  if (group != 16 && group != 32 && group != 64) return DQR_ERR_ARG;
  if (cols % group != 0) return DQR_ERR_ARG;
  if (rows > ((int64_t)1 << 40) / cols) return DQR_ERR_ARG;
  return DQR_OK;
}

static int positive_finite(const float* v, int64_t len) {
  for (int64_t k = 0; k < len; k++)
    if (!(v[k] > 0.0f) || !isfinite(v[k])) return 0;
  return 1;
}

static int w_finite(const ctx_t* c) {
  for (int64_t i = 0; i < c->m; i++)
    for (int64_t j = 0; j < c->n; j++)
      if (!isfinite(w_at(c, i, j))) return 0;
  return 1;
}

/* NVFP4 per-tensor scale (reading; the pages fix only the E4M3 16-element block scale):
 * g = fl32(A / 2688) with A = max|X| of the given scaled tile and 2688 = 6 * 448, so that
 * the largest block maps to the largest E4M3 scale; A = 0 gives g = 1, and g never drops
 * below 2^-126. Computed once from the initial state and then held fixed. */
static float tensor_scale(const ctx_t* c, const float* ra, const float* rb) {
  float A = 0.0f;
#pragma omp parallel for num_threads(g_threads) schedule(static) reduction(max : A)
  for (int64_t i = 0; i < c->m; i++)
    for (int64_t j = 0; j < c->n; j++)
      A = fmaxf(A, fabsf(fl32_mul(fl32_mul(w_at(c, i, j), rb[j]), ra[i])));
  if (A == 0.0f) return 1.0f;
  float g = fl32_div(A, 2688.0f);
  return g < 0x1p-126f ? 0x1p-126f : g;
}

static void emit(const ctx_t* c, const int8_t* q2, const uint16_t* sc, uint8_t* codes,
                 void* scales) {
  const int64_t m = c->m, n = c->n, ng = c->ng;
  for (int64_t i = 0; i < m; i++) {
    for (int64_t j = 0; j < n; j += 2) {
      uint8_t nib[2];
      for (int h = 0; h < 2; h++) {
        int v2 = q2[i * n + j + h];
        if (c->fmt == DQR_FMT_INT4_BF16 || c->fmt == DQR_FMT_MXINT4) {
          nib[h] = (uint8_t)((v2 / 2) & 0xF); /* two's complement nibble */
        } else {
          double mag = fabs(0.5 * v2);
          int idx = 0;
          while (E2M1_GRID[idx] != mag) idx++;
          nib[h] = (uint8_t)((v2 < 0 ? 8 : 0) | idx);
        }
      }
      codes[(i * n + j) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
    for (int64_t gi = 0; gi < ng; gi++) {
      if (c->fmt == DQR_FMT_INT4_BF16)
        ((uint16_t*)scales)[i * ng + gi] = sc[i * ng + gi];
      else
        ((uint8_t*)scales)[i * ng + gi] = (uint8_t)sc[i * ng + gi];
    }
  }
}

/* ------------------------------------------------------------------ public: one Q pass */

int dq_ref_quantize(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group,
                    const float* a, const float* b, float* g_inout, uint8_t* codes,
                    void* scales) {
  int st = check_common(W, wt, rows, cols, fmt, group);
  if (st) return st;
  if (!codes || !scales || (fmt == DQR_FMT_NVFP4 && !g_inout)) return DQR_ERR_ARG;
  if ((a && !positive_finite(a, rows)) || (b && !positive_finite(b, cols))) return DQR_ERR_ARG;
  if (fmt == DQR_FMT_NVFP4 && (isnan(*g_inout) || isinf(*g_inout))) return DQR_ERR_ARG;
  ctx_t c = {W, wt, rows, cols, fmt, group, cols / group, 1.0f, 6.0f};
  if (!w_finite(&c)) return DQR_ERR_NONFINITE;
  float* ra = malloc(sizeof(float) * rows);
  float* rb = malloc(sizeof(float) * cols);
  int8_t* q2 = malloc((size_t)(rows * cols));
  double* dv = malloc(sizeof(double) * rows * c.ng);
  uint16_t* sc = malloc(sizeof(uint16_t) * rows * c.ng);
  if (!ra || !rb || !q2 || !dv || !sc) {
    st = DQR_ERR_INTERNAL;
    goto done;
  }
  for (int64_t i = 0; i < rows; i++) ra[i] = a ? (float)(1.0 / (double)a[i]) : 1.0f;
  for (int64_t j = 0; j < cols; j++) rb[j] = b ? (float)(1.0 / (double)b[j]) : 1.0f;
  if (fmt == DQR_FMT_NVFP4) {
    if (!(*g_inout > 0.0f)) *g_inout = tensor_scale(&c, ra, rb);
    if (!isfinite(*g_inout)) {
      st = DQR_ERR_RANGE;
      goto done;
    }
    c.g = *g_inout;
    c.sixg = fl32_mul(6.0f, c.g);
  }
  st = q_pass(&c, ra, rb, q2, dv, sc);
  if (st == DQR_OK) emit(&c, q2, sc, codes, scales);
done:
  free(ra);
  free(rb);
  free(q2);
  free(dv);
  free(sc);
  return st;
}

/* ------------------------------------------------- public: activation quantization */

/* The consumer side of the factorized product (daiwk notes, "核心公式" eq. 1: X W^T ~=
 * (X D_beta^-1) Qhat^T D_alpha^-1 with D_beta^-1 = D_b; the flowchart's step that scales the
 * real activations by the column inverse scales before quantizing them): every activation
 * row is scaled channel by channel, x_tj = fl32(X_tj * b_j), and quantized by the same group
 * quantizer Q as the weights, in groups of `group` consecutive channels (reading: one
 * quantizer per format for weights and activations, as in the W+A rows of the pages'
 * Table 1). NVFP4: g as for the weights, from max |x| of this tensor unless given. */
int dq_ref_quantize_act(const void* X, int xt, int64_t tokens, int64_t cols, int fmt, int group,
                        const float* b, float* g_inout, uint8_t* codes, void* scales) {
  int st = check_common(X, xt, tokens, cols, fmt, group);
  if (st) return st;
  if (!codes || !scales || (fmt == DQR_FMT_NVFP4 && !g_inout)) return DQR_ERR_ARG;
  if (b && !positive_finite(b, cols)) return DQR_ERR_ARG;
  if (fmt == DQR_FMT_NVFP4 && (isnan(*g_inout) || isinf(*g_inout))) return DQR_ERR_ARG;
  ctx_t c = {X, xt, tokens, cols, fmt, group, cols / group, 1.0f, 6.0f};
  if (!w_finite(&c)) return DQR_ERR_NONFINITE;
  const int64_t n = cols, ng = c.ng;
  float* x = malloc(sizeof(float) * (size_t)(tokens * n));
  int8_t* q2 = malloc((size_t)(tokens * n));
  double* dv = malloc(sizeof(double) * (size_t)(tokens * ng));
  uint16_t* sc = malloc(sizeof(uint16_t) * (size_t)(tokens * ng));
  if (!x || !q2 || !dv || !sc) {
    st = DQR_ERR_INTERNAL;
    goto done;
  }
  float A = 0.0f;
  for (int64_t t = 0; t < tokens; t++)
    for (int64_t j = 0; j < n; j++) {
      const float v = fl32_mul(w_at(&c, t, j), b ? b[j] : 1.0f);
      if (!isfinite(v)) {
        st = DQR_ERR_RANGE;
        goto done;
      }
      x[t * n + j] = v;
      A = fmaxf(A, fabsf(v));
    }
  if (fmt == DQR_FMT_NVFP4) {
    if (!(*g_inout > 0.0f)) {
      float g = A == 0.0f ? 1.0f : fl32_div(A, 2688.0f);
      *g_inout = g < 0x1p-126f ? 0x1p-126f : g;
    }
    c.g = *g_inout;
    c.sixg = fl32_mul(6.0f, c.g);
  }
  for (int64_t t = 0; t < tokens; t++)
    for (int64_t gi = 0; gi < ng; gi++)
      quant_group(&c, x + t * n + gi * group, q2 + t * n + gi * group, dv + t * ng + gi,
                  sc + t * ng + gi);
  emit(&c, q2, sc, codes, scales);
done:
  free(x);
  free(q2);
  free(dv);
  free(sc);
  return st;
}

/* --------------------------------------------------------- public: the W4A4 product */

/* The product the quantized weights serve (daiwk notes, "核心公式" eq. 1: X W^T ~=
 * (X D_beta^-1) Qhat^T D_alpha^-1 = (X D_b) Qhat^T D_a; the flowchart's last step: the matmul
 * of the quantized activations with the weight codes, then the row output scale): with
 * MXFP4 activations x^ = Q(X D_b) (tokens x K) and weights Qhat = codes * 2^(e) (out x K),
 * Y[t][i] = a_i * sum_k x^[t][k] Qhat[i][k], summed in double in ascending k. An E8M0 byte
 * 0xFF is the format's NaN (OCP MX v1.0, E8M0) and makes its block's terms NaN. */
static double e8m0_value(uint8_t s) { return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127); }

int dq_ref_gemm_mx(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                   int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int64_t out,
                   const float* a, double* Y) {
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y) return DQR_ERR_ARG;
  if (tokens <= 0 || out <= 0 || K <= 0 || K % 32 != 0) return DQR_ERR_ARG;
  if (a && !positive_finite(a, out)) return DQR_ERR_ARG;
  const int64_t kb = K / 32;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t t = 0; t < tokens; t++) {
    for (int64_t i = 0; i < out; i++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        const uint8_t cx = act_codes[(t * K + k) / 2], cw = w_codes[(i * K + k) / 2];
        const int nx = (k & 1) ? (cx >> 4) : (cx & 0xF), nw = (k & 1) ? (cw >> 4) : (cw & 0xF);
        const double vx = (nx & 8 ? -1.0 : 1.0) * E2M1_GRID[nx & 7];
        const double vw = (nw & 8 ? -1.0 : 1.0) * E2M1_GRID[nw & 7];
        acc += vx * e8m0_value(act_scales[t * kb + k / 32]) * vw * e8m0_value(w_scales[i * kb + k / 32]);
      }
      Y[t * out + i] = acc * (a ? (double)a[i] : 1.0);
    }
  }
  return DQR_OK;
}

/* ----------------------------------------------------------------- public: the solver */

/* NVFP4 with a per-pass tensor scale: g from the scaled tile about to be quantized */
static int set_pass_g(ctx_t* c, const float* ra, const float* rb) {
  c->g = tensor_scale(c, ra, rb);
  if (!isfinite(c->g)) return DQR_ERR_RANGE;
  c->sixg = fl32_mul(6.0f, c->g);
  return DQR_OK;
}

static int solve_core(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group,
                      int T, const float* a0, const float* b0, float g0, int per_pass,
                      uint8_t* codes, void* scales, float* g_out, float* a, float* b,
                      double* mse, int64_t* changes, double* margin) {
  int st = check_common(W, wt, rows, cols, fmt, group);
  if (st) return st;
  if (T < 0 || !codes || !scales || !a || !b || !mse || (fmt == DQR_FMT_NVFP4 && !g_out))
    return DQR_ERR_ARG;
  if ((a0 && !positive_finite(a0, rows)) || (b0 && !positive_finite(b0, cols)))
    return DQR_ERR_ARG;
  if (isnan(g0) || (g0 > 0.0f && !isfinite(g0))) return DQR_ERR_ARG;

  const int64_t m = rows, n = cols;
  ctx_t c = {W, wt, m, n, fmt, group, n / group, 1.0f, 6.0f};
  if (!w_finite(&c)) return DQR_ERR_NONFINITE;
  e4m3_table_init(); /* before any parallel region reads it */

  float* ra = malloc(sizeof(float) * m);
  float* rb = malloc(sizeof(float) * n);
  int8_t* qA = malloc((size_t)(m * n));
  int8_t* qB = malloc((size_t)(m * n));
  double* dA = malloc(sizeof(double) * m * c.ng);
  double* dB = malloc(sizeof(double) * m * c.ng);
  uint16_t* sA = malloc(sizeof(uint16_t) * m * c.ng);
  uint16_t* sB = malloc(sizeof(uint16_t) * m * c.ng);
  double* row_err = malloc(sizeof(double) * m);
  double* Nc = malloc(sizeof(double) * n);
  double* Dc = malloc(sizeof(double) * n);
  double* mrow = malloc(sizeof(double) * m);
  if (!ra || !rb || !qA || !qB || !dA || !dB || !sA || !sB || !row_err || !Nc || !Dc || !mrow) {
    st = DQR_ERR_INTERNAL;
    goto done;
  }

  /* step 0: initial outer scales, projected onto the scale set (ones by default) */
  for (int64_t i = 0; i < m; i++) a[i] = a0 ? (float)dq_ref_project(fmt, a0[i]) : 1.0f;
  for (int64_t j = 0; j < n; j++) b[j] = b0 ? (float)dq_ref_project(fmt, b0[j]) : 1.0f;
  fill_reciprocals(a, ra, m); /* inner copies synced: alpha = 1/a, beta = 1/b */
  fill_reciprocals(b, rb, n);
  if (fmt == DQR_FMT_NVFP4) {
    c.g = g0 > 0.0f ? g0 : tensor_scale(&c, ra, rb);
    if (!isfinite(c.g)) {
      st = DQR_ERR_RANGE;
      goto done;
    }
    c.sixg = fl32_mul(6.0f, c.g);
    *g_out = c.g;
  }

  for (int t = 0; t < T; t++) {
    /* 1-2: quantize the synced state, record its error */
    if (per_pass && (st = set_pass_g(&c, ra, rb))) goto done;
    if ((st = q_pass(&c, ra, rb, qA, dA, sA))) goto done;
    mse[t] = mse_of(&c, a, b, qA, dA, row_err);
    if (changes && t > 0) {
      changes[4 * (t - 1) + 2] = count_diff_i8(qB, qA, m * n);
      changes[4 * (t - 1) + 3] = count_diff_u16(sB, sA, m * c.ng);
    }

    /* 3: row update with codes fixed, R = Qhat D_b (eq. 2, left) */
    int internal = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static) reduction(| : internal)
    for (int64_t i = 0; i < m; i++) {
      double N = 0.0, D = 0.0;
      for (int64_t j = 0; j < n; j++) {
        double R = dA[i * c.ng + j / group] * (0.5 * qA[i * n + j]) * (double)b[j];
        N += (double)w_at(&c, i, j) * R;
        D += R * R;
      }
      mrow[i] = INFINITY;
      if (D == 0.0) {
        a[i] = 1.0f; /* all-zero code slice: scale 1 */
      } else {
        if (!(N > 0.0)) internal = 1; /* every W*R term is >= 0 */
        a[i] = (float)dq_ref_project(fmt, N / D);
        mrow[i] = dq_ref_proj_margin(fmt, N / D);
      }
    }
    if (internal) {
      st = DQR_ERR_INTERNAL;
      goto done;
    }
    if (margin) {
      double mm = INFINITY;
      for (int64_t i = 0; i < m; i++) mm = fmin(mm, mrow[i]);
      margin[2 * t] = mm;
    }
    fill_reciprocals(a, ra, m);

    /* 4: re-quantize with the synced inner copy of the new a */
    if (per_pass && (st = set_pass_g(&c, ra, rb))) goto done;
    if ((st = q_pass(&c, ra, rb, qB, dB, sB))) goto done;
    if (changes) {
      changes[4 * t + 0] = count_diff_i8(qA, qB, m * n);
      changes[4 * t + 1] = count_diff_u16(sA, sB, m * c.ng);
    }

    /* 5: column update with codes fixed, S = D_a Qhat (eq. 2, right); each column's
     * sums run over rows in ascending order. The blocks of 256 columns only hand the columns
     * out to threads: every column's two sums are the same fp64 additions, in the same order,
     * as the plain loop over i for that j. */
    const int64_t JB = 256;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t j0 = 0; j0 < n; j0 += JB) {
      int64_t j1 = j0 + JB < n ? j0 + JB : n;
      for (int64_t j = j0; j < j1; j++) Nc[j] = Dc[j] = 0.0;
      for (int64_t i = 0; i < m; i++) {
        for (int64_t j = j0; j < j1; j++) {
          double S = (double)a[i] * dB[i * c.ng + j / group] * (0.5 * qB[i * n + j]);
          Nc[j] += (double)w_at(&c, i, j) * S;
          Dc[j] += S * S;
        }
      }
    }
    double mcol = INFINITY;
    for (int64_t j = 0; j < n; j++) {
      if (Dc[j] == 0.0) {
        b[j] = 1.0f;
      } else {
        if (!(Nc[j] > 0.0)) {
          st = DQR_ERR_INTERNAL;
          goto done;
        }
        b[j] = (float)dq_ref_project(fmt, Nc[j] / Dc[j]);
        if (margin) mcol = fmin(mcol, dq_ref_proj_margin(fmt, Nc[j] / Dc[j]));
      }
    }
    if (margin) margin[2 * t + 1] = mcol;
    fill_reciprocals(b, rb, n);
  }

  /* final synced state: codes, inner scales and its error */
  if (per_pass) {
    if ((st = set_pass_g(&c, ra, rb))) goto done;
    *g_out = c.g;
  }
  if ((st = q_pass(&c, ra, rb, qA, dA, sA))) goto done;
  mse[T] = mse_of(&c, a, b, qA, dA, row_err);
  if (changes && T > 0) {
    changes[4 * (T - 1) + 2] = count_diff_i8(qB, qA, m * n);
    changes[4 * (T - 1) + 3] = count_diff_u16(sB, sA, m * c.ng);
  }
  emit(&c, qA, sA, codes, scales);

done:
  free(ra);
  free(rb);
  free(qA);
  free(qB);
  free(dA);
  free(dB);
  free(sA);
  free(sB);
  free(row_err);
  free(Nc);
  free(Dc);
  free(mrow);
  return st;
}

int dq_ref_solve_diag(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group,
                      int T, const float* a0, const float* b0, float g0, uint8_t* codes,
                      void* scales, float* g_out, float* a, float* b, double* mse,
                      int64_t* changes, double* margin) {
  return solve_core(W, wt, rows, cols, fmt, group, T, a0, b0, g0, 0, codes, scales, g_out, a,
                    b, mse, changes, margin);
}

/* NVFP4 with the tensor scale recomputed before every Q pass (reading of the pages'
 * black-box quantizer applied to each scaled tile as it stands; the per-tensor scale is not
 * on the pages): g = fl32(max|X| / 2688) of the tile about to be quantized, for the synced
 * state, the re-quantization after the row update and the final pass alike. */
int dq_ref_solve_pass_g(const void* W, int wt, int64_t rows, int64_t cols, int group, int T,
                        const float* a0, const float* b0, uint8_t* codes, void* scales,
                        float* g_out, float* a, float* b, double* mse) {
  return solve_core(W, wt, rows, cols, DQR_FMT_NVFP4, group, T, a0, b0, 0.0f, 1, codes, scales,
                    g_out, a, b, mse, NULL, NULL);
}

int dq_ref_solve(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group, int T,
                 const float* a0, const float* b0, float g0, uint8_t* codes, void* scales,
                 float* g_out, float* a, float* b, double* mse) {
  return dq_ref_solve_diag(W, wt, rows, cols, fmt, group, T, a0, b0, g0, codes, scales, g_out,
                           a, b, mse, NULL, NULL);
}
