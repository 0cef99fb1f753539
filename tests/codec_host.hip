// Host-side build of the HIP library's codec header, so that its rounding, projection and
// per-group quantizer functions can be checked exhaustively on the CPU (tests/test_device_codecs.py).
// No kernel is launched from here.
#include <float.h>
#include <stdint.h>

#include "../dual_scale_w4a4_amd/csrc/dq_device.h"

extern "C" {

void h_bf16_rne(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::bf16_rne(x[i]);
}
void h_e4m3_rne_sat(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::e4m3_rne_sat(x[i]);
}
void h_e4m3_bits(const float* x, uint32_t* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::e4m3_bits(x[i]);
}
void h_e2m1_mag(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::e2m1_mag(x[i]);
}
void h_project(int fmt, const double* v, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::project(fmt, v[i]);
}
void h_recip32(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = dq::recip32(x[i]);
}

}  // extern "C"

// Q on already-scaled values X (rows x cols, groups of G along a row), exactly as a sweep
// does it per group: codes (signed values) and stored scale encodings.
template <int FMT>
static void quant(const float* X, int64_t rows, int64_t cols, int G, float g, float* q,
                  uint32_t* scode) {
  const float sixg = 6.0f * g;
  for (int64_t i = 0; i < rows; i++)
    for (int64_t k = 0; k < cols / G; k++) {
      const float* x = X + i * cols + k * G;
      float mx = 0.0f;
      for (int j = 0; j < G; j++) mx = fmaxf(mx, fabsf(x[j]));
      const dq::GroupQ gq = dq::group_scale<FMT>(mx, g, sixg);
      for (int j = 0; j < G; j++) q[i * cols + k * G + j] = dq::code_of<FMT>(x[j], gq);
      scode[i * (cols / G) + k] = gq.scode;
    }
}

extern "C" void h_quantize(int fmt, const float* X, int64_t rows, int64_t cols, int G, float g, float* q,
                uint32_t* scode) {
  switch (fmt) {
    case 0: quant<0>(X, rows, cols, G, g, q, scode); break;
    case 1: quant<1>(X, rows, cols, G, g, q, scode); break;
    case 2: quant<2>(X, rows, cols, G, g, q, scode); break;
    default: quant<3>(X, rows, cols, G, g, q, scode); break;
  }
}

// div7(m) against the correctly rounded quotient fl32(m / 7) (a double quotient of two
// floats rounds innocuously to float) for every m with the biased exponents in [e0, e1]
// (0 covers the subnormals); returns the number of mismatches.
extern "C" int64_t h_div7_mismatches(int e0, int e1) {
  int64_t bad = 0;
  for (uint32_t e = (uint32_t)e0; e <= (uint32_t)e1; e++)
    for (uint32_t f = 0; f < (1u << 23); f++) {
      const float m = dq::u2f((e << 23) | f);
      if (dq::div7(m) != (float)((double)m / 7.0)) bad++;
    }
  return bad;
}

// rne_quotient_int at and around every tie (k + 1/2) d of the given divisors, with the
// reciprocal perturbed by up to +-3 ulp (the device's reciprocal is not correctly rounded),
// against the nearest integer of the double quotient (which decides every non-tie exactly
// and is exact at ties), clamped like an INT4 code; returns the number of mismatches.
extern "C" int64_t h_rne_quotient_mismatches(const float* d, int64_t nd) {
  int64_t bad = 0;
  for (int64_t t = 0; t < nd; t++) {
    const float dv = d[t];
    for (int k = -10; k <= 9; k++) {
      const float x0 = ((float)k + 0.5f) * dv;  // exact: few significant bits
      float xs[9];
      xs[0] = x0;
      float up = x0, dn = x0;
      for (int s = 1; s <= 4; s++) {
        up = nextafterf(up, INFINITY);
        dn = nextafterf(dn, -INFINITY);
        xs[2 * s - 1] = up;
        xs[2 * s] = dn;
      }
      for (int ix = 0; ix < 9; ix++) {
        const float x = xs[ix];
        const double ref = nearbyint((double)x / (double)dv);
        // the quantizer's rescale of tiny divisors (exact: a power of two)
        const float sc = dv < 0x1p-100f ? 0x1p32f : 1.0f;
        const float ds = dv * sc;
        float rd = 1.0f / ds;
        for (int s = 0; s < 3; s++) rd = nextafterf(rd, -INFINITY);
        for (int s = -3; s <= 3; s++) {
          const float got = dq::rne_quotient_int(x * sc, ds, 0.5f * ds, rd);
          if ((double)got != ref) bad++;
          rd = nextafterf(rd, INFINITY);
        }
      }
    }
  }
  return bad;
}

// code64 against the oracle-style reference (nearest of the double quotient, which is exact
// away from ties and exact at ties) at and around every rounding boundary of the given
// divisors, with the reciprocal perturbed by up to +-2^-48 relative (the device's reciprocal
// is an estimate refined by Newton steps); fmt 0 = INT4 (boundaries k + 1/2), 3 = E2M1
// (boundaries 1/4, 3/4, ..., 5, and saturation); returns the number of mismatches.
static double ref_e2m1(double v) {  // nearest E2M1 magnitude, ties to the even index
  static const double g[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
  int best = 0;
  for (int i = 1; i < 8; i++) {
    const double db = fabs(v - g[best]), di = fabs(v - g[i]);
    if (di < db || (di == db && (i % 2) == 0)) best = i;
  }
  return g[best];
}

extern "C" int64_t h_code64_mismatches(int fmt, const float* d, int64_t nd) {
  static const double e2m1_b[8] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5};
  int64_t bad = 0;
  dq::GroupQ gq{};
  for (int64_t t = 0; t < nd; t++) {
    const float dv = d[t];
    const int nb = fmt == 0 ? 20 : 16;
    for (int b = 0; b < nb; b++) {
      double h;
      if (fmt == 0) h = (double)(b - 10) + 0.5;
      else h = (b < 8 ? 1.0 : -1.0) * e2m1_b[b % 8];
      const float x0 = (float)(h * (double)dv);  // the nearest float to the boundary
      float xs[11];
      xs[0] = x0;
      float up = x0, dn = x0;
      for (int s = 1; s <= 5; s++) {
        up = nextafterf(up, INFINITY);
        dn = nextafterf(dn, -INFINITY);
        xs[2 * s - 1] = up;
        xs[2 * s] = dn;
      }
      for (int ix = 0; ix < 11; ix++) {
        const float x = xs[ix];
        const double qd = (double)x / (double)dv;
        double ref;
        if (fmt == 0) {
          ref = nearbyint(qd);
          ref = ref < -8.0 ? -8.0 : (ref > 7.0 ? 7.0 : ref);
        } else {
          ref = ref_e2m1(fabs(qd));
          if (x < 0.0f) ref = -ref;
        }
        for (int s = -2; s <= 2; s++) {
          const double r = (1.0 / (double)dv) * (1.0 + (double)s * 0x1p-49);
          const double got = fmt == 0 ? dq::code64<0>(x, r, gq) : dq::code64<3>(x, r, gq);
          if (got != ref && !(fmt == 0 && fabs(qd) >= 7.5)) bad++;  // Q keeps |x / s| <= 7.03
        }
      }
    }
  }
  return bad;
}

// nv_odd_quotient followed by rounding onto E2M1 (e2m1_mag, as the hardware conversion with
// scale 1 rounds), against the code of the exact quotient, at and 1..5 fp32 steps around every
// E2M1 decision point, at quotients 0, 6, 7.99, 8, 9, 100 and 10^6, and at |x| = 10^38 and the
// largest float (whose product with 1 / d overflows for small d), all with both signs, with
// the reciprocal at, and one ulp either side of, the correctly rounded 1 / d (the device
// takes v_rcp_f32, within one ulp); for divisors in [2^-100, 2^100]. Returns the mismatch
// count.
extern "C" int64_t h_nv_odd_mismatches(const float* d, int64_t nd) {
  static const double pts[14] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                                 0.0,  6.0,  7.99, 8.0,  9.0, 100.0, 1e6};
  int64_t bad = 0;
  for (int64_t t = 0; t < nd; t++) {
    const float dv = d[t];
    const float rd0 = (float)(1.0 / (double)dv);
    const float rds[3] = {rd0, nextafterf(rd0, INFINITY), nextafterf(rd0, 0.0f)};
    for (int b = 0; b < 28; b++) {
      const double h = (b < 14 ? 1.0 : -1.0) * pts[b % 14];
      const float x0 = (float)(h * (double)dv);
      float xs[11];
      xs[0] = x0;
      float up = x0, dn = x0;
      for (int k = 1; k <= 5; k++) {
        up = nextafterf(up, INFINITY);
        dn = nextafterf(dn, -INFINITY);
        xs[2 * k - 1] = up;
        xs[2 * k] = dn;
      }
      for (int ix = 0; ix < 11; ix++) {
        const float x = xs[ix];
        const double qd = (double)x / (double)dv;
        const double ref = qd < 0.0 ? -ref_e2m1(-qd) : ref_e2m1(qd);
        for (int r = 0; r < 3; r++) {
          const float z = dq::nv_odd_quotient(x, dv, rds[r], 8.0f * dv);
          const float m = dq::e2m1_mag(fabsf(z));
          const double got = z < 0.0f ? -(double)m : (double)m;
          if (got != ref) bad++;
        }
      }
    }
    const float big[4] = {1e38f, -1e38f, FLT_MAX, -FLT_MAX};
    for (int k = 0; k < 4; k++)
      for (int r = 0; r < 3; r++) {
        const float z = dq::nv_odd_quotient(big[k], dv, rds[r], 8.0f * dv);
        const float m = dq::e2m1_mag(fabsf(z));
        if ((z < 0.0f ? -(double)m : (double)m) != (big[k] < 0.0f ? -6.0 : 6.0)) bad++;
      }
  }
  return bad;
}

// Q of one group through the double-quotient codes (code64), as the two-sweep pass and the
// activation quantizer form them: values q (one per element) and the scale code.
extern "C" void h_group_code64(int fmt, const float* x, int G, float g, double* q, uint32_t* scode) {
  float mx = 0.0f;
  for (int k = 0; k < G; k++) mx = fmaxf(mx, fabsf(x[k]));
  const float sixg = 6.0f * g;
  switch (fmt) {
    case 0: {
      const dq::GroupQ gq = dq::group_scale<0>(mx, g, sixg);
      const double r = dq::recip64(gq.d);
      for (int k = 0; k < G; k++) {
        q[k] = dq::code64<0>(x[k], r, gq);
        if (dq::int4_needs_clamp(gq.d)) q[k] = dq::int4_clamp(q[k]);
      }
      *scode = gq.scode;
      break;
    }
    default: {
      const dq::GroupQ gq = dq::group_scale<3>(mx, g, sixg);
      const double r = dq::recip64(gq.d);
      for (int k = 0; k < G; k++) q[k] = dq::code64<3>(x[k], r, gq);
      *scode = gq.scode;
      break;
    }
  }
}
