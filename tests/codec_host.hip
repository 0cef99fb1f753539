// Host-side build of the HIP library's codec header, so that its rounding, projection and
// per-group quantizer functions can be checked exhaustively on the CPU (tests/test_device_codecs.py).
// No kernel is launched from here.
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
