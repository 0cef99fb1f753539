// dq_device.h -- device-side format codecs and wavefront helpers for the gfx950 solver
// kernels. Every rounding step here is chosen to give exactly the IEEE result the method's
// arithmetic names (one binary32 rounding per "fl32" step, exact quotients for codes), so
// that a single Q pass is bit-identical to an exact-arithmetic evaluation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dq_internal.h"

namespace dq {

constexpr int kWave = 64;
constexpr int kEpl = 8;                 // weight elements per lane per row
constexpr int kTileCols = kWave * kEpl;  // 512 columns per wave-row
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kBlock = kWave * kWaves;

// Codec functions compile for both host and device, so that they can be checked
// exhaustively on the CPU; the cross-lane helpers at the end are device-only.
#define DQ_HD __host__ __device__ __forceinline__

DQ_HD float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
DQ_HD uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
DQ_HD double u2d(unsigned long long u) { return __builtin_bit_cast(double, u); }
DQ_HD unsigned long long d2u(double d) { return __builtin_bit_cast(unsigned long long, d); }

// 2^e as a float for e in [-126, 127]
DQ_HD float exp2i(int e) { return u2f((uint32_t)(e + 127) << 23); }

// ----------------------------------------------------------------------------- rounding

// nearest bf16 value (as float) of a finite non-negative float, ties to even; the bit
// trick is exact for subnormals too because their spacing is uniform
DQ_HD float bf16_rne(float x) {
  uint32_t u = f2u(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u2f(u & 0xFFFF0000u);
}

// nearest E4M3FN value of a finite non-negative float, ties to even, saturating at 448
DQ_HD float e4m3_rne_sat(float u) {
  if (u >= 448.0f) return 448.0f;
  if (u < 0x1p-6f) return rintf(u * 512.0f) * 0x1p-9f;  // subnormal grid, exact scaling
  uint32_t b = f2u(u);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // keep 3 of 23 mantissa bits
  float r = u2f(b & 0xFFF00000u);
  return r > 448.0f ? 448.0f : r;
}

// E4M3FN bits of an exact positive E4M3 value
DQ_HD uint32_t e4m3_bits(float s) {
  if (s < 0x1p-6f) return (uint32_t)(s * 512.0f);
  uint32_t u = f2u(s);
  uint32_t e = ((u >> 23) & 0xFFu) - 127u + 7u;
  return (e << 3) | ((u >> 20) & 7u);
}

// E2M1 magnitude nearest to v in [0, 8), ties to the even index: adding
// C = 2^22 * max(1, 2^floor(log2 v)) makes the fp32 ulp at C equal to the E2M1 spacing of
// v's binade (0.5 below 2, then 1, then 2), so (v + C) - C rounds v to that grid with the
// adder's round-to-nearest-even; the even significand is the even E2M1 index.
DQ_HD float e2m1_mag(float v) {
  uint32_t base = f2u(v) & 0x7F800000u;
  base = base > 0x3F800000u ? base : 0x3F800000u;
  float c = u2f(base + (22u << 23));
  float r = (v + c) - c;
  return fminf(r, 6.0f);
}

// magnitude index 0..7 of an E2M1 magnitude
DQ_HD uint32_t e2m1_index(float r) {
  // 0,.5,1,1.5 -> 2r ; 2,3 -> r + 2 ; 4,6 -> r/2 + 4
  float k = r < 2.0f ? 2.0f * r : (r < 4.0f ? r + 2.0f : 0.5f * r + 4.0f);
  return (uint32_t)k;
}

// nearest integer to the exact quotient x / d (d > 0, |x / d| < 16), ties to even, from an
// approximate reciprocal rd (a few ulp from 1 / d). k = rint(x rd) is at most one off, so
// e = x - k d is exactly representable and the fused multiply-add returns it exactly: |e| >
// d / 2 moves k one step towards e, and |e| = d / 2 is a tie, settled by the hardware's
// round-to-nearest-even of the exact half-integer k +- 1/2.
DQ_HD float rne_quotient_int(float x, float d, float hd, float rd) {
  const float k = rintf(x * rd);
  const float e = fmaf(-k, d, x);
  const float ae = fabsf(e);
  const float adj = ae > hd ? 1.0f : (ae == hd ? 0.5f : 0.0f);
  return rintf(k + copysignf(adj, e));
}

// nearest E2M1 magnitude to the exact quotient ax / d (ax >= 0, d > 0, rd ~ 1/d). The caller
// rescales ax and d by the same power of two when d is tiny, so that the fused multiply-adds
// below cannot underflow. The candidate from ax * rd is at most one grid step off; the exact
// signs of ax - t d at the two neighbouring midpoints t settle the step and any tie.
DQ_HD float e2m1_quotient(float ax, float d, float rd) {
  float r = e2m1_mag(fminf(ax * rd, 8.0f));
  float qa = r < 2.0f ? 0.5f : (r < 4.0f ? 1.0f : 2.0f);   // step to the next value
  float qb = r <= 2.0f ? 0.5f : (r <= 4.0f ? 1.0f : 2.0f);  // step to the previous value
  float dh = fmaf(-(r + 0.5f * qa), d, ax);
  float dl = fmaf(-(r - 0.5f * qb), d, ax);
  bool odd = (e2m1_index(r) & 1u) != 0;
  if (r < 6.0f && (dh > 0.0f || (dh == 0.0f && odd))) return r + qa;
  if (r > 0.0f && (dl < 0.0f || (dl == 0.0f && odd))) return r - qb;
  return r;
}

// ------------------------------------------------------------- projections of outer scales
// Pi_F: the value of the format's scale set nearest to v > 0 (v computed in fp64).

DQ_HD float proj_bf16(double v) {
  if (!(v > 0x1p-126)) return 0x1p-126f;
  unsigned long long u = d2u(v);
  u += 0xFFFFFFFFFFFull + ((u >> 45) & 1ull);  // keep 7 of 52 mantissa bits, ties to even
  u &= ~0x1FFFFFFFFFFFull;
  double r = u2d(u);
  const double mx = 0x1.FEp127;
  return r > mx ? (float)mx : (float)r;
}

DQ_HD float proj_e8m0(double v) {
  unsigned long long u = d2u(v);
  u += 1ull << 51;  // a mantissa >= 1/2 (v >= 1.5 * 2^k) carries into the exponent
  int e = (int)((u >> 52) & 0x7FFull) - 1023;
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  return exp2i(e);
}

DQ_HD float proj_e4m3(double v) {
  double r;
  if (v >= 448.0) {
    r = 448.0;
  } else if (v < 0x1p-6) {
    r = rint(v * 512.0) * 0x1p-9;
  } else {
    unsigned long long u = d2u(v);
    u += ((1ull << 48) - 1ull) + ((u >> 49) & 1ull);  // keep 3 mantissa bits
    u &= ~((1ull << 49) - 1ull);
    r = u2d(u);
    if (r > 448.0) r = 448.0;
  }
  if (r < 0x1p-9) r = 0x1p-9;
  return (float)r;
}

DQ_HD float project(int fmt, double v) {
  if (fmt == kInt4Bf16) return proj_bf16(v);
  if (fmt == kNvFp4) return proj_e4m3(v);
  return proj_e8m0(v);
}

// fl32(1/v), correctly rounded (double quotient rounds innocuously to float)
DQ_HD float recip32(float v) { return (float)(1.0 / (double)v); }

// fl32(m / 7) for finite m >= 0 with one double product. If 7 divides m's integer
// significand the quotient is a float; otherwise its significand (or its subnormal multiple
// of 2^-149) has a fractional part k / 7, k in 1..6, at least 1/14 of a unit from the
// rounding midpoint, while the product is within 2^-52 (relative) of m / 7: both round alike.
DQ_HD float div7(float m) { return (float)((double)m * (1.0 / 7.0)); }

// an approximate reciprocal (within a few ulp) of a positive normal float whose reciprocal
// is normal; only used to find a candidate that an exact fix-up step then corrects
DQ_HD float approx_recip(float v) {
#ifdef __HIP_DEVICE_COMPILE__
  return __builtin_amdgcn_rcpf(v);
#else
  return 1.0f / v;
#endif
}

// ------------------------------------------------------------------- the group quantizer Q

// Per-group quantizer state: divisor d, the operand rescale sc for tiny divisors (a power of
// two; sc = 1 otherwise) with the rescaled divisor ds = d sc, half of it hds and an
// approximate reciprocal rd ~ 1 / ds, and the stored scale encoding.
struct GroupQ {
  float d;
  float rd;
  float sc;
  float ds;
  float hds;
  uint32_t scode;
};

// Q's inner-scale rule for one group with absmax mx (finite):
//   INT4_BF16: s = max(bf16(fl32(mx / 7)), 2^-133), d = s
//   MXINT4 / MXFP4: d = 2^clamp(floor(log2 mx) - 2, -126, 126) (OCP shared exponent, E2M1 and
//              INT4-as-1.2-fixed-point both have emax 2 relative to the integer code)
//   NVFP4: u = fl32(mx / fl32(6 g)), s = max(E4M3(u), 2^-9), d = fl32(s g)
// An all-zero group takes s = 1 (E8M0 exponent 0).
template <int FMT>
DQ_HD GroupQ group_scale(float mx, float g, float sixg) {
  GroupQ r;
  r.sc = 1.0f;
  if (FMT == kInt4Bf16) {
    float s = 1.0f;
    if (mx > 0.0f) s = fmaxf(bf16_rne(div7(mx)), 0x1p-133f);
    r.d = s;
    r.scode = f2u(s) >> 16;
    if (s < 0x1p-100f) r.sc = 0x1p32f;
    r.ds = s * r.sc;
    r.hds = 0.5f * r.ds;
    r.rd = approx_recip(r.ds);
  } else if (FMT == kMxInt4 || FMT == kMxFp4) {
    int e = 0;
    if (mx > 0.0f) {
      int ef = (int)((f2u(mx) >> 23) & 0xFFu);  // 0 for subnormal mx: clamps to -126 below
      e = ef - 129;
      e = e < -126 ? -126 : e;  // ef <= 254 keeps e <= 125
    }
    r.d = exp2i(e);
    r.rd = exp2i(-e);
    r.ds = r.d;
    r.hds = 0.5f * r.d;
    r.scode = (uint32_t)(e + 127);
  } else {
    float s = 1.0f;
    if (mx > 0.0f) s = fmaxf(e4m3_rne_sat((float)((double)mx / (double)sixg)), 0x1p-9f);
    r.d = s * g;
    r.scode = e4m3_bits(s);
    if (r.d < 0x1p-100f) r.sc = 0x1p32f;
    r.ds = r.d * r.sc;
    r.hds = 0.5f * r.ds;
    r.rd = (float)(1.0 / (double)r.ds);
  }
  return r;
}

// the signed code value of x (a float holding the integer or E2M1 value)
template <int FMT>
DQ_HD float code_of(float x, const GroupQ& gq) {
  if (FMT == kInt4Bf16) {
    const float r = rne_quotient_int(x * gq.sc, gq.ds, gq.hds, gq.rd);
    return fminf(fmaxf(r, -8.0f), 7.0f);
  }
  const float ax = fabsf(x);
  float r;
  if (FMT == kMxInt4) {
    r = fminf(rintf(ax * gq.rd), 7.0f);  // exact quotient: d is a power of two
  } else if (FMT == kMxFp4) {
    r = e2m1_mag(ax * gq.rd);
  } else {
    r = e2m1_quotient(ax * gq.sc, gq.ds, gq.rd);
  }
  return x < 0.0f ? -r : r;
}

// ------------------------------------------------------- codes through a double quotient
// For fp32 x and the divisors Q produces (a bf16 value for INT4, an fp32 value for NVFP4, a
// power of two for MX), the quotient x / d either lies exactly on a rounding boundary of
// the code grid (a half-integer, or an E2M1 midpoint 1/4, 3/4, ..., 5) or at least 2^-29
// away from every boundary: x - h d is a nonzero multiple of min(ulp(x), ulp(d)) / 4 and
// x ~ h d bounds how small that is against d. A double quotient p = x * r with r within
// 2^-48 of 1 / d (relative) is within 2^-44 of x / d, so snapping x * r onto the multiples
// of 2^-32 keeps it on the same side of every boundary and makes it equal at a tie; the
// hardware's round-to-nearest-even of the snapped value then gives the exact code.

// 1 / v in double, relative error below 2^-48 (the hardware estimate and two Newton steps)
DQ_HD double recip64(float v) {
  const double d = (double)v;
#ifdef __HIP_DEVICE_COMPILE__
  double r = __builtin_amdgcn_rcp(d);
  double e = fma(-d, r, 1.0);
  r = fma(r, e, r);
  e = fma(-d, r, 1.0);
  return fma(r, e, r);
#else
  return 1.0 / d;
#endif
}

// x * r (|x r| < 2^19) rounded onto the multiples of 2^-32 with one rounding: the fused
// multiply-add rounds the exact product plus C = 1.5 * 2^20, whose ulp is 2^-32
DQ_HD double snap_quotient(double x, double r) { return fma(x, r, 0x1.8p20) - 0x1.8p20; }

// E2M1 magnitude nearest to a snapped quotient v >= 0, ties to the even index, saturating:
// adding C = 2^51 * max(1, 2^floor(log2 v)) puts the double ulp at the grid spacing of v's
// binade (0.5, 1, 2), as e2m1_mag does in fp32
DQ_HD double e2m1_grid64(double v) {
  const uint32_t hi = (uint32_t)(d2u(v) >> 32);
  const uint32_t base = (hi & 0x7FF00000u) > 0x3FF00000u ? (hi & 0x7FF00000u) : 0x3FF00000u;
  const double c = u2d((unsigned long long)(base + (51u << 20)) << 32);
  const double r = (v + c) - c;
  return r < 6.0 ? r : 6.0;
}

// INT4 codes need their clamp to [-8, 7] only where s is a subnormal bf16 value (s < 2^-126):
// a normal s lies within 2^-9 (relative) of mx / 7, so |x / s| <= 7.03, but the subnormal
// grid is coarser (spacing 2^-133) and |x / s| can reach about 8.4 there
DQ_HD double int4_clamp(double q) { return q < -8.0 ? -8.0 : (q > 7.0 ? 7.0 : q); }
DQ_HD bool int4_needs_clamp(float d) { return d < 0x1p-126f; }

// the signed code of x given r ~ 1 / d (see above), before INT4's clamp (int4_clamp, needed
// only where int4_needs_clamp(d))
template <int FMT>
DQ_HD double code64(float x, double r, const GroupQ& gq) {
  if (FMT == kInt4Bf16) return rint(snap_quotient((double)x, r));
  if (FMT == kNvFp4) {
    const double m = e2m1_grid64(snap_quotient((double)fabsf(x), r));
    return x < 0.0f ? -m : m;
  }
  return (double)code_of<FMT>(x, gq);  // MX: d is a power of two, the fp32 quotient is exact
}

// ----------------------------------------------------------------- NVFP4 codes in fp32
// The group scale: NVFP4 takes u = fl32(mx / fl32(6 g)). With r6 = 1 / fl32(6 g) correctly
// rounded in fp64, fl32(mx * r6) is that value: mx * r6 lies within 2^-52 (relative) of the
// quotient, and a quotient of two fp32 values is an fp32 value or lies at least 2^-47
// (relative) from every midpoint between fp32 values, so both round to the same fp32 value.
// The rest of the rule is the one group_scale applies.
__device__ __forceinline__ GroupQ nv_group_scale(float mx, float g, double r6) {
  GroupQ r;
  float s = 1.0f;
  if (mx > 0.0f) s = fmaxf(e4m3_rne_sat((float)((double)mx * r6)), 0x1p-9f);
  r.d = s * g;
  r.scode = e4m3_bits(s);
  r.rd = __builtin_amdgcn_rcpf(r.d);  // within one ulp of 1 / d
  r.sc = 1.0f;
  r.ds = r.d;
  r.hds = 0.5f * r.d;
  return r;
}

// The code of x / d rounded onto E2M1, in fp32: t = |x| rd and one correction give t1 within
// one ulp of |x| / d (the correction's own error is below 2^-45 relative, as rd is within one
// ulp), and t1 equals |x| / d where that is an fp32 value. The residual |x| - t1 d is then
// exact, so its sign says on which side of t1 the quotient lies, and z below is the quotient
// rounded to odd (t1 itself when exact, else the odd one of the two fp32 values around it).
// E2M1's decision points (1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5) are even fp32 values, so z lies on
// the same side of each as |x| / d and equals one only at a tie: rounding z onto E2M1 (the
// hardware conversion with scale 1) gives the code of |x| / d. |x| is first clamped to 8 d:
// every quotient of 5 or more takes the saturated code 6, and below 8 nothing overflows and
// the residuals stay exact. Valid for 2^-100 <= d <= 2^100; the caller checks that. CLAMP =
// false leaves the clamp out where the caller knows every |x| < 7 d.
template <bool CLAMP = true>
DQ_HD float nv_odd_quotient(float x, float d, float rd, float d8) {
  const float ax = CLAMP ? fminf(fabsf(x), d8) : fabsf(x);
  const float t = ax * rd;
  const float t1 = fmaf(fmaf(-t, d, ax), rd, t);
  const uint32_t rb = f2u(fmaf(-t1, d, ax));  // +0 when exact
  const uint32_t z = (f2u(t1) - (rb >> 31)) | ((rb << 1) != 0u ? 1u : 0u);
  return u2f(z | (f2u(x) & 0x80000000u));
}

// 8 NVFP4 codes as nibbles (column 2k low) through nv_odd_quotient. CLAMP = false when no
// quotient of the wave's groups can reach 8 (every group max below 7 d).
template <bool CLAMP>
__device__ __forceinline__ uint32_t nv_pack8_fast(const float* x, float d, float rd) {
  const float d8 = 8.0f * d;
  auto z = [&](int k) { return nv_odd_quotient<CLAMP>(x[k], d, rd, d8); };
  uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, z(0), z(1), 1.0f, 0);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, z(2), z(3), 1.0f, 1);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, z(4), z(5), 1.0f, 2);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, z(6), z(7), 1.0f, 3);
  const uint32_t mag = pk & 0x77777777u;  // keep the sign only where the magnitude is
  const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;  // nonzero (no -0 code)
  return mag | (pk & nz);
}

template <int FMT>
DQ_HD uint32_t nibble_of(float q) {
  if (FMT == kInt4Bf16 || FMT == kMxInt4) return (uint32_t)((int)q) & 0xFu;
  const uint32_t idx = e2m1_index(fabsf(q));
  return idx == 0 ? 0u : ((q < 0.0f ? 8u : 0u) | idx);
}

// ------------------------------------------------------------------------ cross-lane helpers

__device__ __forceinline__ float lane_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// max over aligned groups of `lanes` lanes (2, 4 or 8)
__device__ __forceinline__ float group_max(float v, int lanes) {
  v = lane_xor_max(v, 1);
  if (lanes > 2) v = lane_xor_max(v, 2);
  if (lanes > 4) v = lane_xor_max(v, 4);
  return v;
}

// DPP lane permutations (within quads / 16-lane rows; every source lane exists)
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// max over aligned groups of LANES lanes (2, 4 or 8) with DPP
template <int LANES>
__device__ __forceinline__ float group_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  if (LANES > 2) v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  if (LANES > 4) v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  return v;
}

// (the old value 0 is the identity of the unsigned max the result feeds, which lets the
// compiler fold the permutation into that max)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max over aligned groups of LANES lanes of non-negative float bit patterns (for those the
// unsigned order is the float order), no NaN canonicalization needed
template <int LANES>
__device__ __forceinline__ uint32_t group_max_bits(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  if (LANES > 2) v = max(v, dpp_u32<kDppQuadXor2>(v));
  if (LANES > 4) v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  return v;
}

// sum over aligned groups of 8 lanes, fixed order, result in all 8 lanes
__device__ __forceinline__ double sum8_dpp(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowHalfMirror>(v);
  return v;
}

// sum over aligned groups of 16 lanes, fixed order, result in all 16 lanes
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15 - i within each 16 lanes
__device__ __forceinline__ double sum16_dpp(double v) {
  v = sum8_dpp(v);
  v += dpp_f64<kDppRowMirror>(v);
  return v;
}

// sum over aligned groups of 32 lanes, fixed order, result in all 32 lanes (the pair of
// 16-lane sums added the same way round in both halves)
__device__ __forceinline__ double sum32_lanes(double v) {
  v = sum16_dpp(v);
  return v + __shfl_xor(v, 16, kWave);
}

// sum over a workgroup of 4 waves in a fixed order, the result returned to every thread:
// 16-lane sums, the wave's four in lane order, the waves' in wave order. `red` is LDS of at
// least 4 doubles; one barrier (the caller keeps `red` untouched until all have read it).
__device__ __forceinline__ double block_sum4(double v, double* red) {
  v = sum16_dpp(v);
  const double w = ((__shfl(v, 0, kWave) + __shfl(v, 16, kWave)) + __shfl(v, 32, kWave)) +
                   __shfl(v, 48, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = w;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// butterfly sum over the 64 lanes, the same fixed order in every lane and run
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) v = fmaxf(v, __shfl_xor(v, mask, kWave));
  return v;
}

}  // namespace dq
