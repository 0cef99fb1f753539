// dq_act.hip -- activation quantization with the column inverse scales.
//
// The consumer side of the factorized product (daiwk notes, "核心公式" eq. 1: X W^T ~=
// (X D_beta^-1) Qhat^T D_alpha^-1, with D_beta^-1 = D_b; the flowchart scales the real
// activations by the column inverse scales, then quantizes them): every activation row
// (token) is scaled channel by channel, x_tj = fl32(X_tj * b_j), and quantized with the
// weights' group quantizer Q in groups of G consecutive channels. Scaling and quantization
// run in one kernel, so the scaled activations never touch memory (trove summary, "Evidence":
// folding beta into the activation quantizer is what keeps its overhead small).
//
// Layout: a workgroup of four waves owns a 1024-channel tile of a chunk of tokens; a lane
// owns 16 consecutive channels, so its b values stay in registers for the whole chunk and a
// group of G channels spans G / 16 lanes. Each wave keeps four token rows of loads in
// flight. Per row a lane stores 8 bytes of packed codes (a wave-row is one contiguous
// 512-byte segment) and, from every G / 16-th lane, one inner scale.
//
// Codes: MXFP4 through gfx950's scaled FP4 conversion (it rounds x / c to the nearest E2M1
// value, ties to even, saturating, exactly for power-of-two c; used for c in [2^-100, 2^20],
// the range it was checked on, otherwise the exact fp32 path); MXINT4 through the exact
// power-of-two quotient; INT4/BF16 and NVFP4 through the snapped double quotient (code64).
#include <float.h>

#include "dq_device.h"
#include "dq_internal.h"

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace dq {

constexpr int kActEpl = 16;                  // consecutive channels per lane
constexpr int kActCols = kWave * kActEpl;    // 1024 channels per tile
constexpr int kActRows = 4;                  // rows of loads in flight per wave

template <bool BF>
struct ActLoad;
template <>
struct ActLoad<true> {  // 16 bf16 = two 128-bit loads
  uint4 v[2];
};
template <>
struct ActLoad<false> {  // 16 fp32 = four 128-bit loads
  uint4 v[4];
};

template <bool BF>
__device__ __forceinline__ void act_load(const void* X, int64_t off, ActLoad<BF>& L) {
  const uint4* src = reinterpret_cast<const uint4*>(
      BF ? (const void*)(static_cast<const uint16_t*>(X) + off)
         : (const void*)(static_cast<const float*>(X) + off));
#pragma unroll
  for (int k = 0; k < (BF ? 2 : 4); k++) L.v[k] = src[k];
}

template <bool BF>
__device__ __forceinline__ void act_unpack(const ActLoad<BF>& L, float (&w)[kActEpl]) {
  if (BF) {
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const uint32_t u[4] = {L.v[k].x, L.v[k].y, L.v[k].z, L.v[k].w};
#pragma unroll
      for (int h = 0; h < 4; h++) {
        w[8 * k + 2 * h] = u2f(u[h] << 16);
        w[8 * k + 2 * h + 1] = u2f(u[h] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      w[4 * k] = u2f(L.v[k].x);
      w[4 * k + 1] = u2f(L.v[k].y);
      w[4 * k + 2] = u2f(L.v[k].z);
      w[4 * k + 3] = u2f(L.v[k].w);
    }
  }
}

// 8 codes as nibbles (column 2k low) from 8 scaled values
template <int FMT>
__device__ __forceinline__ uint32_t act_pack8(const float* x, const GroupQ& gq, double r,
                                              bool clamp) {
  uint32_t packed = 0u;
  if (FMT == kMxFp4 && gq.d >= 0x1p-100f && gq.d <= 0x1p20f) {
    uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], gq.d, 0);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x[2], x[3], gq.d, 1);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x[4], x[5], gq.d, 2);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x[6], x[7], gq.d, 3);
    const uint32_t mag = pk & 0x77777777u;  // keep the sign only where the magnitude is
    const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;  // nonzero (no -0 code)
    return mag | (pk & nz);
  }
  if (FMT == kMxFp4 || FMT == kMxInt4) {
#pragma unroll
    for (int k = 0; k < 8; k++) packed |= nibble_of<FMT>(code_of<FMT>(x[k], gq)) << (4 * k);
    return packed;
  }
  if (FMT == kInt4Bf16 && clamp) {  // rare: a subnormal scale somewhere in the wave
#pragma unroll
    for (int k = 0; k < 8; k++)
      packed |= nibble_of<FMT>((float)int4_clamp(code64<FMT>(x[k], r, gq))) << (4 * k);
    return packed;
  }
#pragma unroll
  for (int k = 0; k < 8; k++) packed |= nibble_of<FMT>((float)code64<FMT>(x[k], r, gq)) << (4 * k);
  return packed;
}

template <int FMT, int G, bool BF, bool PARTIAL>
__global__ __launch_bounds__(kBlock) void k_act(ActArgs p) {
  constexpr int LPG = G / kActEpl;
  constexpr int E = kActEpl;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ct = blockIdx.x % p.nct;
  const int rc = blockIdx.x / p.nct;
  const int64_t r_begin = (int64_t)rc * p.rpc;
  const int64_t r_end = r_begin + p.rpc < p.m ? r_begin + p.rpc : p.m;
  const int64_t col = (int64_t)ct * kActCols + lane * E;
  const bool act = col < p.n;          // n is a multiple of 16: a lane is wholly in or out
  const int64_t lcol = act ? col : 0;  // in-bounds address

  float bv[E];
#pragma unroll
  for (int h = 0; h < E / 4; h++) {
    float4 v = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    if (p.b) v = reinterpret_cast<const float4*>(p.b + lcol)[h];
    bv[4 * h] = v.x;
    bv[4 * h + 1] = v.y;
    bv[4 * h + 2] = v.z;
    bv[4 * h + 3] = v.w;
  }
  float g = 1.0f, sixg = 6.0f;
  double r6 = 0.0;
  if (FMT == kNvFp4) {
    g = p.gs ? p.gs[0] : p.g;
    sixg = 6.0f * g;
    r6 = 1.0 / (double)sixg;
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
  }
  int flags = 0;
  for (int64_t i0 = r_begin + (int64_t)wave * kActRows; i0 < r_end; i0 += kWaves * kActRows) {
    ActLoad<BF> L[kActRows];
#pragma unroll
    for (int u = 0; u < kActRows; u++) {
      const int64_t row = i0 + u < r_end ? i0 + u : r_begin;  // in-bounds; skipped below
      act_load<BF>(p.X, row * p.n + lcol, L[u]);
    }
#pragma unroll
    for (int u = 0; u < kActRows; u++) {
      const int64_t i = i0 + u;
      if (i >= r_end) break;  // uniform across the wave
      float w[E], x[E];
      act_unpack<BF>(L[u], w);
      float mx = 0.0f, chk = 0.0f;
#pragma unroll
      for (int k = 0; k < E; k++) {
        x[k] = w[k] * bv[k];
        mx = fmaxf(mx, fabsf(x[k]));
        chk = fmaf(x[k], 0.0f, chk);  // NaN once any x is not finite
      }
      if (chk != 0.0f) {  // rare: a non-finite input, or the scaling overflowed
        bool in_bad = false;
#pragma unroll
        for (int k = 0; k < E; k++) in_bad |= !(fabsf(w[k]) <= FLT_MAX);
        flags |= in_bad ? kStNonFinite : kStRange;
        mx = 0.0f;
      }
      const float gm = LPG > 1 ? u2f(group_max_bits<LPG>(f2u(mx))) : mx;
      GroupQ gq;
      uint32_t lo, hi;
      if (FMT == kNvFp4) {
        gq = nv_group_scale(gm, g, r6);
        // fp32 codes unless a group of the wave has a divisor outside [2^-100, 2^100]: those
        // rows take the double quotient
        if (__all(gq.d >= 0x1p-100f && gq.d <= 0x1p100f)) {
          if (__any(!(gm < 7.0f * gq.d))) {  // some scale saturated at 448
            lo = nv_pack8_fast<true>(x, gq.d, gq.rd);
            hi = nv_pack8_fast<true>(x + 8, gq.d, gq.rd);
          } else {
            lo = nv_pack8_fast<false>(x, gq.d, gq.rd);
            hi = nv_pack8_fast<false>(x + 8, gq.d, gq.rd);
          }
        } else {
          const double r = recip64(gq.d);
          lo = act_pack8<FMT>(x, gq, r, false);
          hi = act_pack8<FMT>(x + 8, gq, r, false);
        }
      } else {
        gq = group_scale<FMT>(gm, g, sixg);
        const double r = FMT == kInt4Bf16 ? recip64(gq.d) : 0.0;
        const bool clamp = FMT == kInt4Bf16 && __any(int4_needs_clamp(gq.d));
        lo = act_pack8<FMT>(x, gq, r, clamp);
        hi = act_pack8<FMT>(x + 8, gq, r, clamp);
      }
      if (!PARTIAL || act) {
        // nontemporal: the codes and scales are written once and not read back here
        const u32x2 cw = {lo, hi};
        __builtin_nontemporal_store(cw, reinterpret_cast<u32x2*>(p.codes + ((i * p.n + lcol) >> 1)));
        if ((lane % LPG) == 0) {
          const int64_t si = i * (p.n / G) + lcol / G;
          if (FMT == kInt4Bf16)
            __builtin_nontemporal_store((uint16_t)gq.scode, static_cast<uint16_t*>(p.scales) + si);
          else
            __builtin_nontemporal_store((uint8_t)gq.scode, static_cast<uint8_t*>(p.scales) + si);
        }
      }
    }
  }
  if (flags) atomicOr(p.status, flags);  // rare: only lanes that saw a problem
}

// NVFP4 tensor scale from the activations: per-block max |x|, x = fl32(X * b), then one
// block turns the block maxima into g = fl32(A / 2688) (at least 2^-126; 1 if A = 0).
template <bool BF>
__global__ __launch_bounds__(256) void k_act_amax(ActArgs p) {
  __shared__ float red[256];
  const int64_t chunks = p.m * (p.n / kActEpl);
  float mx = 0.0f;
  int flags = 0;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    const int64_t row = c / (p.n / kActEpl);
    const int64_t col = (c % (p.n / kActEpl)) * kActEpl;
    ActLoad<BF> L;
    act_load<BF>(p.X, row * p.n + col, L);
    float w[kActEpl];
    act_unpack<BF>(L, w);
#pragma unroll
    for (int k = 0; k < kActEpl; k++) {
      const float x = w[k] * (p.b ? p.b[col + k] : 1.0f);
      if (!(fabsf(x) <= FLT_MAX)) flags |= (fabsf(w[k]) <= FLT_MAX) ? kStRange : kStNonFinite;
      else mx = fmaxf(mx, fabsf(x));
    }
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) p.part[blockIdx.x] = red[0];
  if (flags) atomicOr(p.status, flags);
}

__global__ __launch_bounds__(256) void k_act_gscale(ActArgs p, int nparts) {
  __shared__ float red[256];
  float mx = 0.0f;
  for (int k = threadIdx.x; k < nparts; k += 256) mx = fmaxf(mx, p.part[k]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float A = red[0];
    const float g = A == 0.0f ? 1.0f : fmaxf((float)((double)A / 2688.0), 0x1p-126f);
    p.gs_out[0] = g;
  }
}

int act_tile_cols() { return kActCols; }
int act_amax_blocks() { return 1024; }

template <int FMT, int G, bool BF>
static hipError_t act_partial(const ActArgs& a, dim3 grid, hipStream_t s) {
  if (a.n % kActCols != 0)
    hipLaunchKernelGGL((k_act<FMT, G, BF, true>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((k_act<FMT, G, BF, false>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool BF>
static hipError_t act_group(const ActArgs& a, dim3 grid, hipStream_t s) {
  switch (a.G) {
    case 16: return act_partial<FMT, 16, BF>(a, grid, s);
    case 32: return act_partial<FMT, 32, BF>(a, grid, s);
    case 64: return act_partial<FMT, 64, BF>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
static hipError_t act_dtype(bool bf16, const ActArgs& a, dim3 grid, hipStream_t s) {
  return bf16 ? act_group<FMT, true>(a, grid, s) : act_group<FMT, false>(a, grid, s);
}

hipError_t launch_act(int fmt, bool bf16, const ActArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.nct * a.nrc));
  switch (fmt) {
    case kInt4Bf16: return act_dtype<kInt4Bf16>(bf16, a, grid, s);
    case kMxInt4: return act_dtype<kMxInt4>(bf16, a, grid, s);
    case kMxFp4: return act_dtype<kMxFp4>(bf16, a, grid, s);
    case kNvFp4: return act_dtype<kNvFp4>(bf16, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_act_gscale(bool bf16, const ActArgs& a, hipStream_t s) {
  const int nb = act_amax_blocks();
  if (bf16)
    hipLaunchKernelGGL(k_act_amax<true>, dim3(nb), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_act_amax<false>, dim3(nb), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_act_gscale, dim3(1), dim3(256), 0, s, a, nb);
  return hipGetLastError();
}

}  // namespace dq
