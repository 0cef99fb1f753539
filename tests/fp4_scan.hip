// Exhaustive GPU scan of the FP4 conversions that the HIP library's kernels rely on, for the
// test tests/test_gpu_fp4_conversion.py (test infrastructure; the library never loads this).
//
// For every non-negative finite fp32 x (bit patterns 0 .. 0x7F7FFFFF, ascending, which is
// ascending in value), the scan computes the E2M1 code that a kernel would store for x and
// for -x, and records only the points where the code of x changes: (u, code(u), code(u+1)).
// The code of a non-negative x is a non-decreasing step function of x, so the recorded
// transitions and the code at 0 describe it completely; the test checks each transition on
// both sides against exact E2M1 rounding of the quotient, which then holds for every x.
//
// Modes (each packs into all four byte positions of a 32-bit word, x at even and -x at odd
// nibbles, and counts words whose four copies disagree):
//   0  v_cvt_scalef32_pk_fp4_f32 with scale p (a power of two): E2M1 of x / p, saturating,
//      the MX formats' conversion
//   1  nv_pack8_fast<true> (the library's NVFP4 fp32 codes, with the clamp) for divisor p
//   2  nv_pack8_fast<false> for divisor p (its caller guarantees |x| < 7 p; the host passes
//      the last such bit pattern)
// Result words: [0] transitions found, [1] sign mismatches (code(-x) is not code(x) with the
// sign bit, or a zero magnitude with anything but 0 / 8), [2] the first x with one, [3] words
// whose byte positions disagree, [4 + 3k ..] transition k: u, code(u), code(u + 1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../dual_scale_w4a4_amd/csrc/dq_device.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 2048;

// the packed word for x in the given mode: nibble 2k holds code(x), 2k + 1 code(-x)
__device__ __forceinline__ uint32_t packed_word(int mode, float x, float p, float rp) {
  if (mode == 0) {
    uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, -x, p, 0);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x, -x, p, 1);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x, -x, p, 2);
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, x, -x, p, 3);
    return pk;
  }
  const float xs[8] = {x, -x, x, -x, x, -x, x, -x};
  return mode == 1 ? dq::nv_pack8_fast<true>(xs, p, rp) : dq::nv_pack8_fast<false>(xs, p, rp);
}

__global__ __launch_bounds__(kThreads) void k_fp4_scan(int mode, float p, uint32_t u_last,
                                                       uint32_t* res, int cap) {
  const float rp = __builtin_amdgcn_rcpf(p);  // as the library forms 1 / d
  const uint64_t n = (uint64_t)u_last + 1;
  const uint64_t nthreads = (uint64_t)kThreads * kBlocks;
  const uint64_t chunk = (n + nthreads - 1) / nthreads;
  const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint64_t u0 = tid * chunk;
  if (u0 >= n) return;
  const uint64_t u1 = u0 + chunk < n ? u0 + chunk : n;
  uint32_t prev = 0xFFFFFFFFu;
  if (u0 > 0) prev = packed_word(mode, __uint_as_float((uint32_t)(u0 - 1)), p, rp) & 0xFu;
  for (uint64_t u = u0; u < u1; u++) {
    const float x = __uint_as_float((uint32_t)u);
    const uint32_t w = packed_word(mode, x, p, rp);
    const uint32_t pos = w & 0xFu, neg = (w >> 4) & 0xFu;
    if ((w & 0xFFu) * 0x01010101u != w) atomicAdd(&res[3], 1u);
    const bool neg_ok = pos == 0u ? (neg == 0u || neg == 8u) : neg == (pos | 8u);
    if (!neg_ok && atomicAdd(&res[1], 1u) == 0u) res[2] = (uint32_t)u;
    if (prev != 0xFFFFFFFFu && pos != prev) {
      const uint32_t k = atomicAdd(&res[0], 1u);
      if ((int)k < cap) {
        res[4 + 3 * k] = (uint32_t)(u - 1);
        res[5 + 3 * k] = prev;
        res[6 + 3 * k] = pos;
      }
    }
    prev = pos;
  }
}

// the decode direction: every byte value at every byte position, scale p
__global__ void k_fp4_decode(float p, float* out) {
  const int t = threadIdx.x;  // 0 .. 1023: byte t & 255 at position t >> 8
  const uint32_t word = (uint32_t)(t & 255) << (8 * (t >> 8));
  float2 v;
  switch (t >> 8) {
    case 0: { const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, p, 0); v = make_float2(r[0], r[1]); break; }
    case 1: { const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, p, 1); v = make_float2(r[0], r[1]); break; }
    case 2: { const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, p, 2); v = make_float2(r[0], r[1]); break; }
    default: { const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, p, 3); v = make_float2(r[0], r[1]); break; }
  }
  out[2 * t] = v.x;
  out[2 * t + 1] = v.y;
}

// the encode direction on given pairs: out[i] = code byte of (x[2 i], x[2 i + 1]) at scale p
__global__ void k_fp4_encode(float p, const float* x, uint32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[2 * i], x[2 * i + 1], p, 0) & 0xFFu;
}

}  // namespace

extern "C" {

// res: device, 4 + 3 * cap words, zeroed by the caller. Returns a hipError_t.
int fp4_scan(int mode, float p, uint32_t u_last, uint32_t* res, int cap, hipStream_t s) {
  if (mode < 0 || mode > 2 || !res || cap < 1 || u_last > 0x7F7FFFFFu) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fp4_scan, dim3(kBlocks), dim3(kThreads), 0, s, mode, p, u_last, res, cap);
  return (int)hipGetLastError();
}

// out: device, 2048 floats
int fp4_decode(float p, float* out, hipStream_t s) {
  if (!out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fp4_decode, dim3(1), dim3(1024), 0, s, p, out);
  return (int)hipGetLastError();
}

// x: device, 2 n floats; out: device, n words
int fp4_encode(float p, const float* x, uint32_t* out, int n, hipStream_t s) {
  if (!x || !out || n < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fp4_encode, dim3((n + 255) / 256), dim3(256), 0, s, p, x, out, n);
  return (int)hipGetLastError();
}

}  // extern "C"
