// dq_pass.hip -- the two-sweep iteration pass for bf16 weights.
//
// With BF16 or E4M3 outer scales (INT4_BF16, NVFP4) the row update changes the codes, so an
// iteration quantizes every element twice (daiwk notes, "核心公式": quantize, row update,
// re-quantize with the inner copies synced, column update): a row pass with the current
// row scales gives N_i = sum_j W_ij R_ij and D_i = sum_j R_ij^2 with R = Qhat D_b, and after
// the row finalize a column pass with the updated scales gives P_j = sum_i W_ij S_ij and
// Q_j = sum_i S_ij^2 with S = D_a Qhat. The MX formats take this pass too when the
// single-sweep identity is not used.
//
// Layout: a workgroup of four 64-lane waves owns a 1024-column tile of a chunk of rows; a
// lane owns 16 consecutive columns (two 128-bit loads per row), so a group of G columns
// spans G / 16 lanes and the per-group work (absmax, scale rule, reciprocal) is shared by
// 16 elements per lane. A wave takes its rows in batches of 8 consecutive rows, 32 rows
// apart across the workgroup, with the loads of the next step, and the row scales of the
// next batch, issued before the current rows are computed.
//
// Codes come from the snapped double quotient (code64): exact, and already in fp64 for the
// sums (NVFP4's final pass takes the fp32 codes of nv_pack8_fast, exact as well, and decodes
// them for its row error). NVFP4's group scale takes u = fl32(mx / fl32(6 g)) as fl32(mx r6)
// (nv_group_scale). Sums: every term (W * q * b, (q * b)^2, W * a * d * q, (a * d * q)^2) is an exact
// product in fp64 and is accumulated in fp64 in a fixed order; a row's 64 lane partials are
// transposed through LDS every 8 rows and added by 8 lanes per row, and the four waves'
// column partials are added through LDS at the end. No floating-point atomics.
#include <float.h>

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {

constexpr int kPassBatch = 8;                // rows per wave between row reductions
constexpr int kPassEpl = 16;                 // consecutive columns per lane
constexpr int kPassCols = kWave * kPassEpl;  // 1024 columns per tile

// One row of this lane's 16 elements: Q, and then (ROW) the lane's contribution to the row
// sums, (COL) the column accumulators, (EMIT) the packed codes and the scale codes.
template <int FMT, int LPG, int MODE, bool PARTIAL>
__device__ __forceinline__ void pass_row(const uint4 (&v)[2], const float (&rb)[kPassEpl],
                                         const double (&bbd)[kPassEpl], float ra, float ai,
                                         float g, float sixg, double r6, uint32_t amask,
                                         double& nacc, double& dacc, double& wacc,
                                         double (&P)[kPassEpl],
                                         double (&Q)[kPassEpl], int& flags, uint32_t* code_word,
                                         void* scale_ptr, float& ymax) {
  constexpr bool ROW = (MODE & kModeRow) != 0;
  constexpr bool COL = (MODE & kModeCol) != 0;
  constexpr bool EMIT = (MODE & kModeEmit) != 0;
  constexpr int E = kPassEpl;
  uint32_t u[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
  // NVFP4's iteration passes need only the codes' magnitudes: q has the sign of x, which is
  // that of w (x = w rb ra with positive scales, and fp32 rounding is symmetric), so they
  // read |w| (sign bits cleared here), scale it into |x|, and the sums take w q = |w| |q|
  constexpr bool kMag = FMT == kNvFp4 && !EMIT;
  if (PARTIAL || kMag) {
    const uint32_t keep = (PARTIAL ? amask : 0xFFFFFFFFu) & (kMag ? 0x7FFF7FFFu : 0xFFFFFFFFu);
#pragma unroll
    for (int k = 0; k < 8; k++) u[k] &= keep;
  }
  float w[E], x[E];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    w[2 * k] = u2f(u[k] << 16);
    w[2 * k + 1] = u2f(u[k] & 0xFFFF0000u);
  }
  float mx = 0.0f, ym = 0.0f;
#pragma unroll
  for (int k = 0; k < E; k++) {
    const float y = w[k] * rb[k];  // column scale first, then row scale; two fp32 roundings
    x[k] = y * ra;
    mx = fmaxf(mx, kMag ? x[k] : fabsf(x[k]));
    if (MODE & kModeYmax) ym = fmaxf(ym, fabsf(y));
  }
  ymax = ym;
  float gm = LPG > 1 ? u2f(group_max_bits<LPG>(f2u(mx))) : mx;
  if (!(gm <= FLT_MAX)) {  // a scaled value overflowed
    flags |= kStRange;
    gm = 0.0f;
  }
  const GroupQ gq = FMT == kNvFp4 ? nv_group_scale(gm, g, r6) : group_scale<FMT>(gm, g, sixg);
  double q[E];  // the codes as values
  uint32_t pk[2] = {0u, 0u};  // the codes packed as stored (EMIT)
  // NVFP4's final pass takes the fp32 codes, which come packed (the nibble packing of the
  // double-quotient codes costs the pass more than their sums); the iteration passes keep
  // the double quotient, with which the row pass stays at three waves per SIMD
  constexpr bool kFast = FMT == kNvFp4 && EMIT;
  if (kFast && __all(gq.d >= 0x1p-100f && gq.d <= 0x1p100f)) {
    if (__any(!(gm < 7.0f * gq.d))) {  // some scale saturated at 448
      pk[0] = nv_pack8_fast<true>(x, gq.d, gq.rd);
      pk[1] = nv_pack8_fast<true>(x + 8, gq.d, gq.rd);
    } else {
      pk[0] = nv_pack8_fast<false>(x, gq.d, gq.rd);
      pk[1] = nv_pack8_fast<false>(x + 8, gq.d, gq.rd);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 0);
      const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 1);
      const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 2);
      const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 3);
      const float qv[8] = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
#pragma unroll
      for (int k = 0; k < 8; k++) q[8 * h + k] = (double)qv[k];
    }
  } else {
    const double r = (FMT == kInt4Bf16 || FMT == kNvFp4) ? recip64(gq.d) : 0.0;
    if (FMT == kInt4Bf16 && __any(int4_needs_clamp(gq.d))) {  // rare: a subnormal scale
#pragma unroll
      for (int k = 0; k < E; k++) q[k] = int4_clamp(code64<FMT>(x[k], r, gq));
    } else if (kMag) {
#pragma unroll
      for (int k = 0; k < E; k++) q[k] = e2m1_grid64(snap_quotient((double)x[k], r));
    } else {
#pragma unroll
      for (int k = 0; k < E; k++) q[k] = code64<FMT>(x[k], r, gq);
    }
    if (EMIT) {
#pragma unroll
      for (int k = 0; k < E; k++) pk[k / 8] |= nibble_of<FMT>((float)q[k]) << (4 * (k % 8));
    }
  }

  if (ROW) {
    double nl = 0.0, dl = 0.0, wl = 0.0;
#pragma unroll
    for (int k = 0; k < E; k++) {
      const double t = q[k] * bbd[k];  // R / d, exact
      nl = fma((double)w[k], t, nl);
      dl = fma(t, t, dl);
      if (MODE & kModeStat) wl = fma((double)w[k], (double)w[k], wl);  // W^2, exact
    }
    wacc = wl;
    const double dd = (double)gq.d;
    nacc = nl * dd;
    dacc = dl * (dd * dd);
  }
  if (COL) {
    const double c = (double)ai * (double)gq.d;  // exact
#pragma unroll
    for (int k = 0; k < E; k++) {
      const double s = c * q[k];  // S, exact
      P[k] = fma((double)w[k], s, P[k]);
      Q[k] = fma(s, s, Q[k]);
    }
  }
  if (EMIT && (!PARTIAL || amask != 0u)) {
    *reinterpret_cast<uint2*>(code_word) = make_uint2(pk[0], pk[1]);
    if ((__lane_id() % LPG) == 0) {
      if (FMT == kInt4Bf16)
        *static_cast<uint16_t*>(scale_ptr) = (uint16_t)gq.scode;
      else
        *static_cast<uint8_t*>(scale_ptr) = (uint8_t)gq.scode;
    }
  }
}

// The pass on one workgroup's tile (block `bid` of the matrix's grid). MODE: kModeRow,
// kModeCol or kModeRow | kModeEmit (the final Q with the row sums of its error), optionally
// | kModeYmax (NVFP4's per-pass tensor scale), or kModeRow | kModeStat (a solve's first row
// pass, which also sums W^2 per row and tile for E_i and the finite check). S: rows per load
// step. G >= 16; LPG = G / 16 lanes per group.
template <int FMT, int G, int MODE, bool PARTIAL, int S>
__device__ __forceinline__ void pass_block(const SweepArgs& p, int bid) {
  constexpr bool ROW = (MODE & kModeRow) != 0;
  constexpr bool COL = (MODE & kModeCol) != 0;
  constexpr bool EMIT = (MODE & kModeEmit) != 0;
  constexpr int LPG = G / kPassEpl;
  constexpr int E = kPassEpl;
  // LDS: a wave's [8 rows][64 lanes] row partials, or the column combine of half a tile
  constexpr int kLds = kWaves * kPassBatch * kWave;
  static_assert(kLds == kWaves * (kPassCols / 2), "one LDS buffer serves both");
  __shared__ double2 smem[kLds];

  const uint16_t* W = static_cast<const uint16_t*>(p.W);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ct = bid % p.nct;
  const int rc = bid / p.nct;
  const int64_t r_begin = (int64_t)rc * p.rpc;
  const int64_t r_end = r_begin + p.rpc < p.m ? r_begin + p.rpc : p.m;
  const int64_t col = (int64_t)ct * kPassCols + lane * E;
  const bool act = col < p.n;          // n is a multiple of 16: a lane is wholly in or out
  const int64_t lcol = act ? col : 0;  // in-bounds address
  const uint32_t amask = act ? 0xFFFFFFFFu : 0u;

  float rb[E];
  double bbd[E];
#pragma unroll
  for (int h = 0; h < E / 4; h++) {
    const float4 rv = reinterpret_cast<const float4*>(p.rb + lcol)[h];
    const float4 bv = reinterpret_cast<const float4*>(p.b + lcol)[h];
    const float rr[4] = {rv.x, rv.y, rv.z, rv.w};
    const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      rb[4 * h + k] = act ? rr[k] : 1.0f;
      bbd[4 * h + k] = act ? (double)bb[k] : 0.0;
    }
  }
  float g = 1.0f, sixg = 6.0f;
  double r6 = 0.0;  // 1 / fl32(6 g), correctly rounded
  if (FMT == kNvFp4) {
    g = p.gs[0];
    sixg = p.gs[1];
    r6 = 1.0 / (double)sixg;
  }
  double P[E], Q[E];
#pragma unroll
  for (int k = 0; k < E; k++) P[k] = Q[k] = 0.0;
  int flags = 0;

  const int64_t first = r_begin + (int64_t)wave * kPassBatch;
  const int64_t nbatch =
      first < r_end ? (r_end - first + kWaves * kPassBatch - 1) / (kWaves * kPassBatch) : 0;
  // loads of rows i .. i+S-1 from in-bounds addresses (rows past the chunk reload its first
  // row and are skipped below; columns past n are masked in pass_row)
  auto load = [&](int64_t i, uint4 (&buf)[S][2]) {
#pragma unroll
    for (int r = 0; r < S; r++) {
      const int64_t row = i + r < r_end ? i + r : r_begin;
      const uint4* src = reinterpret_cast<const uint4*>(W + row * p.n + lcol);
      buf[r][0] = src[0];
      buf[r][1] = src[1];
    }
  };
  // the row scales of a batch: lane l holds those of row row0 + (l & 7) (clamped into the
  // chunk), loaded one batch ahead so that no row waits on a load of its own; a row takes
  // them with a readlane
  auto load_rows = [&](int64_t row0, float& ra_v, float& a_v) {
    int64_t i = row0 + (lane & 7);
    i = i < r_end ? i : r_begin;
    ra_v = p.ra[i];
    if (COL) a_v = p.a[i];
  };
  constexpr bool YMAX = (MODE & kModeYmax) != 0;
  __shared__ float ysmem[YMAX ? kWaves * kPassBatch * kWave : 1];
  float* Ry = ysmem + (YMAX ? wave * (kPassBatch * kWave) : 0);  // [8 rows][64 lanes] max |y|
  double2* R = smem + wave * (kPassBatch * kWave);  // this wave's [8 rows][64 lanes] partials
  // the first pass of a solve (STAT): each row's sum of W^2 over the tile's columns, for E_i
  constexpr bool STAT = (MODE & kModeStat) != 0;
  __shared__ double wsmem[STAT ? kWaves * kPassBatch * kWave : 1];
  double* Rw = wsmem + (STAT ? wave * (kPassBatch * kWave) : 0);
  float ra_cur = 0.0f, a_cur = 0.0f, ra_nxt = 0.0f, a_nxt = 0.0f;
  auto row_step = [&](const uint4 (&v)[2], int64_t i, int r) {
    double nacc = 0.0, dacc = 0.0, wacc = 0.0;
    float ym = 0.0f;
    if (i < r_end) {  // uniform across the wave
      const float ra = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ra_cur), r));
      const float ai = COL ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a_cur), r)) : 0.0f;
      uint32_t* code_word = nullptr;
      void* scale_ptr = nullptr;
      if (EMIT) {
        code_word = reinterpret_cast<uint32_t*>(p.codes) + ((i * p.n + lcol) >> 3);
        const int64_t si = i * (p.n / G) + lcol / G;
        scale_ptr = FMT == kInt4Bf16 ? (void*)(static_cast<uint16_t*>(p.scales) + si)
                                     : (void*)(static_cast<uint8_t*>(p.scales) + si);
      }
      pass_row<FMT, LPG, MODE, PARTIAL>(v, rb, bbd, ra, ai, g, sixg, r6, amask, nacc, dacc, wacc, P,
                                        Q, flags, code_word, scale_ptr, ym);
    }
    if (ROW) R[r * kWave + lane] = make_double2(nacc, dacc);
    if (YMAX) Ry[r * kWave + lane] = ym;
    if (STAT) Rw[r * kWave + lane] = wacc;
  };

  constexpr int kSteps = kPassBatch / S;
  static_assert(kSteps % 2 == 0, "an even number of steps per batch");
  uint4 bufA[S][2], bufB[S][2];
  if (nbatch > 0) {
    load_rows(first, ra_cur, a_cur);
    load(first, bufA);
  }
  for (int64_t bt = 0; bt < nbatch; bt++) {
    const int64_t row0 = first + bt * (kWaves * kPassBatch);
    load_rows(row0 + kWaves * kPassBatch, ra_nxt, a_nxt);  // clamped past the last batch
#pragma unroll
    for (int st = 0; st < kSteps; st += 2) {
      load(row0 + (st + 1) * S, bufB);
#pragma unroll
      for (int r = 0; r < S; r++) row_step(bufA[r], row0 + st * S + r, st * S + r);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 2 < kSteps)
        load(row0 + (st + 2) * S, bufA);
      else if (bt + 1 < nbatch)
        load(row0 + kWaves * kPassBatch, bufA);
#pragma unroll
      for (int r = 0; r < S; r++) row_step(bufB[r], row0 + (st + 1) * S + r, (st + 1) * S + r);
      __builtin_amdgcn_sched_barrier(0);
    }
    ra_cur = ra_nxt;
    a_cur = a_nxt;
    if (ROW) {
      // 8 rows done: 8 lanes per row add 8 lane partials each (transposed through LDS),
      // then across the 8 lanes in a fixed order
      __builtin_amdgcn_wave_barrier();
      const double2* src = R + (lane >> 3) * kWave + (lane & 7) * 8;
      double N = 0.0, D = 0.0;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const double2 v = src[k];
        N += v.x;
        D += v.y;
      }
      N = sum8_dpp(N);
      D = sum8_dpp(D);
      const int64_t i = row0 + (lane >> 3);
      if ((lane & 7) == 0 && i < r_end) p.rowpart[(int64_t)ct * p.m + i] = make_double2(N, D);
      if (STAT) {  // the same for the row's W^2
        const double* wsrc = Rw + (lane >> 3) * kWave + (lane & 7) * 8;
        double Wq = 0.0;
#pragma unroll
        for (int k = 0; k < 8; k++) Wq += wsrc[k];
        Wq = sum8_dpp(Wq);
        if ((lane & 7) == 0 && i < r_end) p.epart[(int64_t)ct * p.m + i] = Wq;
      }
      if (YMAX) {  // the same for the row max of |y| (bit patterns of non-negative floats)
        const float* ysrc = Ry + (lane >> 3) * kWave + (lane & 7) * 8;
        uint32_t yb = 0u;
#pragma unroll
        for (int k = 0; k < 8; k++) yb = max(yb, f2u(ysrc[k]));
        yb = group_max_bits<8>(yb);
        if ((lane & 7) == 0 && i < r_end) p.ymax[(int64_t)ct * p.m + i] = u2f(yb);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  if (COL) {
    // the four waves' column sums, added in wave order, half a tile (lanes 0..31, then
    // 32..63) at a time
    constexpr int kHalf = kPassCols / 2;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      __syncthreads();
      if ((lane >> 5) == h) {
#pragma unroll
        for (int k = 0; k < E; k++)
          smem[wave * kHalf + (lane & 31) * E + k] = make_double2(P[k], Q[k]);
      }
      __syncthreads();
      for (int c = threadIdx.x; c < kHalf; c += kBlock) {
        double2 s = smem[c];
#pragma unroll
        for (int v = 1; v < kWaves; v++) {
          s.x += smem[v * kHalf + c].x;
          s.y += smem[v * kHalf + c].y;
        }
        const int64_t j = (int64_t)ct * kPassCols + h * kHalf + c;
        if (j < p.n) p.colpart[(int64_t)rc * p.n + j] = s;
      }
    }
  }
  if (flags) atomicOr(p.status, flags);  // rare: only lanes that saw a problem
}

template <int FMT, int G, int MODE, bool PARTIAL, int S>
__global__ __launch_bounds__(kBlock) void k_pass(SweepArgs p) {
  pass_block<FMT, G, MODE, PARTIAL, S>(p, blockIdx.x);
}

// Several matrices in one launch: workgroups [start[k], start[k+1]) run matrix k's grid.
template <int FMT, int G, int MODE, bool PARTIAL, int S>
__global__ __launch_bounds__(kBlock) void k_pass_multi(PassMulti m) {
  int k = 0;
  while (k + 1 < m.n && (int)blockIdx.x >= m.start[k + 1]) k++;
  pass_block<FMT, G, MODE, PARTIAL, S>(m.a[k], (int)blockIdx.x - m.start[k]);
}

// Rows per load step: INT4's row pass loads one row ahead instead of two, which keeps it at
// 168 VGPRs (three waves per SIMD instead of two)
template <int FMT, int MODE>
constexpr int pass_step_rows() { return FMT == kInt4Bf16 && (MODE & ~kModeStat) == kModeRow ? 1 : 2; }

template <int FMT, int G, int MODE>
static hipError_t pass_partial(const SweepArgs& a, dim3 grid, hipStream_t s) {
  constexpr int S = pass_step_rows<FMT, MODE>();
  if (a.n % kPassCols != 0)
    hipLaunchKernelGGL((k_pass<FMT, G, MODE, true, S>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((k_pass<FMT, G, MODE, false, S>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int G, int MODE>
static hipError_t pass_multi_partial(const PassMulti& m, hipStream_t s) {
  bool partial = false;
  for (int k = 0; k < m.n; k++) partial |= m.a[k].n % kPassCols != 0;
  const dim3 grid((unsigned)m.start[m.n]);
  constexpr int S = pass_step_rows<FMT, MODE>();
  if (partial)
    hipLaunchKernelGGL((k_pass_multi<FMT, G, MODE, true, S>), grid, dim3(kBlock), 0, s, m);
  else
    hipLaunchKernelGGL((k_pass_multi<FMT, G, MODE, false, S>), grid, dim3(kBlock), 0, s, m);
  return hipGetLastError();
}

template <int FMT, int MODE>
static hipError_t pass_multi_group(const PassMulti& m, hipStream_t s) {
  switch (m.a[0].G) {
    case 16: return pass_multi_partial<FMT, 16, MODE>(m, s);
    case 32: return pass_multi_partial<FMT, 32, MODE>(m, s);
    case 64: return pass_multi_partial<FMT, 64, MODE>(m, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
static hipError_t pass_multi_mode(int mode, const PassMulti& m, hipStream_t s) {
  switch (mode) {
    case kModeRow: return pass_multi_group<FMT, kModeRow>(m, s);
    case kModeCol: return pass_multi_group<FMT, kModeCol>(m, s);
    case kModeRow | kModeYmax:
      if constexpr (FMT == kNvFp4) return pass_multi_group<FMT, kModeRow | kModeYmax>(m, s);
      return hipErrorInvalidValue;
    case kModeRow | kModeStat:
      if constexpr (FMT != kNvFp4) return pass_multi_group<FMT, kModeRow | kModeStat>(m, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass_multi(int fmt, int mode, const PassMulti& m, hipStream_t s) {
  if (m.n < 1 || m.n > kMaxMulti) return hipErrorInvalidValue;
  switch (fmt) {
    case kInt4Bf16: return pass_multi_mode<kInt4Bf16>(mode, m, s);
    case kMxInt4: return pass_multi_mode<kMxInt4>(mode, m, s);
    case kMxFp4: return pass_multi_mode<kMxFp4>(mode, m, s);
    case kNvFp4: return pass_multi_mode<kNvFp4>(mode, m, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int MODE>
static hipError_t pass_group(const SweepArgs& a, dim3 grid, hipStream_t s) {
  switch (a.G) {
    case 16: return pass_partial<FMT, 16, MODE>(a, grid, s);
    case 32: return pass_partial<FMT, 32, MODE>(a, grid, s);
    case 64: return pass_partial<FMT, 64, MODE>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
static hipError_t pass_mode(int mode, const SweepArgs& a, dim3 grid, hipStream_t s) {
  switch (mode) {
    case kModeRow: return pass_group<FMT, kModeRow>(a, grid, s);
    case kModeCol: return pass_group<FMT, kModeCol>(a, grid, s);
    case kModeRow | kModeEmit: return pass_group<FMT, kModeRow | kModeEmit>(a, grid, s);
    case kModeRow | kModeStat:
      if constexpr (FMT != kNvFp4) return pass_group<FMT, kModeRow | kModeStat>(a, grid, s);
      return hipErrorInvalidValue;  // NVFP4 needs its tensor scale before the first pass
    case kModeRow | kModeYmax:
      if constexpr (FMT == kNvFp4) return pass_group<FMT, kModeRow | kModeYmax>(a, grid, s);
      return hipErrorInvalidValue;  // only NVFP4 has a tensor scale
    default: return hipErrorInvalidValue;
  }
}

int pass_tile_cols() { return kPassCols; }

hipError_t launch_pass(int fmt, int mode, const SweepArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.nct * a.nrc));
  switch (fmt) {
    case kInt4Bf16: return pass_mode<kInt4Bf16>(mode, a, grid, s);
    case kMxInt4: return pass_mode<kMxInt4>(mode, a, grid, s);
    case kMxFp4: return pass_mode<kMxFp4>(mode, a, grid, s);
    case kNvFp4: return pass_mode<kNvFp4>(mode, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dq
