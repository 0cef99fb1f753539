// dq_kernels.hip -- gfx950 kernels of the DualQuant dual-scale solver.
//
// The hot path is a streaming sweep over W (no contraction, so no MFMA): each workgroup of
// four 64-lane waves owns a 512-column tile of a contiguous chunk of rows. A lane owns 8
// consecutive columns (one 128-bit load of bf16, two of fp32) for every row the wave visits,
// so every wave-row load is one contiguous 1 KiB (bf16) segment. Per row the wave forms the
// scaled tile X = fl32(fl32(W * rb) * ra), the group absmax (2/4/8-lane butterfly), the
// inner scale and the codes (recomputed every sweep, never stored until the final emit), and
// then, depending on the mode:
//   row mode    N_i = sum_j W_ij R_ij, D_i = sum_j R_ij^2 with R = Qhat D_b (daiwk notes,
//               "核心公式" eq. 2, left), reduced over the wave and written per column tile;
//   column mode P_j = sum_i W_ij S_ij, Q_j = sum_i S_ij^2 with S = D_a Qhat (eq. 2, right),
//               kept per lane over the chunk's rows, combined over the 4 waves through LDS
//               in fixed order and written per row chunk;
//   emit        packed codes and encoded inner scales.
// Every term W * R or S^2 is an exact product in fp64 and is accumulated in fp64, so the
// sums differ from an exact evaluation only by fp64 rounding; all reductions have a fixed
// order (no floating-point atomics), so results are bit-reproducible.
#include <float.h>

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {

// ------------------------------------------------------------------------------ helpers

template <bool BF>
__device__ __forceinline__ void load8(const void* W, int64_t off, bool active, float w[8]) {
  if (!active) {
#pragma unroll
    for (int k = 0; k < 8; k++) w[k] = 0.0f;
    return;
  }
  if (BF) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      w[2 * k] = u2f(u[k] << 16);
      w[2 * k + 1] = u2f(u[k] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + off);
    const float4 v0 = p[0], v1 = p[1];
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  }
}

__device__ __forceinline__ void atomic_flag(int* status, int flags) {
  if (flags) atomicOr(status, flags);
}

// ------------------------------------------------------------------------------ the sweep

template <int FMT, bool BF, int MODE>
__global__ __launch_bounds__(kBlock) void k_sweep(SweepArgs p) {
  constexpr bool ROW = (MODE & kModeRow) != 0;
  constexpr bool COL = (MODE & kModeCol) != 0;
  constexpr bool EMIT = (MODE & kModeEmit) != 0;
  constexpr bool GAUGE = (MODE & kModeGauge) != 0;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ct = blockIdx.x % p.nct;
  const int rc = blockIdx.x / p.nct;
  const int64_t r_begin = (int64_t)rc * p.rpc;
  const int64_t r_end = r_begin + p.rpc < p.m ? r_begin + p.rpc : p.m;
  const int64_t col0 = (int64_t)ct * kTileCols + lane * kEpl;
  const bool active = col0 < p.n;
  const int lpg = p.G / kEpl;  // lanes per group: 2, 4 or 8

  float rb[8], bb[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    rb[k] = active ? p.rb[col0 + k] : 1.0f;
    bb[k] = active ? p.b[col0 + k] : 0.0f;
  }
  float g = 1.0f, sixg = 6.0f;
  if (FMT == kNvFp4) {
    g = p.gs[0];
    sixg = p.gs[1];
  }

  double P[8], Q[8];
#pragma unroll
  for (int k = 0; k < 8; k++) P[k] = Q[k] = 0.0;
  int flags = 0;

  for (int64_t i = r_begin + wave; i < r_end; i += kWaves) {
    float w[8];
    load8<BF>(p.W, i * p.n + col0, active, w);
    const float ra = p.ra[i];
    float x[8];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      x[k] = (w[k] * rb[k]) * ra;  // column scale first, then row scale; two fp32 roundings
      mx = fmaxf(mx, fabsf(x[k]));
    }
    mx = group_max(mx, lpg);
    if (!(mx <= FLT_MAX)) {  // a scaled value overflowed
      flags |= kStRange;
      mx = 0.0f;
    }
    const GroupQ gq = group_scale<FMT>(mx, g, sixg);
    if (GAUGE && mx > 0.0f) {
      // single-sweep MX identity: re-quantizing with a' = 2^k a, |k| <= 1, must scale the
      // scaled values and the shared exponent exactly and keep the exponent unclamped
      const int ef = (int)((f2u(mx) >> 23) & 0xFFu);
      if (ef < 9 || ef > 249) flags |= kStGauge;
    }
    float q[8];
#pragma unroll
    for (int k = 0; k < 8; k++) q[k] = code_of<FMT>(x[k], gq);

    if (ROW) {
      double nacc = 0.0, dacc = 0.0;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const double t = (double)q[k] * (double)bb[k];  // R / d, exact
        nacc = fma((double)w[k], t, nacc);
        dacc = fma(t, t, dacc);
      }
      const double dd = (double)gq.d;
      nacc *= dd;
      dacc *= dd * dd;
      nacc = wave_sum(nacc);
      dacc = wave_sum(dacc);
      if (lane == 0) p.rowpart[(int64_t)ct * p.m + i] = make_double2(nacc, dacc);
    }
    if (COL) {
      const double c = (double)p.a[i] * (double)gq.d;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const double s = c * (double)q[k];  // S, exact
        P[k] = fma((double)w[k], s, P[k]);
        Q[k] = fma(s, s, Q[k]);
      }
    }
    if (EMIT && active) {
      uint32_t packed = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) packed |= nibble_of<FMT>(q[k]) << (4 * k);
      reinterpret_cast<uint32_t*>(p.codes)[(i * p.n + col0) >> 3] = packed;
      if ((lane % lpg) == 0) {
        const int64_t si = i * (p.n / p.G) + col0 / p.G;
        if (FMT == kInt4Bf16)
          static_cast<uint16_t*>(p.scales)[si] = (uint16_t)gq.scode;
        else
          static_cast<uint8_t*>(p.scales)[si] = (uint8_t)gq.scode;
      }
    }
  }

  if (COL) {
    __shared__ double2 lds[kWaves][kTileCols];
#pragma unroll
    for (int k = 0; k < 8; k++) lds[wave][lane * kEpl + k] = make_double2(P[k], Q[k]);
    __syncthreads();
    for (int c = threadIdx.x; c < kTileCols; c += kBlock) {
      double2 s = lds[0][c];
#pragma unroll
      for (int v = 1; v < kWaves; v++) {
        s.x += lds[v][c].x;
        s.y += lds[v][c].y;
      }
      const int64_t col = (int64_t)ct * kTileCols + c;
      if (col < p.n) p.colpart[(int64_t)rc * p.n + col] = s;
    }
  }
  atomic_flag(p.status, flags);  // rare: only lanes that saw a problem
}

// --------------------------------------------------------------- single-sweep MX pass
// For MXINT4 / MXFP4 on bf16 weights. With E8M0 outer scales the inner scale of a group is
// fixed by y = fl32(W * rb) alone: the group's shared exponent is e = floor(log2 max|y|) - 2 +
// log2(ra), so c = a_i * d_ig = 2^(floor(log2 max|y|) - 2) and the codes are those of y / c.
// Consequently the re-quantization after the row update reproduces the same codes and the
// same S = a d q (daiwk notes, "核心公式": row update, re-quantize, column update), and one
// read of W gives both closed-form updates. With t = S b = a d q b, the reconstruction
// (R = ra_i t), and the residual r = W - t:
//   row i:    M_i = sum_j W_ij r_ij  and  e_i = sum_j r_ij^2, the row's reconstruction error;
//             with E_i = sum_j W_ij^2 the finalize forms N'_i = sum_j W_ij t_ij = E_i - M_i
//             and D'_i = sum_j t_ij^2 = E_i - 2 M_i + e_i (M and e are small next to E, so
//             their fp32 errors shrink in N' and D')
//   column j: P_j = sum_i W_ij S_ij,   Q_j = sum_i S_ij^2
// This holds while every value stays in fp32's normal range with exact products, which is
// guaranteed when every nonzero group max |y| lies in [2^-32, 2^32) and every a, b in
// [2^-24, 2^24]; otherwise the pass raises kStGauge and the solve is redone on the general
// two-sweep path (so does the finalize when a projection decision lies closer to a boundary
// than the error bound of these sums). MXFP4 codes come from gfx950's scaled FP4
// conversion, which rounds y / c to the nearest E2M1 value (ties to even, saturating) exactly
// for power-of-two c; the matching decode returns S = code * c directly.
//
// Layout: a lane owns 16 columns of a 1024-column tile (two 512-column halves, each one
// 128-bit load per row, contiguous across the wave). Products and r = W - t are exact in
// fp32 (r is one fused multiply-add, W - S b); row sums run in fp32 over at most 16 columns
// (a lane's 16, or two neighbouring lanes' 8) and column sums over the chunk's rows; every
// sum above that is fp64 in a fixed order: a row's lane partials are transposed through LDS
// in batches of 8 rows and added by 8 lanes per row, and the 4 waves' column partials are
// added through LDS at the end.
constexpr int kFusedBatch = 8;  // rows per wave between row reductions

// Column sums run in two levels to keep their error small: Pb / Qb over the 8 rows of a
// batch, then P / Q over the batches (a worst case of (7 + batches) * 2^-24 relative).
template <int NH>
struct FusedLane {
  float rb[8 * NH], bb[8 * NH], P[8 * NH], Q[8 * NH], Pb[8 * NH], Qb[8 * NH];
};

// One row of 8 * NH elements (NH 512-column halves of the tile): codes, the row's partial
// sums and the column accumulators. PARTIAL: the tile extends past column n; amask[h]
// zeroes a half that lies past it. mbo[h] returns the bit pattern of the group max of half h,
// which the caller folds into the range it tracks.
// EMIT: the final pass; instead of the sums for the updates it stores the packed codes and
// the E8M0 inner-scale bytes of the row (abits = bits of a_i) and keeps only the row error.
// first: the batch's first row, which starts the batch column sums Pb / Qb.
template <int FMT, int LPG, int NH, bool PARTIAL, bool EMIT, bool STAT>
__device__ __forceinline__ void fused_row(const uint4 (&v)[NH], FusedLane<NH>& L, float& macc,
                                          float& eacc, double& wsq, uint32_t (&mbo)[NH],
                                          const uint32_t (&amask)[NH],
                                          uint32_t* codes_row, uint8_t* scales_row,
                                          uint32_t abits, bool first) {
  macc = 0.0f;
  eacc = 0.0f;
  wsq = 0.0;
#pragma unroll
  for (int h = 0; h < NH; h++) {
    uint32_t u[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
    if (PARTIAL) {
#pragma unroll
      for (int k = 0; k < 4; k++) u[k] &= amask[h];
    }
    float w[8], y[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      w[2 * k] = u2f(u[k] << 16);
      w[2 * k + 1] = u2f(u[k] & 0xFFFF0000u);
    }
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      y[k] = w[k] * L.rb[8 * h + k];
      mx = fmaxf(mx, fabsf(y[k]));
      if (STAT) wsq = fma((double)w[k], (double)w[k], wsq);  // W^2 is exact in fp64
    }
    const uint32_t mb = group_max_bits<LPG>(f2u(mx));
    mbo[h] = mb;
    // c = 2^(floor(log2 mx) - 2). The scaled FP4 conversions read only the exponent field of
    // their fp32 scale, so for MXFP4 the max's own bits less two in the exponent are c; the
    // subtraction saturates at 0 (exponent field 0, the scale 2^-127) for an all-zero group,
    // whose codes are 0 whatever the scale. MXINT4 divides and multiplies by c itself, so there
    // c is an exact power of two and an all-zero group gets a harmless normal one.
    const uint32_t cb = FMT == kMxFp4 ? __builtin_elementwise_sub_sat(mb, 2u << 23)
                                      : max(mb & 0x7F800000u, 3u << 23) - (2u << 23);
    const float c = u2f(cb);
    float S[8];
    uint32_t packed = 0;  // the 8 codes as nibbles, column 2k low (EMIT)
    if (FMT == kMxFp4) {
      // the four conversions write all four bytes, so the first one's other bytes may hold
      // anything (a register that is free anyway saves clearing one)
      uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u[0], y[0], y[1], c, 0);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y[2], y[3], c, 1);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y[4], y[5], c, 2);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, y[6], y[7], c, 3);
      const auto s0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, c, 0);
      const auto s1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, c, 1);
      const auto s2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, c, 2);
      const auto s3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, c, 3);
      S[0] = s0[0]; S[1] = s0[1]; S[2] = s1[0]; S[3] = s1[1];
      S[4] = s2[0]; S[5] = s2[1]; S[6] = s3[0]; S[7] = s3[1];
      if (EMIT) {  // keep the sign bit only where the magnitude is nonzero (no -0 code)
        const uint32_t mag = pk & 0x77777777u;
        const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;
        packed = mag | (pk & nz);
      }
    } else {
      const float ic = u2f((254u << 23) - cb);  // 1 / c
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const float q = fminf(fmaxf(rintf(y[k] * ic), -7.0f), 7.0f);
        S[k] = q * c;
        if (EMIT) packed |= ((uint32_t)(int)q & 0xFu) << (4 * k);
      }
    }
    if (EMIT && (!PARTIAL || amask[h] != 0u)) {  // store inside the matrix only
      // nontemporal: the codes and scales are written once and not read back by the solve
      __builtin_nontemporal_store(packed, codes_row + h * (kTileCols / 8));  // 8 columns of half h
      if ((__lane_id() % LPG) == 0) {
        // E8M0 byte e + 127 with e = floor(log2(mx * ra_i)) - 2 = E(mx) - 129 - log2 a_i
        const uint32_t ey = (mb >> 23) & 0xFFu;
        __builtin_nontemporal_store((uint8_t)(mb == 0u ? 127u : ey + 125u - (abits >> 23)),
                                    scales_row + h * (kTileCols / (8 * LPG)));
      }
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int e = 8 * h + k;
      // the residual W_ij - t_ij with t = S b = a d q b, exact: S b is exact and both have at
      // most 8 significant bits, so the fused multiply-add rounds nothing
      const float df = fmaf(-S[k], L.bb[e], w[k]);
      eacc = fmaf(df, df, eacc);
      if (!EMIT) {
        macc = fmaf(w[k], df, macc);
        L.Pb[e] = first ? w[k] * S[k] : fmaf(w[k], S[k], L.Pb[e]);
        L.Qb[e] = first ? S[k] * S[k] : fmaf(S[k], S[k], L.Qb[e]);
      }
    }
  }
}

// The pass. NH: 512-column halves per lane (the tile is 512 * NH columns); S: rows per load
// step; D: load steps in flight (loads run D steps ahead of the rows being computed, in a ring
// of D + 1 register buffers).
template <int FMT, int G, bool PARTIAL, bool EMIT, int NH, int S, int D, bool STAT>
__global__ __launch_bounds__(kBlock) void k_fused_mx(FusedArgs p) {
  constexpr int LPG = G / kEpl;  // lanes per group
  constexpr int kCols = kTileCols * NH;
  __shared__ float2 smem[kWaves * (kCols > kFusedBatch * kWave ? kCols : kFusedBatch * kWave)];
  // STAT (the first pass): each row's sum of W^2 over the tile's columns, for E_i, which the
  // pass's finalize forms; lane partials in fp64 (every square and sum of squares of bf16
  // values is exact or nearly so there, and never overflows), transposed and added like N
  // and e
  __shared__ double smem_e[STAT ? kWaves * kFusedBatch * kWave : 1];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ct = blockIdx.x % p.nct;
  const int rc = blockIdx.x / p.nct;
  // row and column indices fit 32 bits on this path (the host sends larger matrices to the
  // general single-sweep kernel), which keeps the row bookkeeping in scalar registers
  const int m = (int)p.m, n = (int)p.n;
  const int r_begin = rc * (int)p.rpc;
  const int r_end = r_begin + (int)p.rpc < m ? r_begin + (int)p.rpc : m;
  int col[NH], lcol[NH];
  uint32_t loff[NH];  // byte offset of the lane's 8 columns within a row
  bool act[NH];
  uint32_t amask[NH];
#pragma unroll
  for (int h = 0; h < NH; h++) {
    col[h] = ct * kCols + h * kTileCols + lane * kEpl;
    act[h] = col[h] < n;
    lcol[h] = act[h] ? col[h] : 0;  // in-bounds address
    loff[h] = (uint32_t)lcol[h] * 2u;
    amask[h] = act[h] ? 0xFFFFFFFFu : 0u;
  }

  FusedLane<NH> L;
#pragma unroll
  for (int h = 0; h < NH; h++) {
    const float4* rbp = reinterpret_cast<const float4*>(p.rb + lcol[h]);
    const float4* bbp = reinterpret_cast<const float4*>(p.b + lcol[h]);
    const float4 r0 = rbp[0], r1 = rbp[1], b0 = bbp[0], b1 = bbp[1];
    const float rr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int k = 0; k < 8; k++) {
      L.rb[8 * h + k] = act[h] ? rr[k] : 1.0f;
      L.bb[8 * h + k] = act[h] ? bv[k] : 0.0f;
      L.P[8 * h + k] = L.Q[8 * h + k] = L.Pb[8 * h + k] = L.Qb[8 * h + k] = 0.0f;
    }
  }
  uint32_t gmax = 0u, gmin = 0xFFFFFFFFu;

  // this wave's rows: batches of 8 consecutive rows, 32 rows apart across the workgroup
  const int first = r_begin + wave * kFusedBatch;
  const int nbatch =
      first < r_end ? (r_end - first + kWaves * kFusedBatch - 1) / (kWaves * kFusedBatch) : 0;
  // loads of rows i .. i+S-1 from in-bounds addresses (rows past the chunk reload its first
  // row and are skipped below; columns past n are masked in fused_row): a buffer descriptor
  // per row, built in scalar registers, and the lane's 32-bit offset into it
  auto load = [&](int i, uint4 (&buf)[S][NH]) {
#pragma unroll
    for (int r = 0; r < S; r++) {
      const int row = i + r < r_end ? i + r : r_begin;
      const uint16_t* rowp = p.W + (int64_t)row * n;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(rowp), (short)0, n * 2, 0x00020000);
#pragma unroll
      for (int h = 0; h < NH; h++) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, loff[h], 0u, 0);
        buf[r][h] = make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
  };
  float2* R = smem + wave * (kFusedBatch * kWave);  // this wave's [8 rows][64 lanes] partials
  double* RE = smem_e + (STAT ? wave * (kFusedBatch * kWave) : 0);
  // one row, skipped (uniformly) when it lies past the chunk. Its lane partials go to LDS; a
  // skipped row writes none, since the batch reduction stores only rows inside the chunk. mbo
  // returns the row's group max bits per half (0, which changes no range, for a skipped row).
  auto row_step = [&](const uint4 (&v)[NH], int i, int r, uint32_t (&mbo)[NH]) {
    // a batch's first row always lies inside the chunk (nbatch counts batches that start
    // before r_end); were it skipped, the batch column sums would still restart at zero
    if (r == 0 && !EMIT && !(i < r_end)) {
#pragma unroll
      for (int e = 0; e < 8 * NH; e++) L.Pb[e] = L.Qb[e] = 0.0f;
    }
    if (i < r_end) {
      float n_out, e_out;
      double q_out;
      uint32_t* codes_row = nullptr;
      uint8_t* scales_row = nullptr;
      uint32_t abits = 0u;
      if (EMIT) {
        codes_row = reinterpret_cast<uint32_t*>(p.codes) + (((int64_t)i * n + col[0]) >> 3);
        scales_row = p.scales + (int64_t)i * (n / G) + col[0] / G;
        abits = f2u(p.a[i]);
      }
      fused_row<FMT, LPG, NH, PARTIAL, EMIT, STAT>(v, L, n_out, e_out, q_out, mbo, amask,
                                                   codes_row, scales_row, abits, r == 0);
      R[r * kWave + lane] = make_float2(n_out, e_out);
      if (STAT) RE[r * kWave + lane] = q_out;
    } else {
#pragma unroll
      for (int h = 0; h < NH; h++) mbo[h] = 0u;
    }
  };

  // a batch is kFusedBatch / S load steps; before step st computes, the loads of step st + D
  // (of this batch or the next) go out into the buffer step st - 1 has just used, so each
  // step's rows were requested D steps earlier
  constexpr int kSteps = kFusedBatch / S;
  constexpr int NB = D + 1;
  static_assert(kSteps % NB == 0, "a batch is a whole number of turns of the buffer ring");
  uint4 buf[NB][S][NH];
  if (nbatch > 0) {
#pragma unroll
    for (int j = 0; j < D; j++) load(first + j * S, buf[j]);
  }
  for (int bt = 0; bt < nbatch; bt++) {
    const int row0 = first + bt * (kWaves * kFusedBatch);
#pragma unroll
    for (int st = 0; st < kSteps; st++) {
      const int ls = st + D;
      if (ls < kSteps)
        load(row0 + ls * S, buf[ls % NB]);
      else if (bt + 1 < nbatch)
        load(row0 + kWaves * kFusedBatch + (ls - kSteps) * S, buf[ls % NB]);
      uint32_t mbs[S][NH];
#pragma unroll
      for (int r = 0; r < S; r++) row_step(buf[st % NB][r], row0 + st * S + r, st * S + r, mbs[r]);
      // the range of the step's group maxima: gmax the largest, gmin the smallest nonzero one
      // less one (a zero group wraps to 0xFFFFFFFF and never counts)
#pragma unroll
      for (int h = 0; h < NH; h++) {
        if (S == 2) {
          gmax = max(gmax, max(mbs[0][h], mbs[1][h]));
          gmin = min(gmin, min(mbs[0][h] - 1u, mbs[1][h] - 1u));
        } else {
#pragma unroll
          for (int r = 0; r < S; r++) {
            gmax = max(gmax, mbs[r][h]);
            gmin = min(gmin, mbs[r][h] - 1u);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (!EMIT) {  // the next batch's first row restarts Pb / Qb
#pragma unroll
      for (int e = 0; e < 8 * NH; e++) {
        L.P[e] += L.Pb[e];
        L.Q[e] += L.Qb[e];
      }
    }

    // 8 rows done: 8 lanes per row add 8 lane partials each (transposed through LDS), then
    // across the 8 lanes in a fixed order. With 8 columns per lane, neighbouring lanes'
    // partials are first added in fp32 (a 16-column sum, inside the same error bound as a
    // lane's 16 columns); every addition above is fp64.
    __builtin_amdgcn_wave_barrier();
    const float2* src = R + (lane >> 3) * kWave + (lane & 7) * 8;
    float2 v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = src[k];
    double N, Er;
    if (NH == 1) {
      N = (double)(v[0].x + v[1].x);
      Er = (double)(v[0].y + v[1].y);
#pragma unroll
      for (int k = 2; k < 8; k += 2) {
        N += (double)(v[k].x + v[k + 1].x);
        Er += (double)(v[k].y + v[k + 1].y);
      }
    } else {
      N = (double)v[0].x;
      Er = (double)v[0].y;
#pragma unroll
      for (int k = 1; k < 8; k++) {
        N += (double)v[k].x;
        Er += (double)v[k].y;
      }
    }
    N = sum8_dpp(N);
    Er = sum8_dpp(Er);
    const int i = row0 + (lane >> 3);
    if ((lane & 7) == 0 && i < r_end) p.rowpart[(int64_t)ct * m + i] = make_double2(N, Er);
    if (STAT) {
      const double* srce = RE + (lane >> 3) * kWave + (lane & 7) * 8;
      double Q = 0.0;
#pragma unroll
      for (int k = 0; k < 8; k++) Q += srce[k];
      Q = sum8_dpp(Q);
      if ((lane & 7) == 0 && i < r_end) p.epart[(int64_t)ct * m + i] = Q;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // column partials: the 4 waves' fp32 sums added in fp64 in wave order
  if (!EMIT) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; h++)
#pragma unroll
      for (int k = 0; k < 8; k++)
        smem[wave * kCols + h * kTileCols + lane * kEpl + k] = make_float2(L.P[8 * h + k], L.Q[8 * h + k]);
    __syncthreads();
    for (int c = threadIdx.x; c < kCols; c += kBlock) {
      double sp = 0.0, sq = 0.0;
#pragma unroll
      for (int v = 0; v < kWaves; v++) {
        sp += (double)smem[v * kCols + c].x;
        sq += (double)smem[v * kCols + c].y;
      }
      const int j = ct * kCols + c;
      if (j < n) p.colpart[(int64_t)rc * n + j] = make_double2(sp, sq);
    }
  }
  // range check: every nonzero group max in [2^-32, 2^32)
  const bool bad = gmax >= 0x4F800000u || (gmin != 0xFFFFFFFFu && gmin + 1u < 0x2F800000u);
  atomic_flag(p.status, bad ? kStGauge : 0);
}

// ------------------------------------------------------------------------- row statistics
// E_i = sum_j W_ij^2 (fp64, fixed order), a non-finite check on W, and (AMAX) the row max of
// |X| at the initial scales (NVFP4 tensor scale). One wave per row; each step has four
// 512-column tiles in flight, summed into four accumulators that are added in a fixed order.
constexpr int kStatTiles = 4;

template <bool BF, bool AMAX>
__global__ __launch_bounds__(kBlock) void k_rowstat(RowStatArgs p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t i = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  if (i >= p.m) return;
  double e[kStatTiles];
#pragma unroll
  for (int u = 0; u < kStatTiles; u++) e[u] = 0.0;
  float mx = 0.0f;
  const float ra = AMAX ? p.ra[i] : 1.0f;
  for (int64_t c0 = (int64_t)lane * kEpl; c0 < p.n; c0 += kStatTiles * kTileCols) {
    float w[kStatTiles][8], rb[kStatTiles][8];
#pragma unroll
    for (int u = 0; u < kStatTiles; u++) {
      const int64_t c = c0 + u * kTileCols;
      const bool act = c < p.n;
      load8<BF>(p.W, i * p.n + c, act, w[u]);
      if (AMAX) {
        float4 r0 = make_float4(1.0f, 1.0f, 1.0f, 1.0f), r1 = r0;
        if (act) {
          r0 = reinterpret_cast<const float4*>(p.rb + c)[0];
          r1 = reinterpret_cast<const float4*>(p.rb + c)[1];
        }
        rb[u][0] = r0.x; rb[u][1] = r0.y; rb[u][2] = r0.z; rb[u][3] = r0.w;
        rb[u][4] = r1.x; rb[u][5] = r1.y; rb[u][6] = r1.z; rb[u][7] = r1.w;
      }
    }
#pragma unroll
    for (int u = 0; u < kStatTiles; u++)
#pragma unroll
      for (int k = 0; k < 8; k++) {
        e[u] = fma((double)w[u][k], (double)w[u][k], e[u]);
        if (AMAX) mx = fmaxf(mx, fabsf((w[u][k] * rb[u][k]) * ra));
      }
  }
  static_assert(kStatTiles == 4, "the fixed order below adds four accumulators");
  double et = (e[0] + e[1]) + (e[2] + e[3]);
  et = wave_sum(et);
  if (AMAX) mx = wave_max(mx);
  if (lane == 0) {
    p.E[i] = et;
    if (AMAX) p.amax[i] = mx;
    int f = 0;
    if (!(et <= DBL_MAX)) f |= kStNonFinite;     // W^2 never overflows fp64: E is finite
    if (AMAX && !(mx <= FLT_MAX)) f |= kStRange;  // iff W is
    atomic_flag(p.status, f);
  }
}

// ----------------------------------------------------------------------------- small kernels

__global__ void k_clear(int* words, int count) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < count) words[t] = 0;
}

// outer scales: dst = Pi_F(src) (or src as given, or 1) and its synced inner copy fl32(1/dst)
__global__ void k_vec(VecArgs p) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= p.len) return;
  float v = 1.0f;
  if (p.src) {
    v = p.src[k];
    if (!(v > 0.0f) || !(v <= FLT_MAX)) {
      atomic_flag(p.status, kStInitArg);
      v = 1.0f;
    }
    if (p.project) v = project(p.fmt, (double)v);
  }
  if (p.envelope && !(v >= 0x1p-24f && v <= 0x1p24f)) atomic_flag(p.status, kStGauge);
  p.dst[k] = v;
  p.rdst[k] = recip32(v);
  if (p.dst2) p.dst2[k] = v;
}

// NVFP4 tensor scale g = fl32(A / 2688) (2688 = 6 * 448), at least 2^-126; 1 if A = 0.
constexpr int kScaleThreads = 1024;

__global__ __launch_bounds__(kScaleThreads) void k_tensor_scale(ScaleArgs p) {
  __shared__ float red[kScaleThreads];
  float mx = 0.0f;
  constexpr int kU = 8;  // loads in flight per thread
  for (int64_t i0 = threadIdx.x; i0 < p.m; i0 += (int64_t)kU * kScaleThreads) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int64_t i = i0 + (int64_t)u * kScaleThreads;
      v[u] = i < p.m ? p.amax[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; u++) mx = fmaxf(mx, v[u]);
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = kScaleThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float g;
    const float given = p.g_in ? *p.g_in : p.g_fixed;
    if (given > 0.0f) {
      g = given;
    } else {
      const float A = red[0];
      g = A == 0.0f ? 1.0f : fmaxf((float)((double)A / 2688.0), 0x1p-126f);
    }
    if (!(g <= FLT_MAX)) {
      atomic_flag(p.status, kStRange);
      g = 1.0f;
    }
    p.gs[0] = g;
    p.gs[1] = 6.0f * g;
    if (p.g_out) *p.g_out = g;
  }
}

// Relative distance of v > 0 from the nearest decision point of the E8M0 projection
// (1.5 * 2^k). The single-sweep sums are trusted only where it exceeds twice their error
// bound, so that the decision is the one exact sums would give.
__device__ __forceinline__ double e8m0_margin(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const double f = __builtin_bit_cast(double, (u & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  return fabs(f - 1.5) / f;  // f in [1, 2): the mantissa of v
}
// Worst-case relative error of an fp32 sum of k nonnegative terms is (k - 1) * 2^-24; the
// single-sweep lane sums run over at most 16 columns (row sums), and FinArgs::col_terms
// bounds the additions behind a column sum.
constexpr double kRowSumErr = 16.0 * 0x1p-24;

// sum of cnt double2 partials at base, base + stride, ... in index order, loads issued first
__device__ __forceinline__ double2 sum_parts(const double2* base, int64_t stride, int first,
                                             int step, int cnt) {
  double N = 0.0, D = 0.0;
  constexpr int kU = 8;
  for (int k0 = first; k0 < cnt; k0 += kU * step) {
    double2 v[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int k = k0 + u * step;
      v[u] = k < cnt ? base[(int64_t)k * stride] : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int u = 0; u < kU; u++) {
      N += v[u].x;
      D += v[u].y;
    }
  }
  return make_double2(N, D);
}

// mean of the per-block error sums: thread k adds blocks k, k + 256, ..., then a fixed tree
__device__ void mse_collect(const double* part, int count, double* out, double inv_mn,
                            double* red) {
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int k = tid; k < count; k += 256) s += part[k];
  s = block_sum4(s, red);
  if (tid == 0) *out = s * inv_mn;
}

__global__ __launch_bounds__(256) void k_mse_collect(const double* part, int count, double* out,
                                                     double inv_mn) {
  __shared__ double red[256];
  mse_collect(part, count, out, inv_mn, red);
}

// Closed-form updates (eq. 2) and projections, plus the error of the state the row sums were
// taken at, e_i = E_i - 2 a_i N_i + a_i^2 D_i (or the directly summed row error). Per block
// the row errors are added in a fixed order (block_sum4: lane trees, then waves) into
// part_out; the next finalize (or a final collect kernel) adds the block sums in a fixed
// order.
__device__ __forceinline__ void finalize_block(const FinArgs& p, int bid) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  if (bid == 0 && p.prev_out) {
    // the previous finalize's per-block error sums (visible across the kernel boundary)
    mse_collect(p.prev_part, p.prev_count, p.prev_out, p.inv_mn, red);
    __syncthreads();
  }
  if (bid < p.nblk_rows) {
    const int64_t i = (int64_t)bid * 256 + tid;
    double err = 0.0;
    int flags = 0;
    if (i < p.m && p.rowerr) {
      err = p.rowerr[i];  // formed by the row-resident pass, which also updated a
    } else if (i < p.m) {
      if (p.epart) {  // E_i from the first pass's tile partials, in tile order
        double e2 = 0.0;
        for (int k = 0; k < p.nct; k++) e2 += p.epart[(int64_t)k * p.m + i];
        p.E[i] = e2;
        if (!(e2 <= DBL_MAX)) flags |= kStNonFinite;  // W^2 never overflows fp64: iff W is
      }
      const double2 nd = sum_parts(p.rowpart + i, p.m, 0, 1, p.nct);
      double N = nd.x, D = nd.y;
      double rel_err = 0.0;  // error bound of N / D (single-sweep sums only)
      const double ai = (double)p.a[i];
      if (p.row_ra) {
        // single-sweep sums: M = sum W r and e = sum r^2 with the residual r = W - t and
        // R = ra_i t; N' = sum W t = E - M and D' = sum t^2 = E - 2 M + e
        const double M = N, e = D, Ei = p.E[i];
        err = e;
        const double Np = Ei - M;
        const double Dp = Ei - 2.0 * M + e;
        // Inside the envelope a row with a nonzero code has D' >= 2^-114 (its largest |W| is
        // at least 2^-56 and t there at least half of it); D' below 2^-200 means every code
        // of the row is 0 (W zero, or so small that y = W rb underflowed): D = 0, a = 1.
        const bool zero_row = !(Dp >= 0x1p-200);
        const double r = (double)p.ra[i];
        N = zero_row ? 0.0 : Np * r;
        D = zero_row ? 0.0 : Dp * r * r;
        // error bounds: E's fp64 sums (no chain longer than n/64 + 64 additions), the fp32
        // lane sums (sum |W r| <= sqrt(E e) by Cauchy-Schwarz, sum r^2 = e) and the two fp64
        // operations here
        const double eE = ((double)p.n * (1.0 / 64.0) + 64.0) * 0x1p-53 * Ei;
        const double cs = sqrt(Ei * e) * (1.0 + 0x1p-20);
        const double dN = eE + kRowSumErr * cs + 0x1p-50 * (Ei + fabs(M));
        const double dD = eE + kRowSumErr * (2.0 * cs + e) + 0x1p-50 * (Ei + 2.0 * fabs(M) + e);
        rel_err = zero_row ? 0.0 : dN / Np + dD / Dp;
      } else {
        err = fmax(p.E[i] - 2.0 * ai * N + ai * ai * D, 0.0);
      }
      float Y = 0.0f;  // max over this row of |y| = |fl32(W rb)|, from the row pass's tiles
      if (p.ymax)
        for (int k = 0; k < p.nct; k++) Y = fmaxf(Y, p.ymax[(int64_t)k * p.m + i]);
      if (p.update_a) {
        float an = 1.0f;  // an all-zero code slice keeps scale 1
        if (D > 0.0) {
          if (!(N > 0.0)) flags |= kStInternal;
          an = project(p.fmt, N / D);
          if (p.row_ra && e8m0_margin(N / D) < 2.0 * rel_err) flags |= kStGauge;
        }
        if (p.gauge_check) {
          const float ao = p.a[i];
          if (!(an == ao || an == 2.0f * ao || an == 0.5f * ao)) flags |= kStGauge;
        }
        if (p.envelope && !(an >= 0x1p-24f && an <= 0x1p24f)) flags |= kStGauge;
        p.a[i] = an;
        p.ra[i] = recip32(an);
        // the next pass's row max of |x| = |fl32(y ra')|: fl32 is monotone, so it is
        // fl32(max |y| * ra') exactly
        if (p.ymax) p.amax_out[i] = Y * p.ra[i];
      }
    }
    const double esum = block_sum4(err, red);
    if (flags) atomicOr(p.status, flags);
    if (tid == 0 && p.part_out) p.part_out[bid] = esum;
  } else {
    // 32 lanes per column: lane s adds partials s, s + 32, ... in order (one round of loads
    // for up to 256 row chunks), then a fixed tree over the 32 lanes
    const int64_t j = (int64_t)(bid - p.nblk_rows) * kFinColsPerBlock + tid / 32;
    const int sub = tid & 31;
    double2 nd = make_double2(0.0, 0.0);
    if (j < p.n) nd = sum_parts(p.colpart + j, p.n, sub, 32, p.nrc);
    const double N = sum32_lanes(nd.x);
    const double D = sum32_lanes(nd.y);
    if (j >= p.n || sub != 0) return;
    float bn = 1.0f;
    if (D > 0.0) {
      if (!(N > 0.0)) atomicOr(p.status, kStInternal);
      bn = project(p.fmt, N / D);
      // N and D each carry at most col_terms * 2^-24 relative error
      if (p.row_ra && e8m0_margin(N / D) < 4.0 * p.col_terms * 0x1p-24) atomicOr(p.status, kStGauge);
    }
    if (p.envelope && !(bn >= 0x1p-24f && bn <= 0x1p24f)) atomicOr(p.status, kStGauge);
    p.b[j] = bn;
    p.rb[j] = recip32(bn);
  }
}

__global__ __launch_bounds__(256) void k_finalize(FinArgs p) { finalize_block(p, blockIdx.x); }

__global__ __launch_bounds__(256) void k_finalize_multi(FinMulti m) {
  int k = 0;
  while (k + 1 < m.n && (int)blockIdx.x >= m.start[k + 1]) k++;
  finalize_block(m.a[k], (int)blockIdx.x - m.start[k]);
}

// ------------------------------------------------------------------------------- launchers

__global__ __launch_bounds__(256) void k_flush(const uint4* buf, size_t n, int* sink) {
  uint32_t acc = 0u;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) *sink = (int)acc;  // a scratch word; keeps the loads alive
}

hipError_t launch_flush(const void* buf, size_t vec16, int* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_flush, dim3(2048), dim3(256), 0, s, static_cast<const uint4*>(buf), vec16, sink);
  return hipGetLastError();
}

hipError_t launch_clear(int* words, int count, hipStream_t s) {
  hipLaunchKernelGGL(k_clear, dim3((count + 63) / 64), dim3(64), 0, s, words, count);
  return hipGetLastError();
}

hipError_t launch_vec(const VecArgs& a, hipStream_t s) {
  const int64_t blocks = (a.len + 255) / 256;
  hipLaunchKernelGGL(k_vec, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowstat(bool bf16, const RowStatArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.m + kWaves - 1) / kWaves));
  if (bf16) {
    if (a.amax)
      hipLaunchKernelGGL((k_rowstat<true, true>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((k_rowstat<true, false>), grid, dim3(kBlock), 0, s, a);
  } else {
    if (a.amax)
      hipLaunchKernelGGL((k_rowstat<false, true>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((k_rowstat<false, false>), grid, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_tensor_scale(const ScaleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(kScaleThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mse_collect(const double* part, int count, double* out, double inv_mn,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_mse_collect, dim3(1), dim3(256), 0, s, part, count, out, inv_mn);
  return hipGetLastError();
}

hipError_t launch_finalize_multi(const FinMulti& m, hipStream_t s) {
  if (m.n < 1 || m.n > kMaxMulti) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_finalize_multi, dim3((unsigned)m.start[m.n]), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_finalize, dim3(a.nblk_rows + a.nblk_cols), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool PARTIAL, bool EMIT, int NH, int S, int D, bool STAT>
static hipError_t fused_group(const FusedArgs& a, dim3 grid, hipStream_t s) {
  switch (a.G) {
    case 16: hipLaunchKernelGGL((k_fused_mx<FMT, 16, PARTIAL, EMIT, NH, S, D, STAT>), grid, dim3(kBlock), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_fused_mx<FMT, 32, PARTIAL, EMIT, NH, S, D, STAT>), grid, dim3(kBlock), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_fused_mx<FMT, 64, PARTIAL, EMIT, NH, S, D, STAT>), grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, bool EMIT, int NH, int S, int D, bool STAT>
static hipError_t fused_shape(const FusedArgs& a, dim3 grid, hipStream_t s) {
  // masking only when some tile extends past the last column
  return a.n % (kTileCols * NH) != 0 ? fused_group<FMT, true, EMIT, NH, S, D, STAT>(a, grid, s)
                                     : fused_group<FMT, false, EMIT, NH, S, D, STAT>(a, grid, s);
}

// (halves, rows per step, steps in flight): (1, 2, 1), (1, 2, 3), (1, 4, 1), (2, 2, 1), (2, 4, 1)
template <int FMT, bool EMIT, bool STAT>
static hipError_t fused_variant(const FusedArgs& a, dim3 grid, hipStream_t s) {
  if (a.halves == 1) {
    if (a.step_rows == 4) return fused_shape<FMT, EMIT, 1, 4, 1, STAT>(a, grid, s);
    return a.ahead == 3 ? fused_shape<FMT, EMIT, 1, 2, 3, STAT>(a, grid, s)
                        : fused_shape<FMT, EMIT, 1, 2, 1, STAT>(a, grid, s);
  }
  return a.step_rows == 4 ? fused_shape<FMT, EMIT, 2, 4, 1, STAT>(a, grid, s)
                          : fused_shape<FMT, EMIT, 2, 2, 1, STAT>(a, grid, s);
}

template <int FMT>
static hipError_t fused_fmt(bool emit, const FusedArgs& a, dim3 grid, hipStream_t s) {
  if (emit) return fused_variant<FMT, true, false>(a, grid, s);
  return a.epart ? fused_variant<FMT, false, true>(a, grid, s)
                 : fused_variant<FMT, false, false>(a, grid, s);
}

hipError_t launch_fused(int fmt, bool emit, const FusedArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.nct * a.nrc));
  if (fmt == kMxFp4) return fused_fmt<kMxFp4>(emit, a, grid, s);
  if (fmt == kMxInt4) return fused_fmt<kMxInt4>(emit, a, grid, s);
  return hipErrorInvalidValue;
}

template <int FMT, bool BF>
static hipError_t sweep_mode(int mode, const SweepArgs& a, dim3 grid, hipStream_t s) {
  switch (mode) {
    case kModeRow: hipLaunchKernelGGL((k_sweep<FMT, BF, kModeRow>), grid, dim3(kBlock), 0, s, a); break;
    case kModeCol: hipLaunchKernelGGL((k_sweep<FMT, BF, kModeCol>), grid, dim3(kBlock), 0, s, a); break;
    case kModeRow | kModeCol | kModeGauge:
      hipLaunchKernelGGL((k_sweep<FMT, BF, kModeRow | kModeCol | kModeGauge>), grid, dim3(kBlock), 0, s, a);
      break;
    case kModeEmit | kModeRow:
      hipLaunchKernelGGL((k_sweep<FMT, BF, kModeEmit | kModeRow>), grid, dim3(kBlock), 0, s, a);
      break;
    case kModeEmit: hipLaunchKernelGGL((k_sweep<FMT, BF, kModeEmit>), grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t sweep_dtype(bool bf16, int mode, const SweepArgs& a, dim3 grid, hipStream_t s) {
  return bf16 ? sweep_mode<FMT, true>(mode, a, grid, s) : sweep_mode<FMT, false>(mode, a, grid, s);
}

hipError_t launch_sweep(int fmt, bool bf16, int mode, const SweepArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.nct * a.nrc));
  switch (fmt) {
    case kInt4Bf16: return sweep_dtype<kInt4Bf16>(bf16, mode, a, grid, s);
    case kMxInt4: return sweep_dtype<kMxInt4>(bf16, mode, a, grid, s);
    case kMxFp4: return sweep_dtype<kMxFp4>(bf16, mode, a, grid, s);
    case kNvFp4: return sweep_dtype<kNvFp4>(bf16, mode, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dq
