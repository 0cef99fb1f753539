// dq_rowres.hip -- the row-resident iteration pass: one read of W per iteration for the
// formats whose row update changes the codes (INT4_BF16, NVFP4), on bf16 weights.
//
// An iteration quantizes every element twice (daiwk notes, "核心公式": quantize, row update,
// re-quantize with the inner copies synced, column update). The re-quantization after the row
// update needs only each row's own new scale a'_i, so a workgroup that owns whole rows can do
// both Q evaluations of a row from one load of it:
//   phase 1  Q of the row with the current ra_i; the lane's parts of N_i = sum_j W_ij R_ij and
//            D_i = sum_j R_ij^2 with R = Qhat D_b;
//   update   the row's sums over the workgroup (fixed order), e_i = E_i - 2 a_i N_i +
//            a_i^2 D_i for mse, a'_i = Pi(N_i / D_i) (1 for an all-zero code slice), ra'_i;
//   phase 2  Q of the same row, still in registers, with ra'_i; the lane's column sums
//            P_j += W_ij S_ij and Q_j += S_ij^2 with S = D_a' Qhat'.
// Each workgroup then writes its column sums as one row of partials; the column finalize adds
// them in workgroup order and projects b. The per-row errors go to memory, and that finalize
// adds them in a fixed order for mse[t].
//
// Layout: lane l of the workgroup owns columns E l .. E l + E - 1 (E = 8: one 128-bit load per
// row), so a workgroup of n / E lanes spans a whole row and a group of G
// columns spans G / E lanes. Rows go in batches of B: the loads of the next batch are issued
// before the current one is computed. A batch's lane parts of N and D are reduced across the
// wave by a transposing butterfly (each exchange halves the rows a lane carries), then across
// the waves through LDS in wave order.
//
// Arithmetic: every product is exact in fp64 (W q b, (q b)^2, W a d q, (a d q)^2) and every
// sum is fp64 in a fixed order, as in the two-sweep pass; the codes are the same exact codes
// (snapped double quotient), so the result equals the two-sweep path's up to the order of
// fp64 additions.
#include <float.h>

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {

constexpr int kRrMaxWaves = 8;

// Sum over the 64 lanes of each of the B rows' (N, D) lane parts, in a fixed order. Returns
// in every lane l the sums of row rr_row<B>(l) (a transposing butterfly over lane bits 0..log2
// B - 1, each step keeping half of the rows, then a plain butterfly over the other bits).
template <int B>
__device__ __forceinline__ int rr_row(int lane) {
  int r = 0;
#pragma unroll
  for (int s = 0, half = B / 2; half >= 1; s++, half /= 2)
    if (lane & (1 << s)) r += half;
  return r;
}

template <int B>
__device__ __forceinline__ double2 rr_wave_sums(double (&n)[B], double (&d)[B], int lane) {
  int m = 1;
#pragma unroll
  for (int half = B / 2; half >= 1; half /= 2, m <<= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < half; j++) {
      const double sn = up ? n[j] : n[j + half], sd = up ? d[j] : d[j + half];
      const double kn = up ? n[j + half] : n[j], kd = up ? d[j + half] : d[j];
      n[j] = kn + __shfl_xor(sn, m, kWave);
      d[j] = kd + __shfl_xor(sd, m, kWave);
    }
  }
  double N = n[0], D = d[0];
#pragma unroll
  for (; m < kWave; m <<= 1) {
    N += __shfl_xor(N, m, kWave);
    D += __shfl_xor(D, m, kWave);
  }
  return make_double2(N, D);
}

// One row of this lane's E elements quantized with row scale ra: the codes as values (exact
// fp64), the group's divisor d, and a range flag. w receives the weights.
template <int FMT, int E, int LPG, bool PARTIAL>
__device__ __forceinline__ double rr_quantize(const uint4 (&v)[E / 8], const float (&rb)[E],
                                              float ra, float g, float sixg, double r6,
                                              uint32_t amask, float (&w)[E], double (&q)[E],
                                              int& flags) {
  float x[E];
  float mx = 0.0f;
#pragma unroll
  for (int h = 0; h < E / 8; h++) {
    uint32_t u[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      if (PARTIAL) u[k] &= amask;
      w[8 * h + 2 * k] = u2f(u[k] << 16);
      w[8 * h + 2 * k + 1] = u2f(u[k] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int k = 0; k < E; k++) {
    const float y = w[k] * rb[k];  // column scale first, then row scale: two fp32 roundings
    x[k] = y * ra;
    mx = fmaxf(mx, fabsf(x[k]));
  }
  float gm = mx;
  if (LPG > 1) gm = u2f(group_max_bits<LPG>(f2u(mx)));
  if (!(gm <= FLT_MAX)) {  // a scaled value overflowed
    flags |= kStRange;
    gm = 0.0f;
  }
  const GroupQ gq = FMT == kNvFp4 ? nv_group_scale(gm, g, r6) : group_scale<FMT>(gm, g, sixg);
  const double r = recip64(gq.d);
  if (FMT == kInt4Bf16 && __any(int4_needs_clamp(gq.d))) {  // rare: a subnormal scale
#pragma unroll
    for (int k = 0; k < E; k++) q[k] = int4_clamp(code64<FMT>(x[k], r, gq));
  } else {
#pragma unroll
    for (int k = 0; k < E; k++) q[k] = code64<FMT>(x[k], r, gq);
  }
  return (double)gq.d;
}

// The pass on workgroup `bid` of one matrix's grid.
template <int FMT, int G, int E, int B, bool PARTIAL>
__device__ __forceinline__ void rowres_block(const RowResArgs& p, int bid) {
  constexpr int LPG = G / E;  // lanes per group (E <= G)
  constexpr int V = E / 8;    // 128-bit loads per row
  __shared__ double2 red[2][B][kRrMaxWaves];  // per row, each wave's (N, D); two batches
  __shared__ float anew[2][B][2];             // per row, a' and ra'; two batches

  const uint16_t* W = p.W;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = (int)(blockDim.x / kWave);
  const int64_t col = (int64_t)threadIdx.x * E;
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

  const int64_t r0 = (int64_t)bid * p.rpc;
  const int64_t r1 = r0 + p.rpc < p.m ? r0 + p.rpc : p.m;

  // loads of rows i .. i + B - 1 (rows past the workgroup's last reload its first row; they
  // are skipped below)
  auto load = [&](int64_t i, uint4 (&buf)[B][V]) {
#pragma unroll
    for (int r = 0; r < B; r++) {
      const int64_t row = i + r < r1 ? i + r : r0;
      const uint4* src = reinterpret_cast<const uint4*>(W + row * p.n + lcol);
#pragma unroll
      for (int h = 0; h < V; h++) buf[r][h] = src[h];
    }
  };

  // the row values of a batch: lane l holds those of row i0 + l % B (clamped into the
  // workgroup's rows): ra for phase 1 (taken with a readlane), a and E for the update
  struct RowVals {
    float ra, a;
    double wsq;  // E_i = sum_j W_ij^2
  };
  auto load_vals = [&](int64_t i0, RowVals& rv) {
    int64_t i = i0 + (lane % B);
    i = i < r1 ? i : r0;
    rv.ra = p.ra[i];
    rv.a = p.a[i];
    rv.wsq = p.E[i];
  };

  // phase 1 of the batch at i0: codes with the current row scales; the wave's sums of each
  // row's lane parts of N and D go to red[slot]
  auto phase1 = [&](const uint4 (&buf)[B][V], const RowVals& rv, int64_t i0, int slot) {
    double nb[B], db[B];
#pragma unroll
    for (int r = 0; r < B; r++) {
      nb[r] = db[r] = 0.0;
      if (i0 + r < r1) {  // uniform across the workgroup
        float w[E];
        double q[E];
        const float ra = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rv.ra), r));
        const double dd = rr_quantize<FMT, E, LPG, PARTIAL>(buf[r], rb, ra, g, sixg, r6, amask,
                                                             w, q, flags);
        double nl = 0.0, dl = 0.0;
#pragma unroll
        for (int k = 0; k < E; k++) {
          const double t = q[k] * bbd[k];  // R / d, exact
          nl = fma((double)w[k], t, nl);
          dl = fma(t, t, dl);
        }
        nb[r] = nl * dd;
        db[r] = dl * (dd * dd);
      }
    }
    const double2 sums = rr_wave_sums<B>(nb, db, lane);
    if (lane < B) red[slot][rr_row<B>(lane)][wave] = sums;
  };

  // the update of the batch at i0 (after a barrier that makes red[slot] visible): row r by
  // lane r of wave r % nw, so that the waves share the work
  auto update = [&](const RowVals& rv, int64_t i0, int slot) {
    const int r = lane;
    if (r >= B || r % nw != wave) return;
    const int64_t i = i0 + r;
    float an = 1.0f, ran = 1.0f;
    if (i < r1) {
      double N = 0.0, D = 0.0;
      for (int k = 0; k < nw; k++) {  // wave order
        N += red[slot][r][k].x;
        D += red[slot][r][k].y;
      }
      const double ai = (double)rv.a;
      p.rowerr[i] = fmax(rv.wsq - 2.0 * ai * N + ai * ai * D, 0.0);
      if (D > 0.0) {  // else an all-zero code slice: scale 1
        if (!(N > 0.0)) flags |= kStInternal;
        an = project(FMT, N / D);
      }
      ran = recip32(an);
      p.a[i] = an;
      p.ra[i] = ran;
    }
    anew[slot][r][0] = an;
    anew[slot][r][1] = ran;
  };

  // phase 2 of the batch at i0 (after a barrier that makes anew[slot] visible): codes with the
  // new row scales, the lane's column sums
  auto phase2 = [&](const uint4 (&buf)[B][V], int64_t i0, int slot) {
#pragma unroll
    for (int r = 0; r < B; r++) {
      if (i0 + r < r1) {
        // the row's words made opaque, so that phase 1's unpacked and converted weights are
        // recomputed here rather than kept alive between the phases
        uint4 v[V];
#pragma unroll
        for (int h = 0; h < V; h++) {
          v[h] = buf[r][h];
          asm volatile("" : "+v"(v[h].x), "+v"(v[h].y), "+v"(v[h].z), "+v"(v[h].w));
        }
        float w[E];
        double q[E];
        const double dd = rr_quantize<FMT, E, LPG, PARTIAL>(v, rb, anew[slot][r][1], g, sixg,
                                                             r6, amask, w, q, flags);
        const double c = (double)anew[slot][r][0] * dd;  // a'_i d'_ig, exact
#pragma unroll
        for (int k = 0; k < E; k++) {
          const double sv = c * q[k];  // S, exact
          P[k] = fma((double)w[k], sv, P[k]);
          Q[k] = fma(sv, sv, Q[k]);
        }
      }
    }
  };

  // Software pipeline over the batches, one barrier per batch: iteration k runs phase 1 of
  // batch k + 1, the barrier, the update of batch k + 1 and phase 2 of batch k (whose update
  // the previous iteration made). Rows are loaded two batches ahead, through three buffers.
  const int64_t nbat = (r1 - r0 + B - 1) / B;
  uint4 cur[B][V], nxt[B][V], pre[B][V];
  RowVals vcur{}, vnxt{}, vpre{};
  if (nbat > 0) {
    load(r0, cur);
    load_vals(r0, vcur);
  }
  if (nbat > 1) {
    load(r0 + B, nxt);
    load_vals(r0 + B, vnxt);
  }
  if (nbat > 2) {
    load(r0 + 2 * B, pre);
    load_vals(r0 + 2 * B, vpre);
  }
  if (nbat > 0) phase1(cur, vcur, r0, 0);
  __syncthreads();
  if (nbat > 0) update(vcur, r0, 0);
  for (int64_t k = 0; k < nbat; k++) {
    const int64_t i0 = r0 + k * B;
    const int slot = (int)(k & 1);
    if (k + 1 < nbat) phase1(nxt, vnxt, i0 + B, slot ^ 1);
    __syncthreads();
    if (k + 1 < nbat) update(vnxt, i0 + B, slot ^ 1);
    phase2(cur, i0, slot);
#pragma unroll
    for (int r = 0; r < B; r++)
#pragma unroll
      for (int h = 0; h < V; h++) {
        cur[r][h] = nxt[r][h];
        nxt[r][h] = pre[r][h];
      }
    vcur = vnxt;
    vnxt = vpre;
    if (k + 3 < nbat) {
      load(i0 + 3 * B, pre);
      load_vals(i0 + 3 * B, vpre);
    }
  }

  if (act) {
    double2* dst = p.colpart + (int64_t)bid * p.n + col;
#pragma unroll
    for (int k = 0; k < E; k++) dst[k] = make_double2(P[k], Q[k]);
  }
  if (flags) atomicOr(p.status, flags);  // rare: only lanes that saw a problem
}

template <int FMT, int G, int E, int B, int MAXT, bool PARTIAL>
__global__ __launch_bounds__(MAXT) void k_rowres(RowResArgs p) {
  rowres_block<FMT, G, E, B, PARTIAL>(p, blockIdx.x);
}

// ----------------------------------------------------------------------------- launch

// Columns per lane and rows per batch: rows of up to 4096 columns, in workgroups of at most
// 512 lanes (8 waves of up to 256 VGPRs), with E = 8 and batches of B = 4 rows (with three
// row buffers in flight, B = 8 spilled). Wider rows do
// not fit the registers without spills (a lane's fp64 column sums alone take 4 E of them; the
// E = 16 variant for NVFP4 rows of 8192 columns spilled and ran slower than the two-sweep
// passes), and stay on the two-sweep pass.
int rowres_cols_per_lane(int64_t) { return 8; }
int rowres_lanes(int64_t n) { return (int)((n + 8 * kWave - 1) / (8 * kWave)) * kWave; }
bool rowres_shape_ok(int fmt, int64_t n) {
  return (fmt == kInt4Bf16 || fmt == kNvFp4) && n >= 16 && n <= 4096;
}
int rowres_batch_rows(int64_t) { return 4; }

template <int FMT, int G, int E, int B>
static hipError_t rowres_launch(const RowResArgs& a, int nwg, hipStream_t s) {
  const dim3 grid((unsigned)nwg), block((unsigned)rowres_lanes(a.n));
  if (a.n % (E * kWave) != 0)
    hipLaunchKernelGGL((k_rowres<FMT, G, E, B, 512, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_rowres<FMT, G, E, B, 512, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int FMT, int G>
static hipError_t rowres_shape(const RowResArgs& a, int nwg, hipStream_t s) {
  return rowres_launch<FMT, G, 8, 4>(a, nwg, s);
}

template <int FMT>
static hipError_t rowres_group(const RowResArgs& a, int nwg, hipStream_t s) {
  switch (a.G) {
    case 16: return rowres_shape<FMT, 16>(a, nwg, s);
    case 32: return rowres_shape<FMT, 32>(a, nwg, s);
    case 64: return rowres_shape<FMT, 64>(a, nwg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rowres(int fmt, const RowResArgs& a, int nwg, hipStream_t s) {
  if (!rowres_shape_ok(fmt, a.n) || a.n % 16 != 0 || a.G < rowres_cols_per_lane(a.n) ||
      a.rpc % rowres_batch_rows(a.n) != 0 || nwg < 1)
    return hipErrorInvalidValue;
  switch (fmt) {
    case kInt4Bf16: return rowres_group<kInt4Bf16>(a, nwg, s);
    case kNvFp4: return rowres_group<kNvFp4>(a, nwg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dq
