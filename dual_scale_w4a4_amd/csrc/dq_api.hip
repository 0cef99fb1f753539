// dq_api.hip -- host side of libdq.so: argument checks, workspace layout, the launch sequence
// of one solve on the caller's stream, and status reporting.
//
// Launch sequence of dq_solve (daiwk notes, "核心公式" eq. 2 and the conventions under it;
// trove summary, "How it works" flowchart), all on `stream`, no host round trip inside:
//   setup   clear the device status, a <- Pi(a0) or 1, b <- Pi(b0) or 1, ra, rb (synced
//           inner copies), E_i = sum_j W_ij^2 and the finite check, NVFP4 tensor scale g
//   t = 0 .. T-1
//     MX formats (single sweep): one pass gives the codes of X(a, b), the row sums and the
//           column sums; with power-of-two scales the re-quantization after the row update
//           reproduces the same codes and a_i * d_ig (checked per group, see below), so one
//           finalize applies both closed-form updates.
//     otherwise (two sweeps): row pass -> finalize a; column pass on X(a', b) -> finalize b.
//   emit    Q(X(a_T, b_T)): packed codes, inner scales, and the sums for mse[T].
// If the MX single-sweep check fails anywhere, the solve is re-run on the two-sweep path,
// which always re-quantizes; both give the same result whenever the check passes.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/dq.h"
#include "../../include/dq_bench.h"
#include "dq_internal.h"

namespace {

constexpr int kTileCols = 512;
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;  // MI355X's last-level (MALL) cache

// Launch shape of the iteration passes. The defaults were measured best on MI355X for the
// 8B shapes. Row-resident pass (INT4_BF16 / NVFP4 rows of up to 4096 columns): off, since the
// two-sweep passes ran a whole decoder layer faster (the row-resident pass issues more
// instructions per element); when on, 256 workgroups (one 8-wave workgroup per CU; 384 and
// 512 were slower on the 14336-row matrices). Single-sweep MX pass: one 512-column half per
// lane, two rows per load step and about two 4-wave workgroups per CU, so that two matrices solved at once on two streams
// share the GPU (a matrix alone runs its pass as fast with three); a matrix whose bf16 W
// exceeds the 256 MiB Infinity Cache reads W from HBM on every pass, where three workgroups
// per CU keep more loads in flight (4.94 against 4.48 TB/s on a 28672 x 8192 matrix; four per
// CU gave 4.90), so it takes about three. Two-sweep pass for bf16
// weights: 768 workgroups (a sweep of 768-3072 moved it by under 10%). General sweep for
// fp32 weights: 512. The product entry points always take these defaults; only the
// measurement entry point (dq_solve_timed) takes another shape, so the fixed summation order
// and the workspace size of a solve never depend on the environment.
struct LaunchShape {
  int halves = 1;
  int step_rows = 2;
  int ahead = 1;
  int target = 512;
  int target_big = 768;  // W larger than the Infinity Cache
  int pass_target = 768;
  int sweep_target = 512;
  bool row_resident = false;
  int rowres_target = 256;
};

// a caller's shape (fields <= 0 keep the default); false if a field is out of range
bool launch_shape(const dq_launch_shape* in, LaunchShape* out) {
  LaunchShape f;
  if (in) {
    if (in->fused_halves > 0) f.halves = in->fused_halves;
    if (in->fused_step_rows > 0) f.step_rows = in->fused_step_rows;
    if (in->fused_ahead > 0) f.ahead = in->fused_ahead;
    if (in->fused_target > 0) f.target = f.target_big = in->fused_target;
    if (in->pass_target > 0) f.pass_target = in->pass_target;
    if (in->sweep_target > 0) f.sweep_target = in->sweep_target;
    if (in->row_resident != 0) f.row_resident = in->row_resident > 0;
    if (in->rowres_target > 0) f.rowres_target = in->rowres_target;
  }
  if ((f.halves != 1 && f.halves != 2) || (f.step_rows != 2 && f.step_rows != 4) ||
      (f.ahead != 1 && f.ahead != 3) || (f.ahead == 3 && (f.halves != 1 || f.step_rows != 2)) ||
      f.target > 65536 || f.pass_target > 65536 || f.sweep_target > 65536 ||
      f.rowres_target > 65536)
    return false;
  *out = f;
  return true;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  int64_t m = 0, n = 0;
  int G = 0, fmt = 0;
  int nct = 0, nrc = 0;
  int64_t rpc = 0;
  int f_nct = 0, f_nrc = 0;  // single-sweep MX pass: 512 * halves columns, rows in multiples of 32
  int64_t f_rpc = 0;
  // its final (emit) pass, which writes no column partials, in smaller row chunks: about three
  // workgroups per CU, where its code and scale stores run faster than with two
  int f_nrc_emit = 0;
  int64_t f_rpc_emit = 0;
  LaunchShape f_shape;
  int g_nct = 0, g_nrc = 0;  // two-sweep pass for bf16 weights: 512 columns, rows in 32s
  int64_t g_rpc = 0;
  // row-resident pass (INT4_BF16 / NVFP4 rows it takes): workgroups, rows per workgroup
  bool rr_ok = false;
  int rr_nwg = 0;
  int64_t rr_rpc = 0;
  int nblk_rows = 0, nblk_cols = 0;
  size_t off_status = 0, off_ra = 0, off_rb = 0, off_a0 = 0, off_b0 = 0, off_E = 0, off_amax = 0,
         off_gs = 0, off_rowerr = 0;
  size_t off_rowpart = 0, off_colpart = 0, off_msepart = 0, off_ymax = 0, off_epart = 0, total = 0;
};

bool shape_ok(int64_t rows, int64_t cols, int group) {
  if (rows <= 0 || cols <= 0) return false;
  if (group != 16 && group != 32 && group != 64) return false;
  if (cols % group != 0) return false;
  if (rows > ((int64_t)1 << 40) / cols) return false;  // at most 2^40 elements
  return true;
}

bool fmt_ok(int fmt) { return fmt >= 0 && fmt <= 3; }

// the bf16 single-sweep kernel's shapes: row and column indices within 32 bits
bool fast_shape_ok(const Plan& p) { return p.m < INT32_MAX && p.n < INT32_MAX; }

Plan make_plan(int64_t m, int64_t n, int fmt, int G, const LaunchShape& shape = LaunchShape{}) {
  Plan p;
  p.m = m;
  p.n = n;
  p.G = G;
  p.fmt = fmt;
  const int target = shape.sweep_target;
  p.nct = (int)((n + kTileCols - 1) / kTileCols);
  int64_t want = (target + p.nct - 1) / p.nct;
  int64_t max_rc = (m + 3) / 4;  // at least one row per wave
  p.nrc = (int)(want < 1 ? 1 : (want > max_rc ? max_rc : want));
  p.rpc = (m + p.nrc - 1) / p.nrc;
  p.nrc = (int)((m + p.rpc - 1) / p.rpc);  // drop empty trailing chunks
  p.f_shape = shape;
  const int64_t f_cols = (int64_t)kTileCols * p.f_shape.halves;
  p.f_nct = (int)((n + f_cols - 1) / f_cols);
  const int f_target = m * n * 2 > kInfinityCacheBytes ? p.f_shape.target_big : p.f_shape.target;
  int64_t f_want = (f_target + p.f_nct - 1) / p.f_nct;
  if (f_want < 1) f_want = 1;
  p.f_rpc = (m + f_want - 1) / f_want;
  p.f_rpc = (p.f_rpc + 31) / 32 * 32;  // whole 32-row batches per workgroup
  p.f_nrc = (int)((m + p.f_rpc - 1) / p.f_rpc);
  int64_t e_want = (p.f_shape.target * 3 / 2 + p.f_nct - 1) / p.f_nct;
  if (e_want < 1) e_want = 1;
  p.f_rpc_emit = ((m + e_want - 1) / e_want + 31) / 32 * 32;
  p.f_nrc_emit = (int)((m + p.f_rpc_emit - 1) / p.f_rpc_emit);
  p.g_nct = (int)((n + dq::pass_tile_cols() - 1) / dq::pass_tile_cols());
  int64_t g_want = (shape.pass_target + p.g_nct - 1) / p.g_nct;
  if (g_want < 1) g_want = 1;
  p.g_rpc = (m + g_want - 1) / g_want;
  p.g_rpc = (p.g_rpc + 31) / 32 * 32;
  p.g_nrc = (int)((m + p.g_rpc - 1) / p.g_rpc);
  if (shape.row_resident && dq::rowres_shape_ok(fmt, n)) {
    const int64_t B = dq::rowres_batch_rows(n);
    p.rr_ok = true;
    p.rr_rpc = ((m + shape.rowres_target - 1) / shape.rowres_target + B - 1) / B * B;
    p.rr_nwg = (int)((m + p.rr_rpc - 1) / p.rr_rpc);
  }
  p.nblk_rows = (int)((m + 255) / 256);
  p.nblk_cols = (int)((n + dq::kFinColsPerBlock - 1) / dq::kFinColsPerBlock);  // finalize
  size_t o = 0;
  p.off_status = o; o = align_up(o + 64);
  p.off_ra = o; o = align_up(o + sizeof(float) * m);
  p.off_rb = o; o = align_up(o + sizeof(float) * n);
  p.off_a0 = o; o = align_up(o + sizeof(float) * m);
  p.off_b0 = o; o = align_up(o + sizeof(float) * n);
  p.off_E = o; o = align_up(o + sizeof(double) * m);
  p.off_amax = o; o = align_up(o + sizeof(float) * m);
  p.off_gs = o; o = align_up(o + 16);
  const size_t rc_parts = (size_t)(p.nct > p.f_nct ? p.nct : p.f_nct);
  size_t cc_parts = (size_t)(p.nrc > p.f_nrc ? p.nrc : p.f_nrc);
  if ((size_t)p.g_nrc > cc_parts) cc_parts = (size_t)p.g_nrc;
  if ((size_t)p.rr_nwg > cc_parts) cc_parts = (size_t)p.rr_nwg;
  p.off_rowpart = o; o = align_up(o + 2 * sizeof(double) * rc_parts * m);
  p.off_colpart = o; o = align_up(o + 2 * sizeof(double) * cc_parts * n);
  p.off_msepart = o; o = align_up(o + 2 * sizeof(double) * p.nblk_rows);
  if (p.rr_ok) {  // the row-resident pass's per-row errors
    p.off_rowerr = o;
    o = align_up(o + sizeof(double) * m);
  }
  if (fmt == DQ_FMT_NVFP4) {  // per-pass tensor scale: the row pass's row maxima of |y|
    p.off_ymax = o;
    o = align_up(o + sizeof(float) * (size_t)p.g_nct * m);
  }
  if (fmt != DQ_FMT_NVFP4) {  // the first pass's W^2 partials (single sweep or bf16 two-sweep)
    const bool mx = fmt == DQ_FMT_MXINT4 || fmt == DQ_FMT_MXFP4;
    const size_t parts = (size_t)(mx && p.f_nct > p.g_nct ? p.f_nct : p.g_nct);
    p.off_epart = o;
    o = align_up(o + sizeof(double) * parts * m);
  }
  p.total = o;
  return p;
}

// workspace status word [0]: device flags
template <class T>
T* at(char* base, size_t off) {
  return reinterpret_cast<T*>(base + off);
}

struct Timer {
  dq_timing* out;
  hipStream_t s;
  std::vector<hipEvent_t> ev;
  std::vector<int> kind;
  hipEvent_t pending = nullptr;
  void before(int k) {
    if (!out) return;
    hipEvent_t e0;
    (void)hipEventCreate(&e0);
    (void)hipEventRecord(e0, s);
    pending = e0;
    kind.push_back(k);
  }
  void after() {
    if (!out) return;
    hipEvent_t e1;
    (void)hipEventCreate(&e1);
    (void)hipEventRecord(e1, s);
    ev.push_back(pending);
    ev.push_back(e1);
  }
  void collect() {
    if (!out) return;
    for (size_t k = 0; k < kind.size(); k++) {
      float ms = 0.0f;
      (void)hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]);
      out->ms[kind[k]] += ms;
      out->launches[kind[k]] += 1;
    }
  }
  ~Timer() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

#define DQ_TRY(expr)                     \
  do {                                   \
    if ((expr) != hipSuccess) return DQ_ERR_HIP; \
  } while (0)

dq_status map_status(int flags) {
  if (flags & dq::kStInitArg) return DQ_ERR_ARG;
  if (flags & dq::kStNonFinite) return DQ_ERR_NONFINITE;
  if (flags & dq::kStRange) return DQ_ERR_RANGE;
  if (flags & dq::kStInternal) return DQ_ERR_INTERNAL;
  return DQ_OK;
}

}  // namespace

extern "C" {

const char* dq_status_str(dq_status s) {
  switch (s) {
    case DQ_OK: return "DQ_OK";
    case DQ_ERR_ARG: return "DQ_ERR_ARG: invalid argument";
    case DQ_ERR_UNSUPPORTED: return "DQ_ERR_UNSUPPORTED: unknown format or weight dtype";
    case DQ_ERR_NONFINITE: return "DQ_ERR_NONFINITE: W holds a NaN or an infinity";
    case DQ_ERR_RANGE: return "DQ_ERR_RANGE: a scaled weight value overflowed";
    case DQ_ERR_WORKSPACE: return "DQ_ERR_WORKSPACE: workspace too small";
    case DQ_ERR_HIP: return "DQ_ERR_HIP: HIP runtime error";
    case DQ_ERR_INTERNAL: return "DQ_ERR_INTERNAL: non-positive closed-form numerator";
    default: return "unknown dq_status";
  }
}

size_t dq_workspace_bytes(int64_t rows, int64_t cols, dq_format fmt, int group) {
  if (!fmt_ok(fmt) || !shape_ok(rows, cols, group)) return 0;
  return make_plan(rows, cols, fmt, group).total;
}

}  // extern "C"

namespace {

struct SolveIo {
  const void* W;
  bool bf16;
  const dq_init* init;
  uint8_t* codes;
  void* scales;
  float* tensor_scale;
  float* a;
  float* b;
  double* mse;
  int T;
};

// Enqueue one full solve. `fused` selects the MX single-sweep path. `again` re-runs a solve
// from the projected initial scales that the first attempt saved in the workspace (the
// caller's a0 / b0 may alias the outputs a / b, which the first attempt overwrote).
dq_status enqueue_solve(const Plan& p, char* ws, const SolveIo& io, bool fused, bool again,
                        Timer& tm, hipStream_t s) {
  using namespace dq;
  int* status = at<int>(ws, p.off_status);
  float* ra = at<float>(ws, p.off_ra);
  float* rb = at<float>(ws, p.off_rb);
  double* E = at<double>(ws, p.off_E);
  float* amax = at<float>(ws, p.off_amax);
  float* gs = at<float>(ws, p.off_gs);
  double2* rowpart = at<double2>(ws, p.off_rowpart);
  double2* colpart = at<double2>(ws, p.off_colpart);
  double* msepart = at<double>(ws, p.off_msepart);  // two sets of per-block error sums
  const bool nv = p.fmt == kNvFp4;

  tm.before(DQ_K_SETUP);
  DQ_TRY(launch_clear(status, 16, s));
  float* a0s = at<float>(ws, p.off_a0);
  float* b0s = at<float>(ws, p.off_b0);
  const float* a_src = again ? a0s : (io.init ? io.init->a0 : nullptr);
  const float* b_src = again ? b0s : (io.init ? io.init->b0 : nullptr);
  // the single-sweep kernel for bf16 weights (32-bit row and column indices; larger matrices
  // take the general single-sweep kernel)
  const bool fast = fused && io.bf16 && fast_shape_ok(p);
  const bool pass_g = nv && io.init && (io.init->flags & DQ_SOLVE_PER_PASS_G);
  // the row-resident pass (bf16 weights, a tensor scale fixed for the solve, shapes it takes)
  const bool rowres = !fused && io.bf16 && !pass_g && p.rr_ok;
  VecArgs va{a_src, io.a, ra, again ? nullptr : a0s, p.m, p.fmt, 1, fast ? 1 : 0, status};
  DQ_TRY(launch_vec(va, s));
  VecArgs vb{b_src, io.b, rb, again ? nullptr : b0s, p.n, p.fmt, 1, fast ? 1 : 0, status};
  DQ_TRY(launch_vec(vb, s));
  // E_i = sum_j W_ij^2 and the finite check: in their own sweep of W, or, with at least one
  // iteration, inside the first iteration's pass: the single-sweep pass, or the bf16 two-sweep
  // row pass where no tensor scale has to be known before it (not NVFP4) and the row-resident
  // pass is not taken
  const bool stat_in_pass = fast && io.T > 0;
  const bool stat_in_row_pass = !fused && io.bf16 && !nv && !rowres && io.T > 0;
  if (!stat_in_pass && !stat_in_row_pass) {
    RowStatArgs rs{io.W, p.m, p.n, ra, rb, E, nv ? amax : nullptr, status};
    DQ_TRY(launch_rowstat(io.bf16, rs, s));
  }
  if (nv) {
    ScaleArgs sa{amax, p.m, nullptr, io.init ? io.init->g0 : 0.0f, gs, io.tensor_scale, status};
    DQ_TRY(launch_tensor_scale(sa, s));
  }
  tm.after();

  // NVFP4 with a per-pass tensor scale: g from the scaled tile about to be quantized
  auto pass_scale = [&]() -> dq_status {
    tm.before(DQ_K_SETUP);
    RowStatArgs r2{io.W, p.m, p.n, ra, rb, E, amax, status};
    DQ_TRY(launch_rowstat(io.bf16, r2, s));
    ScaleArgs s2{amax, p.m, nullptr, 0.0f, gs, io.tensor_scale, status};
    DQ_TRY(launch_tensor_scale(s2, s));
    tm.after();
    return DQ_OK;
  };

  SweepArgs sw{};
  sw.W = io.W;
  sw.m = p.m;
  sw.n = p.n;
  sw.G = p.G;
  sw.ra = ra;
  sw.rb = rb;
  sw.a = io.a;
  sw.b = io.b;
  sw.gs = gs;
  sw.nct = p.nct;
  sw.nrc = p.nrc;
  sw.rpc = p.rpc;
  sw.rowpart = rowpart;
  sw.colpart = colpart;
  sw.codes = io.codes;
  sw.scales = io.scales;
  sw.status = status;

  SweepArgs sp = sw;  // the two-sweep pass for bf16 weights
  sp.ymax = p.off_ymax ? at<float>(ws, p.off_ymax) : nullptr;
  sp.nct = p.g_nct;
  sp.nrc = p.g_nrc;
  sp.rpc = p.g_rpc;

  FinArgs fa{};
  fa.m = p.m;
  fa.n = p.n;
  fa.fmt = p.fmt;
  fa.rowpart = rowpart;
  fa.E = E;
  fa.a = io.a;
  fa.ra = ra;
  fa.inv_mn = 1.0 / ((double)p.m * (double)p.n);
  fa.colpart = colpart;
  fa.b = io.b;
  fa.rb = rb;
  fa.status = status;
  fa.prev_count = p.nblk_rows;

  FusedArgs fu{};
  fu.W = static_cast<const uint16_t*>(io.W);
  fu.m = p.m;
  fu.n = p.n;
  fu.G = p.G;
  fu.rb = rb;
  fu.b = io.b;
  fu.nct = p.f_nct;
  fu.nrc = p.f_nrc;
  fu.rpc = p.f_rpc;
  fu.halves = p.f_shape.halves;
  fu.step_rows = p.f_shape.step_rows;
  fu.ahead = p.f_shape.ahead;
  fu.rowpart = rowpart;
  fu.colpart = colpart;
  fu.codes = io.codes;
  fu.scales = static_cast<uint8_t*>(io.scales);
  fu.a = io.a;
  fu.status = status;

  RowResArgs rr{};
  rr.W = static_cast<const uint16_t*>(io.W);
  rr.m = p.m;
  rr.n = p.n;
  rr.G = p.G;
  rr.a = io.a;
  rr.ra = ra;
  rr.rb = rb;
  rr.b = io.b;
  rr.gs = gs;
  rr.E = E;
  rr.rowerr = p.off_rowerr ? at<double>(ws, p.off_rowerr) : nullptr;
  rr.colpart = colpart;
  rr.rpc = p.rr_rpc;
  rr.status = status;

  // mse[t]: a finalize that takes row sums writes per-block error sums into one of two
  // buffers; the next finalize (or the final collect) adds them up into mse[t]
  int produced = 0, pend_idx = -1;
  auto finalize = [&](bool rows, bool cols, bool update) -> dq_status {
    fa.nblk_rows = rows ? p.nblk_rows : 0;
    fa.nblk_cols = cols ? p.nblk_cols : 0;
    fa.update_a = update ? 1 : 0;
    fa.prev_part = pend_idx >= 0 ? msepart + (size_t)(pend_idx % 2) * p.nblk_rows : nullptr;
    fa.prev_out = pend_idx >= 0 ? io.mse + pend_idx : nullptr;
    pend_idx = -1;
    fa.part_out = nullptr;
    if (rows) {
      fa.part_out = msepart + (size_t)(produced % 2) * p.nblk_rows;
      pend_idx = produced++;
    }
    tm.before(DQ_K_FINAL);
    DQ_TRY(launch_finalize(fa, s));
    tm.after();
    return DQ_OK;
  };
  dq_status st = DQ_OK;

  for (int t = 0; t < io.T; t++) {
    if (fast) {
      double* epart = stat_in_pass && t == 0 ? at<double>(ws, p.off_epart) : nullptr;
      fu.epart = epart;
      tm.before(DQ_K_FUSED);
      DQ_TRY(launch_fused(p.fmt, false, fu, s));
      tm.after();
      fu.epart = nullptr;
      fa.nct = p.f_nct;
      fa.nrc = p.f_nrc;
      fa.gauge_check = 0;
      fa.row_ra = 1;
      fa.envelope = 1;
      fa.col_terms = 8 + (int)((p.f_rpc + 31) / 32);  // 8 rows per batch, then the batches
      fa.epart = epart;
      if ((st = finalize(true, true, true)) != DQ_OK) return st;
      fa.epart = nullptr;
    } else if (fused) {
      tm.before(DQ_K_FUSED);
      DQ_TRY(launch_sweep(p.fmt, io.bf16, kModeRow | kModeCol | kModeGauge, sw, s));
      tm.after();
      fa.nct = p.nct;
      fa.nrc = p.nrc;
      fa.gauge_check = 1;
      if ((st = finalize(true, true, true)) != DQ_OK) return st;
    } else if (io.bf16 && rowres) {
      // one read of W: both Q evaluations, the row update and the column partials
      tm.before(DQ_K_ROWRES);
      DQ_TRY(launch_rowres(p.fmt, rr, p.rr_nwg, s));
      tm.after();
      fa.nct = 0;
      fa.nrc = p.rr_nwg;
      fa.rowerr = rr.rowerr;
      if ((st = finalize(true, true, false)) != DQ_OK) return st;
      fa.rowerr = nullptr;
    } else if (io.bf16) {
      if (pass_g && t > 0 && (st = pass_scale()) != DQ_OK) return st;
      tm.before(DQ_K_ROW);
      // per-pass tensor scale: the row pass also records each row's max |fl32(W rb)|, from
      // which the finalize forms the column pass's row maxima of |X| without a read of W; the
      // first row pass of a solve may also sum W^2 (E_i, and the finite check)
      const bool stat = stat_in_row_pass && t == 0;
      sp.epart = stat ? at<double>(ws, p.off_epart) : nullptr;
      DQ_TRY(launch_pass(p.fmt, pass_g ? (kModeRow | kModeYmax) : (stat ? kModeRow | kModeStat : kModeRow),
                         sp, s));
      tm.after();
      fa.nct = p.g_nct;
      fa.nrc = p.g_nrc;
      fa.ymax = pass_g ? sp.ymax : nullptr;
      fa.amax_out = pass_g ? amax : nullptr;
      fa.epart = sp.epart;
      if ((st = finalize(true, false, true)) != DQ_OK) return st;
      fa.ymax = nullptr;
      fa.amax_out = nullptr;
      fa.epart = nullptr;
      sp.epart = nullptr;
      if (pass_g) {
        tm.before(DQ_K_SETUP);
        ScaleArgs s2{amax, p.m, nullptr, 0.0f, gs, io.tensor_scale, status};
        DQ_TRY(launch_tensor_scale(s2, s));
        tm.after();
      }
      tm.before(DQ_K_COL);
      DQ_TRY(launch_pass(p.fmt, kModeCol, sp, s));
      tm.after();
      if ((st = finalize(false, true, false)) != DQ_OK) return st;
    } else {
      if (pass_g && t > 0 && (st = pass_scale()) != DQ_OK) return st;
      tm.before(DQ_K_ROW);
      DQ_TRY(launch_sweep(p.fmt, io.bf16, kModeRow, sw, s));
      tm.after();
      fa.nct = p.nct;
      fa.nrc = p.nrc;
      if ((st = finalize(true, false, true)) != DQ_OK) return st;
      if (pass_g && (st = pass_scale()) != DQ_OK) return st;
      tm.before(DQ_K_COL);
      DQ_TRY(launch_sweep(p.fmt, io.bf16, kModeCol, sw, s));
      tm.after();
      if ((st = finalize(false, true, false)) != DQ_OK) return st;
    }
  }
  if (pass_g && io.T > 0 && (st = pass_scale()) != DQ_OK) return st;
  tm.before(DQ_K_EMIT);
  if (fast) {
    FusedArgs fe = fu;  // the emit pass's own row chunks (its row errors are per column tile)
    fe.nrc = p.f_nrc_emit;
    fe.rpc = p.f_rpc_emit;
    DQ_TRY(launch_fused(p.fmt, true, fe, s));
    fa.nct = p.f_nct;
    fa.row_ra = 1;
  } else if (io.bf16) {
    DQ_TRY(launch_pass(p.fmt, kModeEmit | kModeRow, sp, s));
    fa.nct = p.g_nct;
    fa.row_ra = 0;
  } else {
    DQ_TRY(launch_sweep(p.fmt, io.bf16, kModeEmit | kModeRow, sw, s));
    fa.nct = p.nct;
    fa.row_ra = 0;
  }
  tm.after();
  fa.envelope = 0;
  fa.gauge_check = 0;
  if ((st = finalize(true, false, false)) != DQ_OK) return st;
  tm.before(DQ_K_FINAL);
  DQ_TRY(launch_mse_collect(msepart + (size_t)(pend_idx % 2) * p.nblk_rows, p.nblk_rows,
                            io.mse + pend_idx, fa.inv_mn, s));
  tm.after();
  return DQ_OK;
}

// ------------------------------------------------------------------------- batch solves
// One matrix of a batch solve on the two-sweep path for bf16 weights: the same state, kernels
// and order of operations as enqueue_solve's two-sweep branch, stepped phase by phase so that
// the per-iteration passes and finalizes of all matrices share launches.
struct BatchMat {
  Plan p;
  char* ws = nullptr;
  SolveIo io{};
  bool pass_g = false;
  bool stat_first = false;  // E_i and the finite check from the first row pass (as enqueue_solve)
  int* status = nullptr;
  float *ra = nullptr, *rb = nullptr, *amax = nullptr, *gs = nullptr;
  double* E = nullptr;
  double* epart = nullptr;
  double* msepart = nullptr;
  dq::SweepArgs sp{};
  dq::FinArgs fa{};
  int produced = 0, pend_idx = -1;

  dq_status setup(const dq_init* init, hipStream_t s) {
    using namespace dq;
    status = at<int>(ws, p.off_status);
    ra = at<float>(ws, p.off_ra);
    rb = at<float>(ws, p.off_rb);
    E = at<double>(ws, p.off_E);
    amax = at<float>(ws, p.off_amax);
    gs = at<float>(ws, p.off_gs);
    msepart = at<double>(ws, p.off_msepart);
    const bool nv = p.fmt == kNvFp4;
    DQ_TRY(launch_clear(status, 16, s));
    VecArgs va{init->a0, io.a, ra, nullptr, p.m, p.fmt, 1, 0, status};
    DQ_TRY(launch_vec(va, s));
    VecArgs vb{init->b0, io.b, rb, nullptr, p.n, p.fmt, 1, 0, status};
    DQ_TRY(launch_vec(vb, s));
    stat_first = !nv && io.T > 0;
    epart = stat_first ? at<double>(ws, p.off_epart) : nullptr;
    if (!stat_first) {
      RowStatArgs rs{io.W, p.m, p.n, ra, rb, E, nv ? amax : nullptr, status};
      DQ_TRY(launch_rowstat(true, rs, s));
    }
    if (nv) {
      ScaleArgs sa{amax, p.m, nullptr, init->g0, gs, io.tensor_scale, status};
      DQ_TRY(launch_tensor_scale(sa, s));
    }
    sp = SweepArgs{};
    sp.W = io.W;
    sp.m = p.m;
    sp.n = p.n;
    sp.G = p.G;
    sp.ra = ra;
    sp.rb = rb;
    sp.a = io.a;
    sp.b = io.b;
    sp.gs = gs;
    sp.nct = p.g_nct;
    sp.nrc = p.g_nrc;
    sp.rpc = p.g_rpc;
    sp.rowpart = at<double2>(ws, p.off_rowpart);
    sp.colpart = at<double2>(ws, p.off_colpart);
    sp.codes = io.codes;
    sp.scales = io.scales;
    sp.status = status;
    sp.ymax = p.off_ymax ? at<float>(ws, p.off_ymax) : nullptr;
    fa = FinArgs{};
    fa.m = p.m;
    fa.n = p.n;
    fa.fmt = p.fmt;
    fa.rowpart = sp.rowpart;
    fa.E = E;
    fa.a = io.a;
    fa.ra = ra;
    fa.inv_mn = 1.0 / ((double)p.m * (double)p.n);
    fa.colpart = sp.colpart;
    fa.b = io.b;
    fa.rb = rb;
    fa.status = status;
    fa.prev_count = p.nblk_rows;
    fa.nct = p.g_nct;
    fa.nrc = p.g_nrc;
    return DQ_OK;
  }

  // per-pass tensor scale of the tile about to be quantized (a read of W)
  dq_status pass_scale(hipStream_t s) {
    using namespace dq;
    RowStatArgs r2{io.W, p.m, p.n, ra, rb, E, amax, status};
    DQ_TRY(launch_rowstat(true, r2, s));
    ScaleArgs s2{amax, p.m, nullptr, 0.0f, gs, io.tensor_scale, status};
    DQ_TRY(launch_tensor_scale(s2, s));
    return DQ_OK;
  }

  // the arguments of one finalize launch, with the double-buffered mse bookkeeping
  dq::FinArgs fin(bool rows, bool cols, bool update) {
    fa.nblk_rows = rows ? p.nblk_rows : 0;
    fa.nblk_cols = cols ? p.nblk_cols : 0;
    fa.update_a = update ? 1 : 0;
    fa.prev_part = pend_idx >= 0 ? msepart + (size_t)(pend_idx % 2) * p.nblk_rows : nullptr;
    fa.prev_out = pend_idx >= 0 ? io.mse + pend_idx : nullptr;
    pend_idx = -1;
    fa.part_out = nullptr;
    if (rows) {
      fa.part_out = msepart + (size_t)(produced % 2) * p.nblk_rows;
      pend_idx = produced++;
    }
    return fa;
  }

  dq_status emit(hipStream_t s) {
    using namespace dq;
    if (pass_g && io.T > 0) {
      const dq_status st = pass_scale(s);
      if (st != DQ_OK) return st;
    }
    DQ_TRY(launch_pass(p.fmt, kModeEmit | kModeRow, sp, s));
    fa.ymax = nullptr;
    fa.amax_out = nullptr;
    DQ_TRY(launch_finalize(fin(true, false, false), s));
    DQ_TRY(launch_mse_collect(msepart + (size_t)(pend_idx % 2) * p.nblk_rows, p.nblk_rows,
                              io.mse + pend_idx, fa.inv_mn, s));
    return DQ_OK;
  }
};

// One iteration of every matrix of a batch: grouped row passes, row finalizes, column passes
// and column finalizes, up to kMaxMulti matrices per launch.
dq_status batch_iteration(BatchMat* mats, int n, int t, hipStream_t s) {
  using namespace dq;
  const int fmt = mats[0].p.fmt;
  const bool pass_g = mats[0].pass_g;
  for (int k0 = 0; k0 < n; k0 += kMaxMulti) {
    const int cnt = n - k0 < kMaxMulti ? n - k0 : kMaxMulti;
    BatchMat* b = mats + k0;
    if (pass_g && t > 0)
      for (int k = 0; k < cnt; k++) {
        const dq_status st = b[k].pass_scale(s);
        if (st != DQ_OK) return st;
      }
    // the first row pass also sums W^2 per row where no tensor scale comes first (every
    // matrix of a batch has the same format)
    const bool stat = t == 0 && b[0].stat_first;
    PassMulti pm{};
    pm.n = cnt;
    for (int k = 0; k < cnt; k++) {
      pm.a[k] = b[k].sp;
      pm.a[k].epart = stat ? b[k].epart : nullptr;
      pm.start[k + 1] = pm.start[k] + b[k].p.g_nct * b[k].p.g_nrc;
    }
    DQ_TRY(launch_pass_multi(fmt, pass_g ? (kModeRow | kModeYmax) : (stat ? kModeRow | kModeStat : kModeRow),
                             pm, s));
    FinMulti fm{};
    fm.n = cnt;
    for (int k = 0; k < cnt; k++) {
      b[k].fa.ymax = pass_g ? b[k].sp.ymax : nullptr;
      b[k].fa.amax_out = pass_g ? b[k].amax : nullptr;
      b[k].fa.epart = stat ? b[k].epart : nullptr;
      fm.a[k] = b[k].fin(true, false, true);
      fm.start[k + 1] = fm.start[k] + b[k].p.nblk_rows;
      b[k].fa.ymax = nullptr;
      b[k].fa.amax_out = nullptr;
      b[k].fa.epart = nullptr;
    }
    DQ_TRY(launch_finalize_multi(fm, s));
    if (pass_g)
      for (int k = 0; k < cnt; k++) {
        ScaleArgs s2{b[k].amax, b[k].p.m, nullptr, 0.0f, b[k].gs, b[k].io.tensor_scale, b[k].status};
        DQ_TRY(launch_tensor_scale(s2, s));
      }
    for (int k = 0; k < cnt; k++) pm.a[k] = b[k].sp;
    DQ_TRY(launch_pass_multi(fmt, kModeCol, pm, s));
    for (int k = 0; k < cnt; k++) {
      fm.a[k] = b[k].fin(false, true, false);
      fm.start[k + 1] = fm.start[k] + b[k].p.nblk_cols;
    }
    DQ_TRY(launch_finalize_multi(fm, s));
  }
  return DQ_OK;
}

// Re-run the single-sweep pass back to back between one pair of events (after the solve, on
// its final b; only the workspace's partial sums change) to time the kernel without the
// per-launch event overhead.
dq_status time_isolated(const Plan& p, char* ws, const void* W, float* a, const float* b,
                        dq_timing* out, hipStream_t s) {
  using namespace dq;
  constexpr int kReps = 8;
  FusedArgs fu{};
  fu.W = static_cast<const uint16_t*>(W);
  fu.m = p.m;
  fu.n = p.n;
  fu.G = p.G;
  fu.rb = at<float>(ws, p.off_rb);
  fu.b = b;
  fu.nct = p.f_nct;
  fu.nrc = p.f_nrc;
  fu.rpc = p.f_rpc;
  fu.halves = p.f_shape.halves;
  fu.step_rows = p.f_shape.step_rows;
  fu.ahead = p.f_shape.ahead;
  fu.rowpart = at<double2>(ws, p.off_rowpart);
  fu.colpart = at<double2>(ws, p.off_colpart);
  fu.a = a;
  fu.status = at<int>(ws, p.off_status) + 1;  // a scratch word: flags are not reread
  hipEvent_t e0, e1;
  DQ_TRY(hipEventCreate(&e0));
  DQ_TRY(hipEventCreate(&e1));
  DQ_TRY(launch_fused(p.fmt, false, fu, s));  // warm
  DQ_TRY(hipEventRecord(e0, s));
  for (int r = 0; r < kReps; r++) DQ_TRY(launch_fused(p.fmt, false, fu, s));
  DQ_TRY(hipEventRecord(e1, s));
  DQ_TRY(hipEventSynchronize(e1));
  float ms = 0.0f;
  DQ_TRY(hipEventElapsedTime(&ms, e0, e1));
  out->isolated_ms = ms;
  out->isolated_launches = kReps;
  if (out->flush && out->flush_bytes >= 16) {
    // one launch at a time, after a full read of the flush buffer (cold) and without (warm)
    double cold = 0.0, warm = 0.0;
    for (int pass = 0; pass < 2; pass++)
      for (int r = 0; r < kReps; r++) {
        if (pass == 0) DQ_TRY(launch_flush(out->flush, out->flush_bytes / 16, fu.status + 1, s));
        DQ_TRY(hipEventRecord(e0, s));
        DQ_TRY(launch_fused(p.fmt, false, fu, s));
        DQ_TRY(hipEventRecord(e1, s));
        DQ_TRY(hipEventSynchronize(e1));
        DQ_TRY(hipEventElapsedTime(&ms, e0, e1));
        (pass == 0 ? cold : warm) += ms;
      }
    out->cold_ms = cold;
    out->warm_ms = warm;
    out->per_launch = kReps;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return DQ_OK;
}

// Launch shape and workspace of the activation quantizer: 1024-channel tiles, chunks of
// tokens in multiples of 16 (four waves of four rows), about 1024 workgroups.
struct ActPlan {
  int nct = 0, nrc = 0;
  int64_t rpc = 0;
  size_t off_status = 0, off_part = 0, off_gs = 0, total = 0;
};

ActPlan act_plan(int64_t m, int64_t n) {
  ActPlan p;
  p.nct = (int)((n + dq::act_tile_cols() - 1) / dq::act_tile_cols());
  int64_t want = (1024 + p.nct - 1) / p.nct;
  if (want < 1) want = 1;
  p.rpc = (m + want - 1) / want;
  p.rpc = (p.rpc + 15) / 16 * 16;
  p.nrc = (int)((m + p.rpc - 1) / p.rpc);
  size_t o = 0;
  p.off_status = o; o = align_up(o + 64);
  p.off_part = o; o = align_up(o + sizeof(float) * (size_t)dq::act_amax_blocks());
  p.off_gs = o; o = align_up(o + 16);
  p.total = o;
  return p;
}

dq_status read_flags(char* ws, const Plan& p, hipStream_t s, int* flags) {
  int host[2] = {0, 0};
  DQ_TRY(hipMemcpyAsync(host, ws + p.off_status, sizeof host, hipMemcpyDeviceToHost, s));
  DQ_TRY(hipStreamSynchronize(s));
  *flags = host[0];
  return DQ_OK;
}

dq_status check_common(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                       int group, const uint8_t* codes, const void* scales) {
  if (!fmt_ok(fmt) || (wt != DQ_F32 && wt != DQ_BF16)) return DQ_ERR_UNSUPPORTED;
  if (!W || !codes || !scales) return DQ_ERR_ARG;
  if (!shape_ok(rows, cols, group)) return DQ_ERR_ARG;
  if (((uintptr_t)W & 15u) != 0 || ((uintptr_t)codes & 3u) != 0) return DQ_ERR_ARG;
  if (fmt == DQ_FMT_INT4_BF16 && ((uintptr_t)scales & 1u) != 0) return DQ_ERR_ARG;
  return DQ_OK;
}

// Owns the workspace for one call: the caller's, or a stream-ordered allocation.
struct WsGuard {
  char* ptr = nullptr;
  bool owned = false;
  hipStream_t s = nullptr;
  ~WsGuard() {
    if (owned && ptr) (void)hipFreeAsync(ptr, s);
  }
};

// OR a finished solve's status word into a caller's (one lane; integer atomic, so calls on
// several streams may share the caller's word)
__global__ void k_status_or(const int* src, int* dst) {
  if (threadIdx.x == 0 && src[0] != 0) atomicOr(dst, src[0]);
}

dq_status get_workspace(const Plan& p, void* workspace, size_t bytes, hipStream_t s, WsGuard& g) {
  g.s = s;
  if (workspace) {
    if (bytes < p.total) return DQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return DQ_ERR_ARG;
    g.ptr = static_cast<char*>(workspace);
    return DQ_OK;
  }
  void* ptr = nullptr;
  DQ_TRY(hipMallocAsync(&ptr, p.total, s));
  g.ptr = static_cast<char*>(ptr);
  g.owned = true;
  return DQ_OK;
}

// The workspace of dq_solve_async_noalloc, for callers that cannot allocate: one per device
// (each GPU the library runs on holds its own copy until the process ends). Host code never
// passes the array's name to a kernel: it is a host-side stand-in, and the device address is
// looked up per device with hipGetSymbolAddress.
static __device__ __align__(256) char scratch[DQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];  // the device address of `scratch` on each device, or null

// The address of `scratch` on the current device, which `stream` must belong to; looked up on
// the first call on each device (with that device current), then kept.
dq_status scratch_address(hipStream_t stream, char** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur < 0 || cur >= kMaxDevices) return DQ_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return DQ_ERR_HIP;
    if (sdev != cur) return DQ_ERR_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DQ_ERR_HIP;
    g_scratch_ptr[cur] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[cur];
  return DQ_OK;
}

// a, b: the outputs the passes read back (b in 128-bit loads)
bool scale_outputs_ok(const float* a, const float* b) {
  return a && b && ((uintptr_t)a & 3u) == 0 && ((uintptr_t)b & 15u) == 0;
}

dq_status check_solve(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                      int group, int T, const dq_init* init, const uint8_t* codes,
                      const void* inner_scales, const float* tensor_scale, const float* a,
                      const float* b, const double* mse) {
  dq_status st = check_common(W, wt, rows, cols, fmt, group, codes, inner_scales);
  if (st != DQ_OK) return st;
  if (T < 0 || !scale_outputs_ok(a, b) || !mse || (fmt == DQ_FMT_NVFP4 && !tensor_scale))
    return DQ_ERR_ARG;
  if (init && (init->g0 != init->g0 || (init->g0 > 0.0f && init->g0 > 3.4028234663852886e38f)))
    return DQ_ERR_ARG;
  if (init && fmt == DQ_FMT_NVFP4 && (init->flags & DQ_SOLVE_PER_PASS_G) && init->g0 > 0.0f)
    return DQ_ERR_ARG;
  return DQ_OK;
}

// The blocking solve of dq_solve / dq_solve_timed: enqueue, wait, read the device status,
// and redo the solve on the two-sweep path if the MX single-sweep identity was not
// guaranteed somewhere.
dq_status solve_blocking(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                         int group, int T, const dq_init* init, uint8_t* codes,
                         void* inner_scales, float* tensor_scale, float* a, float* b,
                         double* mse, void* workspace, size_t workspace_bytes,
                         const LaunchShape& shape, dq_timing* timing, hipStream_t stream) {
  dq_status st = check_solve(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                             tensor_scale, a, b, mse);
  if (st != DQ_OK) return st;
  const Plan p = make_plan(rows, cols, fmt, group, shape);
  WsGuard ws;
  st = get_workspace(p, workspace, workspace_bytes, stream, ws);
  if (st != DQ_OK) return st;

  SolveIo io{W, wt == DQ_BF16, init, codes, inner_scales, tensor_scale, a, b, mse, T};
  const bool mx = fmt == DQ_FMT_MXINT4 || fmt == DQ_FMT_MXFP4;
  bool fused = mx && !(init && (init->flags & DQ_SOLVE_TWO_SWEEP));

  int flags = 0;
  const void* flush = timing ? timing->flush : nullptr;
  const size_t flush_bytes = timing ? timing->flush_bytes : 0;
  for (int attempt = 0; attempt < 2; attempt++) {
    if (timing) {
      memset(timing, 0, sizeof *timing);
      timing->flush = flush;
      timing->flush_bytes = flush_bytes;
    }
    Timer tm{timing, stream};
    st = enqueue_solve(p, ws.ptr, io, fused, attempt > 0, tm, stream);
    if (st != DQ_OK) return st;
    st = read_flags(ws.ptr, p, stream, &flags);
    if (st != DQ_OK) return st;
    tm.collect();
    if (timing) timing->used_fused = fused ? 1 : 0;
    if (timing && fused && wt == DQ_BF16 && fast_shape_ok(p) && T > 0 && flags == 0) {
      st = time_isolated(p, ws.ptr, W, a, b, timing, stream);
      if (st != DQ_OK) return st;
    }
    if (fused && (flags & dq::kStGauge) && !(flags & ~dq::kStGauge)) {
      fused = false;  // the single-sweep identity was not guaranteed: redo on the general path
      continue;
    }
    break;
  }
  return map_status(flags & ~dq::kStGauge);
}

}  // namespace

extern "C" {

dq_status dq_solve(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                   int group, int T, const dq_init* init, uint8_t* codes, void* inner_scales,
                   float* tensor_scale, float* a, float* b, double* mse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return solve_blocking(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                        tensor_scale, a, b, mse, workspace, workspace_bytes, LaunchShape{},
                        nullptr, stream);
}

size_t dq_bench_workspace_bytes(int64_t rows, int64_t cols, dq_format fmt, int group,
                                const dq_launch_shape* shape) {
  LaunchShape sh;
  if (!fmt_ok(fmt) || !shape_ok(rows, cols, group) || !launch_shape(shape, &sh)) return 0;
  return make_plan(rows, cols, fmt, group, sh).total;
}

dq_status dq_solve_timed(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                         int group, int T, const dq_init* init, uint8_t* codes,
                         void* inner_scales, float* tensor_scale, float* a, float* b,
                         double* mse, void* workspace, size_t workspace_bytes,
                         const dq_launch_shape* shape, dq_timing* timing, hipStream_t stream) {
  LaunchShape sh;
  if (!launch_shape(shape, &sh)) return DQ_ERR_ARG;
  return solve_blocking(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                        tensor_scale, a, b, mse, workspace, workspace_bytes, sh, timing, stream);
}

dq_status dq_solve_async(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                         int group, int T, const dq_init* init, uint8_t* codes,
                         void* inner_scales, float* tensor_scale, float* a, float* b,
                         double* mse, int* status, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  dq_status st = check_solve(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                             tensor_scale, a, b, mse);
  if (st != DQ_OK) return st;
  if (!status || ((uintptr_t)status & 3u) != 0) return DQ_ERR_ARG;
  const Plan p = make_plan(rows, cols, fmt, group);
  WsGuard ws;  // an owned workspace is freed stream-ordered, after the solve's kernels
  st = get_workspace(p, workspace, workspace_bytes, stream, ws);
  if (st != DQ_OK) return st;
  SolveIo io{W, wt == DQ_BF16, init, codes, inner_scales, tensor_scale, a, b, mse, T};
  const bool mx = fmt == DQ_FMT_MXINT4 || fmt == DQ_FMT_MXFP4;
  const bool fused = mx && !(init && (init->flags & DQ_SOLVE_TWO_SWEEP));
  Timer tm{nullptr, stream};
  st = enqueue_solve(p, ws.ptr, io, fused, false, tm, stream);
  if (st != DQ_OK) return st;
  hipLaunchKernelGGL(k_status_or, dim3(1), dim3(64), 0, stream, at<int>(ws.ptr, p.off_status),
                     status);
  DQ_TRY(hipGetLastError());
  return DQ_OK;
}

dq_status dq_solve_async_noalloc(const void* W, dq_dtype wt, int64_t rows, int64_t cols,
                                 dq_format fmt, int group, int T, const dq_init* init,
                                 uint8_t* codes, void* inner_scales, float* tensor_scale,
                                 float* a, float* b, double* mse, int* status,
                                 hipStream_t stream) {
  dq_status st = check_solve(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                             tensor_scale, a, b, mse);
  if (st != DQ_OK) return st;
  if (!status || ((uintptr_t)status & 3u) != 0) return DQ_ERR_ARG;
  if (dq_workspace_bytes(rows, cols, fmt, group) > (size_t)DQ_NOALLOC_SCRATCH_BYTES)
    return DQ_ERR_WORKSPACE;
  char* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != DQ_OK) return st;
  // the same enqueue as dq_solve_async with a caller workspace: no allocation on any path
  return dq_solve_async(W, wt, rows, cols, fmt, group, T, init, codes, inner_scales,
                        tensor_scale, a, b, mse, status, ws, (size_t)DQ_NOALLOC_SCRATCH_BYTES,
                        stream);
}

dq_status dq_quantize(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                      int group, const float* a, const float* b, float* tensor_scale_inout,
                      uint8_t* codes, void* inner_scales, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  using namespace dq;
  dq_status st = check_common(W, wt, rows, cols, fmt, group, codes, inner_scales);
  if (st != DQ_OK) return st;
  if (fmt == DQ_FMT_NVFP4 && !tensor_scale_inout) return DQ_ERR_ARG;
  const Plan p = make_plan(rows, cols, fmt, group);
  WsGuard ws;
  st = get_workspace(p, workspace, workspace_bytes, stream, ws);
  if (st != DQ_OK) return st;
  char* base = ws.ptr;
  int* status = at<int>(base, p.off_status);
  float* ra = at<float>(base, p.off_ra);
  float* rb = at<float>(base, p.off_rb);
  float* amax = at<float>(base, p.off_amax);
  float* gs = at<float>(base, p.off_gs);
  // a, b are used as given: copy them into the synced slots (no projection)
  float* acopy = at<float>(base, p.off_rowpart);  // rowpart holds >= 4 m floats
  float* bcopy = at<float>(base, p.off_colpart);  // colpart holds >= 4 n floats
  const bool nv = fmt == DQ_FMT_NVFP4;

  DQ_TRY(launch_clear(status, 16, stream));
  VecArgs va{a, acopy, ra, nullptr, rows, fmt, 0, 0, status};
  DQ_TRY(launch_vec(va, stream));
  VecArgs vb{b, bcopy, rb, nullptr, cols, fmt, 0, 0, status};
  DQ_TRY(launch_vec(vb, stream));
  RowStatArgs rs{W, rows, cols, ra, rb, at<double>(base, p.off_E), nv ? amax : nullptr, status};
  DQ_TRY(launch_rowstat(wt == DQ_BF16, rs, stream));
  if (nv) {
    ScaleArgs sa{amax, rows, tensor_scale_inout, 0.0f, gs, tensor_scale_inout, status};
    DQ_TRY(launch_tensor_scale(sa, stream));
  }
  SweepArgs sw{};
  sw.W = W;
  sw.m = rows;
  sw.n = cols;
  sw.G = group;
  sw.ra = ra;
  sw.rb = rb;
  sw.a = acopy;
  sw.b = bcopy;
  sw.gs = gs;
  sw.nct = p.nct;
  sw.nrc = p.nrc;
  sw.rpc = p.rpc;
  sw.codes = codes;
  sw.scales = inner_scales;
  sw.status = status;
  DQ_TRY(launch_sweep(fmt, wt == DQ_BF16, kModeEmit, sw, stream));
  int flags = 0;
  st = read_flags(base, p, stream, &flags);
  if (st != DQ_OK) return st;
  return map_status(flags);
}

size_t dq_act_workspace_bytes(int64_t tokens, int64_t cols, dq_format fmt, int group) {
  if (!fmt_ok(fmt) || !shape_ok(tokens, cols, group)) return 0;
  return act_plan(tokens, cols).total;
}

dq_status dq_quantize_act_async(const void* X, dq_dtype xt, int64_t tokens, int64_t cols,
                                dq_format fmt, int group, const float* b, float g,
                                float* tensor_scale, uint8_t* codes, void* inner_scales,
                                int* status, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  using namespace dq;
  dq_status st = check_common(X, xt, tokens, cols, fmt, group, codes, inner_scales);
  if (st != DQ_OK) return st;
  if (!status || ((uintptr_t)status & 3u) != 0) return DQ_ERR_ARG;
  if (((uintptr_t)codes & 7u) != 0 || ((uintptr_t)b & 15u) != 0) return DQ_ERR_ARG;
  if (g != g || g > 3.4028234663852886e38f) return DQ_ERR_ARG;
  const ActPlan p = act_plan(tokens, cols);
  const bool amax = fmt == DQ_FMT_NVFP4 && !(g > 0.0f);
  WsGuard ws;
  if (amax) {  // only the amax pass uses the workspace
    if (workspace) {
      if (workspace_bytes < p.total) return DQ_ERR_WORKSPACE;
      if (((uintptr_t)workspace & 255u) != 0) return DQ_ERR_ARG;
      ws.ptr = static_cast<char*>(workspace);
      ws.s = stream;
    } else {
      void* ptr = nullptr;
      DQ_TRY(hipMallocAsync(&ptr, p.total, stream));
      ws.ptr = static_cast<char*>(ptr);
      ws.owned = true;
      ws.s = stream;
    }
  }
  ActArgs aa{};
  aa.X = X;
  aa.m = tokens;
  aa.n = cols;
  aa.G = group;
  aa.b = b;
  aa.g = g;
  aa.gs = nullptr;
  aa.gs_out = amax ? at<float>(ws.ptr, p.off_gs) : nullptr;
  aa.g_out = fmt == DQ_FMT_NVFP4 ? tensor_scale : nullptr;
  aa.part = amax ? at<float>(ws.ptr, p.off_part) : nullptr;
  aa.nct = p.nct;
  aa.nrc = p.nrc;
  aa.rpc = p.rpc;
  aa.codes = codes;
  aa.scales = inner_scales;
  aa.status = status;
  if (amax) {
    DQ_TRY(launch_act_gscale(xt == DQ_BF16, aa, stream));
    aa.gs = aa.gs_out;
  }
  DQ_TRY(launch_act(fmt, xt == DQ_BF16, aa, stream));
  return DQ_OK;
}

dq_status dq_quantize_act(const void* X, dq_dtype xt, int64_t tokens, int64_t cols,
                          dq_format fmt, int group, const float* b, float g, float* tensor_scale,
                          uint8_t* codes, void* inner_scales, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  using namespace dq;
  dq_status st = check_common(X, xt, tokens, cols, fmt, group, codes, inner_scales);
  if (st != DQ_OK) return st;
  if (((uintptr_t)codes & 7u) != 0 || ((uintptr_t)b & 15u) != 0) return DQ_ERR_ARG;
  if (g != g || g > 3.4028234663852886e38f) return DQ_ERR_ARG;
  const ActPlan p = act_plan(tokens, cols);
  WsGuard ws;
  if (workspace) {
    if (workspace_bytes < p.total) return DQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return DQ_ERR_ARG;
    ws.ptr = static_cast<char*>(workspace);
    ws.s = stream;
  } else {
    void* ptr = nullptr;
    DQ_TRY(hipMallocAsync(&ptr, p.total, stream));
    ws.ptr = static_cast<char*>(ptr);
    ws.owned = true;
    ws.s = stream;
  }
  int* status = at<int>(ws.ptr, p.off_status);
  DQ_TRY(launch_clear(status, 16, stream));
  st = dq_quantize_act_async(X, xt, tokens, cols, fmt, group, b, g, tensor_scale, codes,
                             inner_scales, status, ws.ptr, p.total, stream);
  if (st != DQ_OK) return st;
  int host[2] = {0, 0};
  DQ_TRY(hipMemcpyAsync(host, status, sizeof host, hipMemcpyDeviceToHost, stream));
  DQ_TRY(hipStreamSynchronize(stream));
  return map_status(host[0]);
}

size_t dq_batch_workspace_bytes(int n, const dq_batch_item* items, dq_format fmt, int group) {
  if (n < 1 || n > DQ_BATCH_MAX || !items || !fmt_ok(fmt)) return 0;
  size_t total = 0;
  for (int k = 0; k < n; k++) {
    if (!shape_ok(items[k].rows, items[k].cols, group)) return 0;
    total += align_up(make_plan(items[k].rows, items[k].cols, fmt, group).total);
  }
  return total;
}

dq_status dq_solve_batch(int n, const dq_batch_item* items, dq_dtype wt, dq_format fmt, int group,
                         int T, unsigned flags, dq_status* item_status, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  using namespace dq;
  if (n < 1 || n > DQ_BATCH_MAX || !items || T < 0) return DQ_ERR_ARG;
  if (!fmt_ok(fmt) || wt != DQ_BF16) return DQ_ERR_UNSUPPORTED;
  const bool pass_g = fmt == DQ_FMT_NVFP4 && (flags & DQ_SOLVE_PER_PASS_G);
  for (int k = 0; k < n; k++) {
    const dq_batch_item& it = items[k];
    dq_status st = check_common(it.W, wt, it.rows, it.cols, fmt, group, it.codes, it.inner_scales);
    if (st != DQ_OK) return st;
    if (!scale_outputs_ok(it.a, it.b) || !it.mse || (fmt == DQ_FMT_NVFP4 && !it.tensor_scale))
      return DQ_ERR_ARG;
    if (it.g0 != it.g0 || it.g0 > 3.4028234663852886e38f || (pass_g && it.g0 > 0.0f))
      return DQ_ERR_ARG;
  }
  const size_t need = dq_batch_workspace_bytes(n, items, fmt, group);
  WsGuard ws;
  if (workspace) {
    if (workspace_bytes < need) return DQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return DQ_ERR_ARG;
    ws.ptr = static_cast<char*>(workspace);
    ws.s = stream;
  } else {
    void* ptr = nullptr;
    DQ_TRY(hipMallocAsync(&ptr, need, stream));
    ws.ptr = static_cast<char*>(ptr);
    ws.owned = true;
    ws.s = stream;
  }
  std::vector<BatchMat> mats(n);
  size_t off = 0;
  for (int k = 0; k < n; k++) {
    const dq_batch_item& it = items[k];
    BatchMat& m = mats[k];
    m.p = make_plan(it.rows, it.cols, fmt, group);
    m.ws = ws.ptr + off;
    off += align_up(m.p.total);
    m.io = SolveIo{it.W, true, nullptr, it.codes, it.inner_scales, it.tensor_scale, it.a, it.b,
                   it.mse, T};
    m.pass_g = pass_g;
    dq_init init{it.a0, it.b0, it.g0, flags};
    dq_status st = m.setup(&init, stream);
    if (st != DQ_OK) return st;
  }
  for (int t = 0; t < T; t++) {
    dq_status st = batch_iteration(mats.data(), n, t, stream);
    if (st != DQ_OK) return st;
  }
  for (int k = 0; k < n; k++) {
    dq_status st = mats[k].emit(stream);
    if (st != DQ_OK) return st;
  }
  // every matrix's status word
  std::vector<int> host(2 * (size_t)n, 0);
  for (int k = 0; k < n; k++)
    DQ_TRY(hipMemcpyAsync(&host[2 * k], mats[k].status, 2 * sizeof(int), hipMemcpyDeviceToHost,
                          stream));
  DQ_TRY(hipStreamSynchronize(stream));
  dq_status first = DQ_OK;
  for (int k = 0; k < n; k++) {
    const dq_status st = map_status(host[2 * k]);
    if (item_status) item_status[k] = st;
    if (first == DQ_OK) first = st;
  }
  return first;
}

}  // extern "C"
