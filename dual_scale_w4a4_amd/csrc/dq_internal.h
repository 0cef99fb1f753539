// dq_internal.h -- kernel argument blocks and launchers shared by dq_kernels.hip and dq_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

enum Fmt : int { kInt4Bf16 = 0, kMxInt4 = 1, kMxFp4 = 2, kNvFp4 = 3 };

// finalize: columns per 256-thread block (32 lanes add each column's partial sums)
constexpr int kFinColsPerBlock = 8;

// device status word bits
enum : int {
  kStNonFinite = 1,  // W has a NaN / Inf
  kStRange = 2,      // a scaled value overflowed
  kStInitArg = 4,    // an init value was not finite and positive
  kStGauge = 8,      // the MX single-sweep identity could not be guaranteed
  kStInternal = 16,  // N <= 0 with D > 0 (cannot happen with exact products)
};

// sweep modes (bit set)
enum : int { kModeRow = 1, kModeCol = 2, kModeEmit = 4, kModeGauge = 8, kModeYmax = 16, kModeStat = 32 };

struct SweepArgs {
  const void* W;
  int64_t m, n;
  int G;
  const float* ra;  // rows: fl32(1 / a), the synced inner copy
  const float* rb;  // cols: fl32(1 / b)
  const float* a;   // rows: outer inverse scales (column sums use a_i * d_ig)
  const float* b;   // cols: outer inverse scales (row sums use q_ij * b_j)
  const float* gs;  // NVFP4: gs[0] = g, gs[1] = fl32(6 g)
  int nct;          // column tiles of 512 columns
  int nrc;          // row chunks
  int64_t rpc;      // rows per chunk
  double2* rowpart;  // [nct][m] (N, D)
  double2* colpart;  // [nrc][n] (P, Q)
  uint8_t* codes;
  void* scales;
  int* status;
  float* ymax;       // kModeYmax: [nct][m] row maxima of |fl32(W rb)| per column tile
  double* epart;     // kModeStat (two-sweep pass): [nct][m] sums of W^2 over each tile's columns
};

// Single-sweep MX pass on bf16 weights (see k_fused_mx).
struct FusedArgs {
  const uint16_t* W;
  int64_t m, n;
  int G;
  const float* rb;
  const float* b;
  int nct;          // column tiles of 512 * halves columns
  int nrc;          // row chunks
  int64_t rpc;      // rows per chunk
  int halves;       // 512-column halves per lane: 1 or 2
  int step_rows;    // rows per load step: 2 or 4
  int ahead;        // load steps in flight: 1, or 3 with one half and two rows per step
  double2* rowpart;  // [nct][m] (sum_j W t, sum_j (W - t)^2) with t = S b: R = ra * t
  double2* colpart;  // [nrc][n] (sum_i W S, sum_i S^2)
  double* epart;     // first pass (or null): [nct][m] partial sums of W^2 over each tile's columns
  // final pass only: packed codes, E8M0 inner scales, the outer row scales
  uint8_t* codes;
  uint8_t* scales;
  const float* a;
  int* status;
};

// Row-resident iteration pass on bf16 weights (see k_rowres): both Q evaluations of an
// iteration from one read of W, for formats whose row update changes the codes.
struct RowResArgs {
  const uint16_t* W;
  int64_t m, n;
  int G;
  float* a;          // rows: in the current a, out the updated a'
  float* ra;         // rows: in fl32(1 / a), out fl32(1 / a')
  const float* rb;   // cols: fl32(1 / b)
  const float* b;    // cols
  const float* gs;   // NVFP4: gs[0] = g, gs[1] = fl32(6 g)
  const double* E;   // rows: sum_j W_ij^2
  double* rowerr;    // rows, out: E_i - 2 a_i N_i + a_i^2 D_i of the state before the update
  double2* colpart;  // [workgroups][n] (P, Q) with S = D_a' Qhat'
  int64_t rpc;       // rows per workgroup, a multiple of rowres_batch_rows(n)
  int* status;
};

struct RowStatArgs {
  const void* W;
  int64_t m, n;
  const float* ra;
  const float* rb;
  double* E;     // rows: sum_j W_ij^2
  float* amax;   // rows: max_j |X_ij| (may be null)
  int* status;
};

struct VecArgs {
  const float* src;  // may be null: ones
  float* dst;
  float* rdst;       // fl32(1 / dst)
  float* dst2;       // optional second copy of dst
  int64_t len;
  int fmt;
  int project;       // 1: project src onto the format's scale set
  int envelope;      // 1: flag kStGauge if a value leaves [2^-24, 2^24] (single-sweep range)
  int* status;
};

struct ScaleArgs {
  const float* amax;
  int64_t m;
  const float* g_in;  // device pointer to a caller value (> 0 fixes g), may be null
  float g_fixed;      // host value (> 0 fixes g)
  float* gs;          // out: g, fl32(6 g)
  float* g_out;       // out: copy of g for the caller (may be null)
  int* status;
};

struct FinArgs {
  int64_t m, n;
  int fmt;
  // rows
  int nblk_rows;
  const double2* rowpart;
  int nct;
  double* E;
  const double* epart;  // if set: E_i = sum over the nct tiles of epart, stored into E first
  float* a;
  float* ra;
  int update_a;
  int gauge_check;
  int row_ra;          // single-sweep MX sums: rowpart holds (N', e) with R = ra_i t
  int envelope;        // flag kStGauge if a new a or b leaves [2^-24, 2^24]
  int col_terms;       // single-sweep: bound on the fp32 additions behind one column sum
  double* part_out;         // per-block row-error sums of this launch, or null
  const double* prev_part;  // a previous launch's block sums to finish, or null
  int prev_count;
  double* prev_out;         // where their mean goes
  double inv_mn;
  // cols
  int nblk_cols;        // blocks of 32 columns
  const double2* colpart;
  int nrc;
  float* b;
  float* rb;
  int* status;
  // rows, NVFP4 with a per-pass tensor scale: the row pass's [nct][m] maxima of |y| in, and
  // the next pass's row maxima of |x| out
  const float* ymax;
  float* amax_out;
  // rows: per-row errors already formed by the row-resident pass (then the rows' part only
  // adds them up; rowpart is not read)
  const double* rowerr;
};

// Several matrices per launch (a batch solve): workgroups [start[k], start[k+1]) belong to
// matrix k; the argument blocks travel in the kernel arguments.
constexpr int kMaxMulti = 16;  // keeps FinMulti (the larger block) under 4 KiB of arguments
struct PassMulti {
  int n;
  int start[kMaxMulti + 1];
  SweepArgs a[kMaxMulti];
};
struct FinMulti {
  int n;
  int start[kMaxMulti + 1];
  FinArgs a[kMaxMulti];
};
static_assert(sizeof(FinMulti) <= 4096 && sizeof(PassMulti) <= 4096, "kernel argument size");

// Activation quantization x = fl32(X * b), then Q (dq_act.hip).
struct ActArgs {
  const void* X;
  int64_t m, n;      // tokens, channels
  int G;
  const float* b;    // channels, or null for ones
  float g;           // NVFP4: the tensor scale when gs is null
  const float* gs;   // NVFP4: device tensor scale (from the amax pass), or null
  float* gs_out;     // the amax pass's result
  float* g_out;      // NVFP4: the tensor scale used, for the caller (may be null)
  float* part;       // amax pass: per-block maxima
  int nct, nrc;      // tiles of act_tile_cols() channels, chunks of rpc tokens
  int64_t rpc;
  uint8_t* codes;
  void* scales;
  int* status;
};

hipError_t launch_clear(int* words, int count, hipStream_t s);
// reads `vec16` 16-byte words of buf in full (to evict other data from the caches); `sink`
// is written only if the data has an impossible checksum, so that the reads stay
hipError_t launch_flush(const void* buf, size_t vec16, int* sink, hipStream_t s);
hipError_t launch_vec(const VecArgs& a, hipStream_t s);
hipError_t launch_rowstat(bool bf16, const RowStatArgs& a, hipStream_t s);
hipError_t launch_tensor_scale(const ScaleArgs& a, hipStream_t s);
hipError_t launch_sweep(int fmt, bool bf16, int mode, const SweepArgs& a, hipStream_t s);
// two-sweep pass for bf16 weights (dq_pass.hip): mode kModeRow, kModeCol or kModeRow | kModeEmit;
// SweepArgs::nct counts tiles of pass_tile_cols() columns
hipError_t launch_pass(int fmt, int mode, const SweepArgs& a, hipStream_t s);
int pass_tile_cols();
hipError_t launch_pass_multi(int fmt, int mode, const PassMulti& m, hipStream_t s);
hipError_t launch_finalize_multi(const FinMulti& m, hipStream_t s);
hipError_t launch_act(int fmt, bool bf16, const ActArgs& a, hipStream_t s);
hipError_t launch_act_gscale(bool bf16, const ActArgs& a, hipStream_t s);  // amax pass + g
int act_tile_cols();
int act_amax_blocks();
hipError_t launch_finalize(const FinArgs& a, hipStream_t s);
// row-resident pass (dq_rowres.hip): nwg workgroups of rowres_lanes(n) threads, each owning
// RowResArgs::rpc rows (a multiple of rowres_batch_rows(n)); for the shapes rowres_shape_ok
// accepts (INT4_BF16 and NVFP4 rows of up to 4096 columns)
hipError_t launch_rowres(int fmt, const RowResArgs& a, int nwg, hipStream_t s);
bool rowres_shape_ok(int fmt, int64_t n);
int rowres_lanes(int64_t n);
int rowres_batch_rows(int64_t n);
hipError_t launch_fused(int fmt, bool emit, const FusedArgs& a, hipStream_t s);  // a.epart: first pass
hipError_t launch_mse_collect(const double* part, int count, double* out, double inv_mn,
                              hipStream_t s);

}  // namespace dq
