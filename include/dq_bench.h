/*
 * dq_bench.h -- measurement hooks of libdq.so. They are not part of the solver's interface
 * (include/dq.h): they serve benchmarks and launch-shape sweeps. A solve through them gives
 * the same results as dq_solve when the launch shape is the default one; another launch shape
 * splits the fixed-order sums differently, so a, b and mse may then differ in their last bits.
 */
#ifndef DQ_BENCH_H
#define DQ_BENCH_H

#include "dq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Per-kernel timing of one solve (HIP events recorded on `stream` around each launch, which
 * adds a little overhead). Index ms / launches by dq_kernel_kind. */
typedef enum {
  DQ_K_SETUP = 0,  /* init vectors, row statistics, tensor scale */
  DQ_K_FUSED = 1,  /* MX single-sweep pass: codes, row sums and column sums */
  DQ_K_ROW = 2,    /* general row pass */
  DQ_K_COL = 3,    /* general column pass */
  DQ_K_FINAL = 4,  /* closed-form updates and projections */
  DQ_K_EMIT = 5,   /* final codes and inner scales */
  DQ_K_ROWRES = 6, /* row-resident pass: both Q evaluations of an iteration from one read */
  DQ_K_KINDS = 7
} dq_kernel_kind;

typedef struct {
  double ms[DQ_K_KINDS];
  int64_t launches[DQ_K_KINDS];
  int used_fused; /* 1 if the MX single-sweep path produced the result */
  /* single-sweep path only: after the solve, the pass is re-run isolated_launches times
     back to back between one pair of events (results unchanged); this is its time */
  double isolated_ms;
  int isolated_launches;
  /* in (kept by the call): an optional device buffer of flush_bytes bytes (a multiple of 16).
     When given, the re-runs are also timed one launch at a time, cold_ms after a full read
     of this buffer before each launch (evicting W from the caches when it is larger than
     them) and warm_ms without it; per_launch re-runs each */
  const void* flush;
  size_t flush_bytes;
  double cold_ms;
  double warm_ms;
  int per_launch;
} dq_timing;

/* Launch shape of the iteration passes; a field <= 0 keeps the default.
 *  fused_halves:     single-sweep MX pass, 512-column halves per lane (1 or 2; default 1)
 *  fused_step_rows:  single-sweep MX pass, rows per load step (2 or 4; default 2)
 *  fused_target:     single-sweep MX pass, target workgroup count (default 512, and 768 for a
 *                    matrix whose bf16 W exceeds 256 MiB; a value given here applies to both)
 *  fused_ahead:      single-sweep MX pass, load steps in flight per wave (1 or 3; 3 only with
 *                    one half and two rows per step; default 1)
 *  pass_target:      two-sweep pass for bf16 weights, target workgroup count (default 768)
 *  sweep_target:     general sweep (fp32 weights), target workgroup count (default 512)
 *  row_resident:     INT4_BF16 / NVFP4 on bf16 weights (tensor scale fixed for the solve), rows
 *                    of up to 4096 columns: 1 takes the row-resident pass (one read of W per
 *                    iteration), -1 or 0 the two-sweep passes (the default: they solve a
 *                    whole decoder layer faster on MI355X)
 *  rowres_target:    row-resident pass, target workgroup count (default 256) */
typedef struct {
  int fused_halves;
  int fused_step_rows;
  int fused_target;
  int pass_target;
  int sweep_target;
  int row_resident;
  int rowres_target;
  int fused_ahead;
} dq_launch_shape;

/* dq_workspace_bytes for a solve in the given launch shape (NULL: the default one). */
size_t dq_bench_workspace_bytes(int64_t rows, int64_t cols, dq_format fmt, int group,
                                const dq_launch_shape* shape);

/* dq_solve in the given launch shape (NULL: the default one), filling *timing (may be NULL).
 * The arguments, checks, results and blocking behaviour are those of dq_solve; the workspace
 * must hold dq_bench_workspace_bytes(..., shape) bytes. Returns DQ_ERR_ARG for a launch-shape
 * field outside its range. */
dq_status dq_solve_timed(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                         int group, int T, const dq_init* init, uint8_t* codes,
                         void* inner_scales, float* tensor_scale, float* a, float* b,
                         double* mse, void* workspace, size_t workspace_bytes,
                         const dq_launch_shape* shape, dq_timing* timing, hipStream_t stream);

/* The matrix cores' attainable rate for the W4A4 product's instruction (the scaled 32x32x64
 * MFMA with E2M1 operands and E8M0 scales): a stream of it on register operands only, nothing
 * read or written in the loop, eight independent accumulators per wave and four 4-wave
 * workgroups per CU, `iters` rounds of eight instructions per wave (1 .. 2^20), timed with HIP
 * events on `stream` after one untimed launch. *tflops receives the dense-equivalent TFLOP/s
 * (2 * 32 * 32 * 64 flops per instruction): what the chip sustains at the clock it holds under
 * such load, beside the published peak. Blocks until the timed launch ends. Returns DQ_ERR_ARG
 * for iters out of range or a null tflops, DQ_ERR_HIP if a HIP call fails. */
dq_status dq_bench_fp4_mfma_rate(int iters, hipStream_t stream, double* tflops);

#ifdef __cplusplus
}
#endif
#endif /* DQ_BENCH_H */
