/*
 * dq.h -- C ABI of libdq.so, the MI355X (gfx950) DualQuant dual-scale weight-reconstruction
 * solver.
 *
 * The method (DualQuant pages: daiwk reproduction notes, "核心公式" eq. 1-2 and the
 * conventions under them; trove summary, "How it works"):
 *   W ~= D_a * Qhat * D_b,   Qhat = Q(D_alpha * W * D_beta),   a = 1/alpha, b = 1/beta,
 * solved by block-coordinate descent that needs only the static weight: quantize the scaled
 * tile, update every row's outer inverse scale a_i in closed form (1-D least squares against
 * R = Qhat D_b) and project it onto the format's scale set, re-quantize with the inner copies
 * synced (alpha = 1/a), update every column's b_j the same way against S = D_a Qhat, project,
 * re-quantize; repeat T times. An all-zero slice takes scale 1.
 *
 * Conventions shared by every entry point:
 *  - Array arguments are DEVICE pointers owned by the caller (for example torch tensors).
 *    The library never frees or retains them. W must be 16-byte aligned, codes 4-byte
 *    aligned; all arrays are dense and row-major.
 *  - W is rows x cols: a row is an output channel, a column an input channel (X W^T).
 *    Groups of `group` consecutive columns share one inner scale. cols % group == 0 and
 *    group is 16, 32 or 64.
 *  - Arguments are checked on the host before anything is enqueued; on a failed check the
 *    call returns DQ_ERR_ARG / DQ_ERR_UNSUPPORTED / DQ_ERR_WORKSPACE and enqueues nothing.
 *  - Work is enqueued on `stream`; the call then synchronizes `stream` so that errors found
 *    on the device (non-finite W, non-finite scaled values, invalid init values) can be
 *    returned. Outputs are unspecified when the call returns an error.
 *  - Calls keep no state between them: the library holds no global mutable data (except
 *    dq_solve_async_noalloc's scratch, see there). Calls that share a workspace must not
 *    overlap.
 *  - Results are deterministic: every reduction has a fixed order (no floating-point
 *    atomics), so the same inputs give bit-identical outputs.
 *
 * Codes: two per byte, column 2k in the low nibble and 2k+1 in the high nibble. INT4 and
 * MXINT4 codes are two's-complement nibbles (INT4 uses [-8, 7], MXINT4 [-7, 7]); E2M1 codes
 * (MXFP4, NVFP4) are sign in bit 3 and magnitude index 0..7 (0, 0.5, 1, 1.5, 2, 3, 4, 6) in
 * bits 0..2, and a zero is always stored as 0x0.
 * Inner scales: rows x (cols/group) entries: u16 bf16 bits (INT4_BF16), u8 E8M0 biased
 * exponent e + 127 (MXINT4, MXFP4), u8 E4M3FN bits (NVFP4).
 */
#ifndef DQ_H
#define DQ_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DQ_OK = 0,
  DQ_ERR_ARG = 1,         /* invalid argument (checked on the host, or invalid init values) */
  DQ_ERR_UNSUPPORTED = 2, /* unknown format or weight dtype */
  DQ_ERR_NONFINITE = 3,   /* W holds a NaN or an infinity */
  DQ_ERR_RANGE = 4,       /* a scaled value D_alpha W D_beta overflowed */
  DQ_ERR_WORKSPACE = 5,   /* workspace smaller than dq_workspace_bytes() */
  DQ_ERR_HIP = 6,         /* a HIP runtime call failed */
  DQ_ERR_INTERNAL = 7     /* a closed-form numerator was not positive (never expected) */
} dq_status;

/* Formats (daiwk notes Table 1 and "本地复现"; news article's block-format paragraph):
 *  INT4_BF16: INT4 codes, one bf16 inner scale per group (absmax / 7); BF16 outer scales.
 *  MXINT4:    INT4 codes in [-7, 7], E8M0 inner scale per group; E8M0 outer scales with
 *             exponents in [-126, 126].
 *  MXFP4:     E2M1 codes, E8M0 inner scale per group (group 32 is the OCP block); E8M0 outer.
 *  NVFP4:     E2M1 codes, E4M3 inner scale per group (group 16 is the NVIDIA block) times one
 *             fp32 tensor scale g; E4M3 outer scales. */
typedef enum { DQ_FMT_INT4_BF16 = 0, DQ_FMT_MXINT4 = 1, DQ_FMT_MXFP4 = 2, DQ_FMT_NVFP4 = 3 } dq_format;

typedef enum { DQ_F32 = 0, DQ_BF16 = 1 } dq_dtype;

/* Solver options (dq_init.flags). */
#define DQ_SOLVE_TWO_SWEEP 1u /* MX formats: always re-read W for the column pass instead of
                                 reusing the row pass's codes (the general path) */
/* NVFP4 only (ignored for the other formats): recompute the tensor scale g before every Q
 * pass, g = fl32(max|X| / 2688) of the scaled tile about to be quantized (at least 2^-126;
 * 1 if X == 0), instead of fixing it from the initial tile; tensor_scale receives the final
 * pass's g, and init->g0 must then be <= 0. Costs one read of W per Q pass. */
#define DQ_SOLVE_PER_PASS_G 2u

typedef struct {
  const float* a0;   /* device, rows values > 0, or NULL for ones; projected onto the scale set */
  const float* b0;   /* device, cols values > 0, or NULL for ones; projected onto the scale set */
  float g0;          /* NVFP4: > 0 fixes the tensor scale; <= 0 computes it from the initial
                        scaled tile as fl32(max|X| / 2688), at least 2^-126 (1 if X == 0) */
  unsigned flags;    /* DQ_SOLVE_* */
} dq_init;

/* Bytes of device workspace dq_solve / dq_quantize need for this shape (0 on invalid
 * arguments). The workspace is scratch: no contents are expected on entry or kept on exit. */
size_t dq_workspace_bytes(int64_t rows, int64_t cols, dq_format fmt, int group);

/* T >= 0 iterations of the dual-scale block-coordinate descent (daiwk notes, "核心公式"
 * eq. 2; trove summary, "How it works").
 *  W:            rows x cols, fp32 or bf16 (wt).
 *  init:         may be NULL (ones, computed g, default path).
 *  codes:        out, rows*cols/2 bytes, Q(X(a_T, b_T)) packed as described above.
 *  inner_scales: out, rows*(cols/group) entries (u16 or u8, see above).
 *  tensor_scale: out, 1 float: NVFP4's g; ignored (may be NULL) for other formats.
 *  a, b:         out, rows / cols floats: the final outer inverse scales, each exactly a value
 *                of the format's scale set (bf16 normal, 2^k with |k| <= 126, or E4M3FN >= 2^-9).
 *                a is 4-byte and b 16-byte aligned (the passes read b in 128-bit loads).
 *  mse:          out, T+1 doubles: mse[t] = mean (W - D_a Qhat D_b)^2 of the synced state after
 *                t iterations; mse[0] is single-scale round-to-nearest quantization.
 *  workspace:    device scratch of at least dq_workspace_bytes(...) bytes, or NULL to let the
 *                library allocate it with hipMallocAsync / hipFreeAsync on `stream`.
 * Returns DQ_ERR_ARG also when an a0 / b0 value is not finite and positive. */
dq_status dq_solve(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                   int group, int T, const dq_init* init, uint8_t* codes, void* inner_scales,
                   float* tensor_scale, float* a, float* b, double* mse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* One pass of the group quantizer Q on X = fl32(fl32(W * fl32(1/b)) * fl32(1/a)) (daiwk
 * notes, "原始论文总结": Q is a black-box group quantizer of the scaled tile).
 *  a, b: device, rows / cols values > 0 (used as given), or NULL for ones.
 *  tensor_scale_inout: NVFP4 only (else may be NULL): if the stored value is > 0 it is used
 *                      as g, otherwise g is computed from max|X| and written back.
 *  codes, inner_scales: out, as for dq_solve.
 *  workspace: as for dq_solve. */
dq_status dq_quantize(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                      int group, const float* a, const float* b, float* tensor_scale_inout,
                      uint8_t* codes, void* inner_scales, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* dq_solve without the wait, for callers that cannot synchronize per call (a pipeline that
 * solves many matrices, a serving process): the same arguments and results, only enqueued on
 * `stream`, with no host-side retry. Errors found on the device are OR-ed into *status
 * (device, caller-owned, 4-byte aligned; the caller clears it and reads it when it wants;
 * calls on several streams may share it):
 *   1  W holds a NaN or an infinity (DQ_ERR_NONFINITE)
 *   2  a scaled value overflowed (DQ_ERR_RANGE)
 *   4  an init value was not finite and positive (DQ_ERR_ARG)
 *   8  MX formats: the single-sweep pass could not guarantee its result (a group maximum,
 *      a scale or a projection decision outside the range where it is exact); the outputs are
 *      unspecified and the solve must be redone with DQ_SOLVE_TWO_SWEEP, which dq_solve does
 *      by itself
 *  16  internal (never expected)
 * A nonzero status leaves the outputs unspecified. The workspace may be NULL (then allocated and freed stream-ordered). Host-side argument checks return
 * errors as dq_solve does, before anything is enqueued. */
dq_status dq_solve_async(const void* W, dq_dtype wt, int64_t rows, int64_t cols, dq_format fmt,
                         int group, int T, const dq_init* init, uint8_t* codes,
                         void* inner_scales, float* tensor_scale, float* a, float* b,
                         double* mse, int* status, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* dq_solve_async for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. It takes no workspace and
 * calls no allocating routine: its scratch is a device array inside the library of
 * DQ_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the library's first use on that GPU
 * until the process ends. Shapes whose dq_workspace_bytes exceeds it are rejected with
 * DQ_ERR_WORKSPACE before anything is enqueued (64 MiB holds every matrix up to
 * 28672 x 8192 in any format, and much larger ones). `stream` must belong to the current
 * device (else DQ_ERR_ARG). Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (the solve needs none on entry): calls on one GPU must not overlap,
 * so enqueue them on one stream or order their streams; overlapping calls race. Arguments,
 * results and the status word are those of dq_solve_async. */
#define DQ_NOALLOC_SCRATCH_BYTES (64u << 20)
dq_status dq_solve_async_noalloc(const void* W, dq_dtype wt, int64_t rows, int64_t cols,
                                 dq_format fmt, int group, int T, const dq_init* init,
                                 uint8_t* codes, void* inner_scales, float* tensor_scale,
                                 float* a, float* b, double* mse, int* status,
                                 hipStream_t stream);

/* Bytes of device workspace dq_quantize_act needs (0 on invalid arguments); scratch only. */
size_t dq_act_workspace_bytes(int64_t tokens, int64_t cols, dq_format fmt, int group);

/* Activation quantization with the column inverse scales: the consumer side of the
 * factorized product (daiwk notes, "核心公式" eq. 1: X W^T ~= (X D_beta^-1) Qhat^T D_alpha^-1,
 * with D_beta^-1 = D_b; the flowchart scales the real activations by the column inverse
 * scales, then quantizes them; trove summary, "How to use it": beta is applied inside the
 * activation quantizer). Every row (token) of X is scaled channel by channel,
 * x_tj = fl32(X_tj * b_j), and quantized by the weights' group quantizer Q in groups of
 * `group` consecutive channels; the scaled values never go to memory.
 *  X:            tokens x cols, fp32 or bf16 (xt), device, 16-byte aligned, row-major.
 *  b:            device, cols floats > 0 (the solver's column inverse scales, used as given),
 *                16-byte aligned, or NULL for ones.
 *  g:            NVFP4 only: > 0 fixes the tensor scale; <= 0 computes it from this X as
 *                fl32(max|x| / 2688), at least 2^-126 (1 if x == 0), with one extra read of X.
 *  tensor_scale: out (device, 1 float): NVFP4's g as used; ignored (may be NULL) otherwise.
 *  codes:        out, tokens*cols/2 bytes, 8-byte aligned, packed as for dq_solve.
 *  inner_scales: out, tokens*(cols/group) entries (u16 bf16 bits, or u8), as for dq_solve.
 *  workspace:    device scratch of at least dq_act_workspace_bytes(...) bytes, or NULL.
 * Returns DQ_ERR_NONFINITE for a NaN / Inf in X, DQ_ERR_RANGE when X * b overflows; like the
 * other calls it synchronizes `stream` before returning. */
dq_status dq_quantize_act(const void* X, dq_dtype xt, int64_t tokens, int64_t cols,
                          dq_format fmt, int group, const float* b, float g, float* tensor_scale,
                          uint8_t* codes, void* inner_scales, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* dq_quantize_act without the wait, for callers that cannot synchronize per call (a serving
 * loop): the same arguments and results, only enqueued on `stream`. Errors found on the
 * device are OR-ed into *status (device, caller-owned, 4-byte aligned): bit 1 a NaN / Inf
 * in X, bit 2 an overflow of X * b. The caller clears it (0) before the calls it wants to
 * check and reads it afterwards; it accumulates across calls. Only NVFP4 with g <= 0 uses the
 * workspace (which may then be NULL: allocated and freed stream-ordered). Host-side argument
 * checks return errors as dq_quantize_act does, before anything is enqueued. */
dq_status dq_quantize_act_async(const void* X, dq_dtype xt, int64_t tokens, int64_t cols,
                                dq_format fmt, int group, const float* b, float g,
                                float* tensor_scale, uint8_t* codes, void* inner_scales,
                                int* status, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------ batch solves
 * Several matrices of one format solved together, each exactly as dq_solve would solve it
 * (bit-identical results), with the per-iteration passes and updates of several matrices
 * sharing each kernel launch (up to 16 per launch): for a decoder layer's q, k, v, o, gate, up and down weights,
 * whose small matrices alone would leave the GPU idle between launches. bf16 weights only;
 * every matrix takes the two-sweep path (for MX formats its result equals the single-sweep
 * path's). */
#define DQ_BATCH_MAX 64

typedef struct {
  const void* W;         /* device, rows x cols bf16, 16-byte aligned */
  int64_t rows, cols;
  const float* a0;       /* device or NULL, as dq_init.a0 */
  const float* b0;       /* device or NULL, as dq_init.b0 */
  float g0;              /* NVFP4, as dq_init.g0 */
  uint8_t* codes;        /* out, as for dq_solve */
  void* inner_scales;    /* out */
  float* tensor_scale;   /* out, NVFP4 */
  float* a;              /* out, rows, 4-byte aligned */
  float* b;              /* out, cols, 16-byte aligned */
  double* mse;           /* out, T+1 */
} dq_batch_item;

/* Bytes of device workspace for dq_solve_batch (0 on invalid arguments). */
size_t dq_batch_workspace_bytes(int n, const dq_batch_item* items, dq_format fmt, int group);

/* Solve n (1..DQ_BATCH_MAX) matrices. flags: DQ_SOLVE_PER_PASS_G (NVFP4) as for dq_solve.
 * item_status (host, n entries, may be NULL) receives each matrix's status; the return value
 * is the first non-OK one. workspace: as for dq_solve, of dq_batch_workspace_bytes bytes.
 * Arguments are checked on the host before anything is enqueued; the call synchronizes
 * `stream` before returning. */
dq_status dq_solve_batch(int n, const dq_batch_item* items, dq_dtype wt, dq_format fmt, int group,
                         int T, unsigned flags, dq_status* item_status, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ the W4A4 product
 * The matmul the quantized weights are for (daiwk notes, "核心公式" eq. 1: X W^T ~=
 * (X D_b) Qhat^T D_a; the flowchart's last step multiplies the quantized activations by the
 * weight codes and applies the row output scale): MXFP4 activations as dq_quantize_act writes
 * them (codes and E8M0 scales of x = X * b, group 32) times MXFP4 weights as dq_solve writes
 * them (codes and E8M0 scales of Qhat), with the weights' row scales a on the output:
 *     Y[t][i] = a_i * sum_k xhat[t][k] * Qhat[i][k]
 * on gfx950's MX-scaled FP4 matrix cores: both operands stay 4-bit, every product is exact and
 * the sum is accumulated in fp32.
 *  act_codes:  tokens x K/2 bytes, packed as above, 16-byte aligned.
 *  act_scales: tokens x K/32 E8M0 bytes.
 *  w_codes:    out x K/2 bytes, 16-byte aligned.  w_scales: out x K/32 E8M0 bytes.
 *  a:          out floats, 16-byte aligned, or NULL for ones.
 *  Y:          out, tokens x out, row-major, fp32 or bf16 (yt; bf16 rounds to nearest even).
 * K % 32 == 0 and K <= 2^22; any tokens, out >= 1. The fast path wants K % 256 == 0,
 * out % 4 == 0, 8-byte aligned scales and Y aligned to 4 elements; other shapes take a
 * slower path with the same results. An E8M0 byte 0xFF (the format's NaN) makes the outputs
 * it reaches NaN. Arguments are checked on the host; the call only enqueues on `stream`
 * (there is no device-side error to report) and returns. */
dq_status dq_gemm_mx(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                     int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, const float* a,
                     int64_t out, dq_dtype yt, void* Y, hipStream_t stream);

/* The same product with the weights packed once (dq_gemm_pack_weights) into the order the
 * matrix instructions read them, so that the weight operand goes straight from memory into
 * registers and LDS serves only the activations: the faster form for static weights. The
 * packed product sums each 256-k stage in another order than dq_gemm_mx (the results agree
 * to fp32 rounding, not bit for bit). K % 512 == 0 and 512 <= K <= 2^22.
 *
 * dq_gemm_pack_bytes: the sizes of the packed codes and scales for out x K weights (out
 * padded to a multiple of 32 rows). dq_gemm_pack_weights: writes them (device buffers of
 * those sizes; codes 16-byte and scales 4-byte aligned, as are w_codes and w_scales) from the
 * weight codes and E8M0 scales as dq_solve writes them; padding rows get zero codes and scale
 * 2^0. Layout: for each 32-row block rb, 256-k stage s and k step i (0..3), 1 KiB in which
 * lane L (0..63) holds the 16 code bytes of row 32 rb + L % 32, k values
 * 256 s + 32 (4 (L / 32) + i) .. + 31; for each rb and s, 256 bytes in which lane L holds the 4
 * scale bytes of row 32 rb + L % 32, k blocks 8 s + 4 (L / 32) .. + 3. Only enqueues.
 * dq_gemm_mx_packed: as dq_gemm_mx with the packed weights (act_scales 16-byte aligned). */
dq_status dq_gemm_pack_bytes(int64_t out, int64_t K, size_t* codes_bytes, size_t* scales_bytes);
dq_status dq_gemm_pack_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t out,
                               int64_t K, uint8_t* packed_codes, uint8_t* packed_scales,
                               hipStream_t stream);
dq_status dq_gemm_mx_packed(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                            int64_t K, const uint8_t* packed_codes, const uint8_t* packed_scales,
                            const float* a, int64_t out, dq_dtype yt, void* Y,
                            hipStream_t stream);

/* Static string for a status code. */
const char* dq_status_str(dq_status status);

#ifdef __cplusplus
}
#endif
#endif /* DQ_H */
