/*
 * dq_ref.h -- CPU oracle for the DualQuant dual-scale weight-reconstruction solver.
 *
 * TEST INFRASTRUCTURE. This library is the plain, slow, double-precision
 * reference that the HIP library is checked against. Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does. It shares no source, header or constant table with
 * the HIP library: its format ids and status codes are defined here on their
 * own, with the same numeric values the HIP header uses for the same meaning.
 *
 * Method (DualQuant, daiwk reproduction notes "核心公式" eq. 1-2 and the
 * trove summary "How it works"):
 *   W ~= D_a * Qhat * D_b,  Qhat = Q(D_alpha W D_beta),  a = 1/alpha, b = 1/beta
 *   row update    a_i <- Pi_F( sum_j W_ij R_ij / sum_j R_ij^2 ),  R = Qhat D_b
 *   re-quantize with the inner copies synced (alpha = 1/a)
 *   column update b_j <- Pi_F( sum_i W_ij S_ij / sum_i S_ij^2 ), S = D_a Qhat
 *   re-quantize; repeat T times; an all-zero slice gets scale 1.
 *
 * All pointers are HOST pointers owned by the caller. Calls are synchronous and
 * single-threaded unless dq_ref_set_threads() asked for more (the result is
 * bit-identical for any thread count: every sum keeps its ascending order).
 */
#ifndef DQ_REF_H
#define DQ_REF_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* formats: 0 INT4 codes + BF16 scales, 1 MXINT4, 2 MXFP4, 3 NVFP4 */
#define DQR_FMT_INT4_BF16 0
#define DQR_FMT_MXINT4 1
#define DQR_FMT_MXFP4 2
#define DQR_FMT_NVFP4 3
/* weight element types */
#define DQR_F32 0
#define DQR_BF16 1
/* status */
#define DQR_OK 0
#define DQR_ERR_ARG 1
#define DQR_ERR_UNSUPPORTED 2
#define DQR_ERR_NONFINITE 3
#define DQR_ERR_RANGE 4
#define DQR_ERR_INTERNAL 7

/* One Q pass on X = fl32(fl32(W * fl32(1/b)) * fl32(1/a)).
 * a (rows), b (cols): NULL means all ones; otherwise every value must be > 0
 * and finite (they are used as given, not projected).
 * g_inout (NVFP4 only): if *g_inout > 0 it is used, else g is computed from
 * max|X| and written back. codes: rows*cols/2 bytes, column 2k in the low
 * nibble. scales: rows*(cols/group) entries, u16 BF16 bits (INT4_BF16) or u8
 * (E8M0 biased exponent, or E4M3FN bits). */
int dq_ref_quantize(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group,
                    const float* a, const float* b, float* g_inout, uint8_t* codes,
                    void* scales);

/* Activation quantization with the column inverse scales (the consumer side of the
 * factorized product): x_tj = fl32(X_tj * b_j) for X of tokens x cols (xt: DQR_F32 or
 * DQR_BF16), then Q per group of `group` consecutive channels, exactly as dq_ref_quantize
 * quantizes a scaled weight tile. b: NULL means ones, else positive and finite values used
 * as given. g_inout (NVFP4 only): if *g_inout > 0 it is used, else g = fl32(max|x| / 2688)
 * (at least 2^-126; 1 if x == 0) is computed and written back. codes and scales are laid
 * out as for dq_ref_quantize. */
int dq_ref_quantize_act(const void* X, int xt, int64_t tokens, int64_t cols, int fmt, int group,
                        const float* b, float* g_inout, uint8_t* codes, void* scales);

/* The W4A4 product of MXFP4 activations (codes tokens x K/2 bytes, E8M0 scales tokens x K/32)
 * and MXFP4 weights (codes out x K/2, scales out x K/32) with the weights' row scales a (out
 * floats > 0, or NULL for ones): Y[t][i] = a_i * sum_k xhat[t][k] Qhat[i][k] (tokens x out
 * doubles), the sum in double in ascending k. K % 32 == 0. */
int dq_ref_gemm_mx(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                   int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int64_t out,
                   const float* a, double* Y);

/* T iterations of the block-coordinate descent. a0/b0: NULL means ones, else
 * projected onto the format's scale set first; g0 > 0 fixes the NVFP4 tensor
 * scale, g0 <= 0 computes it from the initial scaled tile. Outputs: final codes
 * and inner scales of Q(X(a_T, b_T)), g (NVFP4; may be NULL otherwise), a, b,
 * mse[0..T] (mse[t] = mean squared reconstruction error of the synced state
 * after t iterations). */
int dq_ref_solve(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group, int T,
                 const float* a0, const float* b0, float g0, uint8_t* codes, void* scales,
                 float* g_out, float* a, float* b, double* mse);

/* NVFP4 (group 16) with the tensor scale recomputed before every Q pass: g =
 * fl32(max|X| / 2688) (at least 2^-126; 1 if X == 0) of the scaled tile about to be
 * quantized, for each synced state, each re-quantization after a row update and the final
 * pass. g_out receives the final pass's g. Other arguments as dq_ref_solve. */
int dq_ref_solve_pass_g(const void* W, int wt, int64_t rows, int64_t cols, int group, int T,
                        const float* a0, const float* b0, uint8_t* codes, void* scales,
                        float* g_out, float* a, float* b, double* mse);

/* dq_ref_solve plus diagnostics (either pointer may be NULL):
 * changes[4*t + 0/1]: codes / inner scales that differ between the synced state
 *                     before iteration t and the re-quantization after its row update;
 * changes[4*t + 2/3]: the same between that re-quantization and the one after its
 *                     column update;
 * margin[2*t + 0/1]:  smallest relative distance |v - boundary| / v over the
 *                     row (0) and column (1) updates of iteration t, where v = N/D
 *                     and boundary is the nearest decision point of the projection. */
int dq_ref_solve_diag(const void* W, int wt, int64_t rows, int64_t cols, int fmt, int group,
                      int T, const float* a0, const float* b0, float g0, uint8_t* codes,
                      void* scales, float* g_out, float* a, float* b, double* mse,
                      int64_t* changes, double* margin);

/* Scalar pieces, exposed so that tests can pin them against brute force. */
double dq_ref_project(int fmt, double v);       /* Pi_F of an outer inverse-scale, v > 0 */
double dq_ref_proj_margin(int fmt, double v);   /* relative distance of v to Pi_F's nearest decision point */
double dq_ref_bf16_rne(double v);               /* nearest bf16, ties to even (v >= 0) */
double dq_ref_e4m3_rne_sat(double v);           /* nearest E4M3FN, ties to even, <= 448 */
double dq_ref_e2m1_round(double v);             /* nearest E2M1 value, ties to even index */
int dq_ref_set_threads(int n);                  /* OpenMP threads; returns the count in use */

#ifdef __cplusplus
}
#endif
#endif
