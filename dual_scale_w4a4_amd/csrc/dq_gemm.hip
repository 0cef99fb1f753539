// dq_gemm.hip -- the W4A4 product that the dual-scale weights are for, on gfx950's MX-scaled
// FP4 matrix cores.
//
// What it computes (daiwk notes, "核心公式" eq. 1: X W^T ~= (X D_b) Qhat^T D_a; the flowchart
// ends in the matmul of the quantized activations with the weight codes, then the row output
// scale): with MXFP4 activations x^ = Q(X D_b) (tokens x K codes and E8M0 block scales, as the
// activation quantizer writes them) and MXFP4 weights Qhat (out x K codes and E8M0 block
// scales, as the solver writes them),
//     Y[t][i] = a_i * sum_k x^[t][k] * Qhat[i][k],
// with every product exact (E2M1 x E2M1 times two powers of two), the sum in the matrix
// cores' fp32 accumulators, and a_i applied in the epilogue. Neither operand is ever
// expanded: both stay 4-bit from HBM to the matrix cores, and their E8M0 bytes are the
// instructions' block scales as they are.
//
// Tiling: a workgroup of four waves owns a 256 (weight rows) x 256 (tokens) tile of Y; each
// wave a 128 x 128 quarter as 4 x 4 V_MFMA_SCALE_F32_32X32X64_F8F6F4 blocks (256 fp32
// accumulators per lane). The weights are the instruction's A operand and the tokens its B
// operand, so that a lane's 16 results of one block hold 4 runs of 4 consecutive output
// channels of one token: the epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes at a time.
// K runs in stages of 256 (128 code bytes per row): both operands' stages go through LDS,
// double-buffered, loaded one stage ahead into registers with buffer loads (rows past the end
// read as zero); in LDS a row's eight 16-byte chunks are XOR-swizzled so that neither the
// stores nor the operand reads (a lane reads one 16-byte chunk of its row) conflict. Block
// scales go from global memory straight to registers, one stage ahead.
//
// Operand layouts of the scaled MFMA (checked exactly on gfx950): lane l holds row l % 32 of
// A (column l % 32 of B) for the 32 k values (l / 32) * 32 .. + 31 of the 64-k step, as four
// dwords with value e in nibble e % 8 of dword e / 8 (low nibble first: the packed code
// layout), and its scale byte applies to those 32 values; result v of lane l is
// D[(v / 4) * 8 + (l / 32) * 4 + v % 4][l % 32].
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/dq.h"
#include "../../include/dq_bench.h"

namespace dqg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;                   // weight rows (output channels) per workgroup
constexpr int kBN = 256;                   // tokens per workgroup
constexpr int kBK = 256;                   // k per stage
constexpr int kRowB = kBK / 2;             // code bytes of one row in a stage (8 chunks)
constexpr int kTileB = kBM * kRowB;        // 32 KiB: one operand's stage
constexpr int kThreads = 256;
constexpr int kGroupM = 4;                 // weight tiles per tile group (L2 reuse)
constexpr uint32_t kBufRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

struct GemmArgs {
  const uint8_t* xc;  // tokens x K/2
  const uint8_t* xs;  // tokens x K/32
  const uint8_t* wc;  // out x K/2
  const uint8_t* ws;  // out x K/32
  const float* a;     // out, or null
  void* y;            // tokens x ldy
  int tokens, out, K;
  int64_t ldy;
  int nti, ntt;
};

// Chunk position of chunk c (0..7) of LDS row r: conflict-free for eight lanes on eight
// consecutive rows (one 128-byte bank sweep) and for sixteen (a 256-byte one).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           (int)kBufRsrcWord3);
}

// One operand's stage: 256 rows x 128 bytes, thread tid loads chunk tid % 8 of rows
// tid / 8 + 32 j. The per-thread part of the offset is one register; the row step 32 j and
// the stage go in the wave-uniform offset. Rows past the operand's end (and, on a partial last
// stage, chunks past K) take an offset beyond any buffer and read zero.
constexpr uint32_t kOob = 0x80000000u;

template <bool FULLK>
__device__ __forceinline__ void load_stage(__amdgpu_buffer_rsrc_t rs, int row0, int rows,
                                           int ldb, int kb0, int tid, u32x4 (&v)[8]) {
  const int c = tid & 7, r0 = tid >> 3;
  const uint32_t vbase = (uint32_t)(row0 + r0) * (uint32_t)ldb + (uint32_t)(c * 16);
  const bool kin = FULLK || kb0 + c * 16 < ldb;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const bool in = kin && row0 + r0 + 32 * j < rows;
    v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? vbase : kOob,
                                                 (uint32_t)(32 * j * ldb + kb0), 0);
  }
}

__device__ __forceinline__ void store_stage(uint8_t* lds, int tid, const u32x4 (&v)[8]) {
  const int c = tid & 7;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int r = (tid >> 3) + 32 * j;
    *reinterpret_cast<u32x4*>(lds + r * kRowB + swz(r, c) * 16) = v[j];
  }
}

// Block scales of one row for one stage. FULLK (K % 256 == 0): the stage's 8 bytes of the
// row, loaded raw in one aligned load and unpacked only when the stage is stored, so that the
// load stays in flight during the previous stage's products. `voff` is the row's offset (or
// kOob past the end), `soff` the uniform rest.
__device__ __forceinline__ u32x2 load_scales_raw(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                 uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
}

// The four scale bytes lane `lane` uses in a stage: byte ks is the scale of k block
// 8 s + 2 ks + lane / 32 (the lane's half of k step ks). Rows past the end give 127 (2^0;
// their codes are zero).
__device__ __forceinline__ uint32_t unpack_scales(u32x2 w, bool in_rows, int lane) {
  const uint64_t v = (((uint64_t)w[1] << 32) | w[0]) >> (8 * (lane >> 5));
  const uint32_t out = (uint32_t)(v & 0xFFu) | (uint32_t)((v >> 8) & 0xFF00u) |
                       (uint32_t)((v >> 16) & 0xFF0000u) | (uint32_t)((v >> 24) & 0xFF000000u);
  return in_rows ? out : 0x7F7F7F7Fu;
}

// The same for any K % 32 == 0, byte by byte (blocks past K also give 127).
__device__ __forceinline__ uint32_t load_scales_bytes(const uint8_t* sp, int row, int rows,
                                                      int nkb, int s, int lane) {
  uint32_t out = 0;
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    const int kb = 8 * s + 2 * ks + (lane >> 5);
    const uint32_t b = (row < rows && kb < nkb) ? sp[(int64_t)row * nkb + kb] : 127u;
    out |= b << (8 * ks);
  }
  return out;
}

// 16 scaled MFMAs of one k step: fa / fb the lane's chunks of the four weight-row and four
// token blocks, sw / sx the packed scale bytes.
__device__ __forceinline__ void mfma_step(v16f (&acc)[4][4], const u32x4 (&fa)[4],
                                          const u32x4 (&fb)[4], const uint32_t (&sw)[4],
                                          const uint32_t (&sx)[4], int ks) {
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const v8i A = {(int)fa[m][0], (int)fa[m][1], (int)fa[m][2], (int)fa[m][3], 0, 0, 0, 0};
    const int sa = (int)((sw[m] >> (8 * ks)) & 0xFFu);
#pragma unroll
    for (int n = 0; n < 4; n++) {
      const v8i B = {(int)fb[n][0], (int)fb[n][1], (int)fb[n][2], (int)fb[n][3], 0, 0, 0, 0};
      const int sb = (int)((sx[n] >> (8 * ks)) & 0xFFu);
      acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[m][n], 4, 4, 0, sa,
                                                                  0, sb);
    }
  }
}

__device__ __forceinline__ void read_frags(const uint8_t* lw, const uint8_t* lx, int co,
                                           u32x4 (&fa)[4], u32x4 (&fb)[4]) {
#pragma unroll
  for (int m = 0; m < 4; m++) {
    fa[m] = *reinterpret_cast<const u32x4*>(lw + m * 32 * kRowB + co);
    fb[m] = *reinterpret_cast<const u32x4*>(lx + m * 32 * kRowB + co);
  }
}

// The epilogue. Result v of block (m, n) of the wave is output channel i0 + wi + 32 m +
// 8 (v / 4) + 4 (lane / 32) + v % 4 of token t0 + wt + 32 n + lane % 32, so a lane holds runs
// of 4 channels of one token, and storing them directly would write to 32 rows of Y per
// instruction. Instead the wave's 128 x 128 results go out through LDS, 32 tokens at a time:
// every lane writes its fp32 sums into the wave's region as rows of tokens (128 channels,
// padded by 16 bytes so that the 32 tokens of one write hit distinct banks), then reads back
// 4 channels of one row, 32 lanes to a row, always the same 4 channels: it applies their a
// and stores 8 (bf16) or 16 (fp32) bytes, and each store instruction writes two whole rows
// of 256 or 512 bytes. `stage` is LDS of at least 4 * 32 * 528 bytes, free once the main
// loop is done. VECY: out % 4 == 0 and Y aligned to 4 elements.
constexpr int kRowStage = 128 * 4 + 16;  // padded LDS row of 128 fp32 channels
constexpr int kStageBytes = 4 * 32 * kRowStage;

template <bool BF16, bool VECY, bool EDGE>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const v16f (&acc)[4][4], int i0,
                                           int t0, uint8_t* stage) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rl = lane & 31, h = lane >> 5;
  const int wi = (wave >> 1) * 128, wt = (wave & 1) * 128;
  uint8_t* region = stage + wave * 32 * kRowStage;
  const int ich = i0 + wi + rl * 4;  // the 4 channels this lane stores
  f32x4 av = {1.0f, 1.0f, 1.0f, 1.0f};
  if (p.a) {
    if (!EDGE || ich + 3 < p.out) {
      av = *reinterpret_cast<const f32x4*>(p.a + ich);
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) av[e] = ich + e < p.out ? p.a[ich + e] : 1.0f;
    }
  }
  __syncthreads();  // every wave is done with the main loop's LDS

#pragma unroll
  for (int n = 0; n < 4; n++) {
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const f32x4 y = {acc[m][n][g * 4], acc[m][n][g * 4 + 1], acc[m][n][g * 4 + 2],
                         acc[m][n][g * 4 + 3]};
        *reinterpret_cast<f32x4*>(region + rl * kRowStage + (m * 32 + g * 8 + h * 4) * 4) = y;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int row = h + 2 * r;
      f32x4 y = *reinterpret_cast<const f32x4*>(region + row * kRowStage + rl * 16);
      const int t = t0 + wt + n * 32 + row;
      if (EDGE && t >= p.tokens) continue;
#pragma unroll
      for (int e = 0; e < 4; e++) y[e] *= av[e];
      const bool vec = VECY && (!EDGE || ich + 3 < p.out);
      if (BF16) {
        __bf16* yp = static_cast<__bf16*>(p.y) + (int64_t)t * p.ldy + ich;
        const bf16x4 hv = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        if (vec) {
          __builtin_nontemporal_store(hv, reinterpret_cast<bf16x4*>(yp));
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (ich + e < p.out) yp[e] = hv[e];
        }
      } else {
        float* yp = static_cast<float*>(p.y) + (int64_t)t * p.ldy + ich;
        if (vec) {
          __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(yp));
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (ich + e < p.out) yp[e] = y[e];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next chunk's writes
  }
}

// The stage's 64 products of one wave: four k steps of 16, the next step's operand reads
// issued before this step's products. The scheduling barriers keep that order.
__device__ __forceinline__ void stage_products(v16f (&acc)[4][4], const uint8_t* lw,
                                               const uint8_t* lx, int sterm,
                                               const uint32_t (&sw)[4], const uint32_t (&sx)[4]) {
  u32x4 fa0[4], fb0[4], fa1[4], fb1[4];
  read_frags(lw, lx, (0 ^ sterm) * 16, fa0, fb0);
  read_frags(lw, lx, (2 ^ sterm) * 16, fa1, fb1);
  mfma_step(acc, fa0, fb0, sw, sx, 0);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(lw, lx, (4 ^ sterm) * 16, fa0, fb0);
  mfma_step(acc, fa1, fb1, sw, sx, 1);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(lw, lx, (6 ^ sterm) * 16, fa1, fb1);
  mfma_step(acc, fa0, fb0, sw, sx, 2);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(acc, fa1, fb1, sw, sx, 3);
  __builtin_amdgcn_sched_barrier(0);
}

// One 256 x 256 tile. EDGE: the tile reaches past the last weight row or token (row checks on
// loads and stores); otherwise every row is inside and no check is made.
template <bool BF16, bool FULLK, bool VECY, bool EDGE>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, int i0, int t0,
                                          uint8_t (&lds)[2][2][kTileB]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const int ldb = p.K / 2, nkb = p.K / 32;
  const int nst = (p.K + kBK - 1) / kBK;
  const int rows_w = EDGE ? p.out : INT32_MAX, rows_x = EDGE ? p.tokens : INT32_MAX;

  const __amdgpu_buffer_rsrc_t rwc = rsrc(p.wc, (uint32_t)p.out * (uint32_t)ldb);
  const __amdgpu_buffer_rsrc_t rxc = rsrc(p.xc, (uint32_t)p.tokens * (uint32_t)ldb);
  const __amdgpu_buffer_rsrc_t rws = rsrc(p.ws, (uint32_t)p.out * (uint32_t)nkb);
  const __amdgpu_buffer_rsrc_t rxs = rsrc(p.xs, (uint32_t)p.tokens * (uint32_t)nkb);

  v16f acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; m++)
#pragma unroll
    for (int n = 0; n < 4; n++) acc[m][n] = v16f{};

  const int rl = lane & 31;
  const uint32_t sbw = (uint32_t)(i0 + wi + rl) * (uint32_t)nkb;  // scale row offsets
  const uint32_t sbx = (uint32_t)(t0 + wt + rl) * (uint32_t)nkb;
  u32x4 vw[8], vx[8];
  uint32_t sw[4], sx[4];
  u32x2 rsw[4], rsx[4];

  // stage s's loads: codes into vw / vx, scales raw into rsw / rsx (FULLK) or packed into
  // sw / sx directly (byte path)
  auto issue = [&](int s) {
    load_stage<FULLK>(rwc, i0, rows_w, ldb, s * kRowB, tid, vw);
    load_stage<FULLK>(rxc, t0, rows_x, ldb, s * kRowB, tid, vx);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int iw = i0 + wi + m * 32 + rl, it = t0 + wt + m * 32 + rl;
      if (FULLK) {
        rsw[m] = load_scales_raw(rws, iw < rows_w ? sbw : kOob, m * 32 * nkb + s * 8);
        rsx[m] = load_scales_raw(rxs, it < rows_x ? sbx : kOob, m * 32 * nkb + s * 8);
      }
    }
  };
  auto commit = [&](int s, int buf) {
    store_stage(lds[buf][0], tid, vw);
    store_stage(lds[buf][1], tid, vx);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int iw = i0 + wi + m * 32 + rl, it = t0 + wt + m * 32 + rl;
      if (FULLK) {
        sw[m] = unpack_scales(rsw[m], iw < rows_w, lane);
        sx[m] = unpack_scales(rsx[m], it < rows_x, lane);
      } else {
        sw[m] = load_scales_bytes(p.ws, iw, p.out, nkb, s, lane);
        sx[m] = load_scales_bytes(p.xs, it, p.tokens, nkb, s, lane);
      }
    }
  };

  issue(0);
  commit(0, 0);
  __syncthreads();

  // per-lane LDS read offsets: row wi + m * 32 + lane % 32 (its swizzle term depends on the
  // lane only), chunk 2 ks + lane / 32
  const int sterm = (rl & 7) ^ ((rl >> 3) & 1) ^ (lane >> 5);
  const uint8_t* lw0 = &lds[0][0][(wi + rl) * kRowB];
  const uint8_t* lx0 = &lds[0][1][(wt + rl) * kRowB];
  constexpr int kBufB = 2 * kTileB;

  // stages 0 .. nst - 2: the next stage's loads go out first and stay in flight during this
  // stage's products, then go to the other buffer; the last stage has no successor
  for (int s = 0; s + 1 < nst; s++) {
    const int buf = s & 1;
    issue(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    stage_products(acc, lw0 + buf * kBufB, lx0 + buf * kBufB, sterm, sw, sx);
    commit(s + 1, buf ^ 1);
    __syncthreads();
  }
  stage_products(acc, lw0 + ((nst - 1) & 1) * kBufB, lx0 + ((nst - 1) & 1) * kBufB, sterm, sw,
                 sx);

  store_tile<BF16, VECY, EDGE>(p, acc, i0, t0, &lds[0][0][0]);
}

// Tile order: workgroups are dealt round-robin to the eight XCDs, so consecutive ids are
// spread; give each XCD a contiguous range of tiles, and order tiles in groups of kGroupM
// weight tiles by every token tile, so that the workgroups running together on one XCD share
// weight and token stages in its L2.
__device__ __forceinline__ void tile_origin(const GemmArgs& p, int& i0, int& t0) {
  const int ntiles = p.nti * p.ntt;
  const int bid = blockIdx.x;
  const int full = (ntiles / 8) * 8;
  const int L = bid < full ? (bid % 8) * (ntiles / 8) + bid / 8 : bid;
  const int gsz = kGroupM * p.ntt;
  const int first = (L / gsz) * kGroupM;
  const int gm = min(p.nti - first, kGroupM);
  i0 = (first + (L % gsz) % gm) * kBM;
  t0 = ((L % gsz) / gm) * kBN;
}

template <bool BF16, bool FULLK, bool VECY>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileB];  // [buffer][W, X]

  int i0, t0;
  tile_origin(p, i0, t0);
  if (i0 + kBM <= p.out && t0 + kBN <= p.tokens)
    gemm_tile<BF16, FULLK, VECY, false>(p, i0, t0, lds);
  else
    gemm_tile<BF16, FULLK, VECY, true>(p, i0, t0, lds);
}

// ------------------------------------------------------------ fast path: K % 512 == 0
// The same tile, with both operands' stages moved from global memory straight into LDS by
// gfx950's buffer loads to LDS (no registers, no LDS stores: one wave instruction fills 1 KiB
// of LDS, lane j its 16 bytes at j * 16), so the 4 x 4 fragments of the next k step can be read
// a whole step ahead, and every load sits between two matrix instructions. The block scales go through LDS as well: every second stage each row's
// next 16 scale bytes (two stages' worth, one cache line shared by the 16 k blocks) are
// loaded once for the workgroup, instead of 8 bytes per stage by every wave that uses the row.
constexpr int kScaleRowB = 16;                        // scale bytes per row per period
constexpr int kScaleTileB = kBM * kScaleRowB;         // 4 KiB per operand per period

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct DmaLds {
  uint8_t codes[2][2][kTileB];              // [buffer][W, X]: 128 KiB
  uint8_t scales[2][2][kScaleTileB];        // [period parity][W, X]: 16 KiB
};
static_assert(sizeof(DmaLds::codes) >= kStageBytes, "epilogue staging does not fit");

// One row's scales for stage s from its period's LDS copy, as two dwords whose bytes 0 and 2
// are the k blocks 8 s + 2 ks + lane / 32 of k steps ks = 0, 1 (first dword) and 2, 3
// (second): the matrix instruction picks the byte by its operand select.
__device__ __forceinline__ u32x2 lds_scales2(const uint8_t* row16, int s, int lane) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(row16 + (s & 1) * 8);
  const uint64_t v = (((uint64_t)w[1] << 32) | w[0]) >> (8 * (lane >> 5));
  return u32x2{(uint32_t)v, (uint32_t)(v >> 32)};
}

template <int KS>
__device__ __forceinline__ void mfma_one(v16f& acc, const u32x4& fa, const u32x4& fb,
                                         const u32x2& sa, const u32x2& sb) {
  const v8i A = {(int)fa[0], (int)fa[1], (int)fa[2], (int)fa[3], 0, 0, 0, 0};
  const v8i B = {(int)fb[0], (int)fb[1], (int)fb[2], (int)fb[3], 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, (KS & 1) * 2,
                                                        (int)sa[KS >> 1], (KS & 1) * 2,
                                                        (int)sb[KS >> 1]);
}

// Per-wave state of the fast-path tile loop.
struct DmaCtx {
  __amdgpu_buffer_rsrc_t rwc, rxc, rws, rxs, rnone;
  int i0, t0, rows_w, rows_x, ldb, nkb, wave, lane;
  uint32_t vw[2], vx[2];  // code offsets of this lane's rows for even / odd groups
  uint32_t sbw, sbx;      // scale offsets of this lane's rows (or kOob)
};

// Load number L (0..17) of the loads that fill a stage: 0..7 the weight rows' groups,
// 8..15 the tokens', 16 / 17 the weight / token scales of period q (when `scales`).
template <bool EDGE, int L>
__device__ __forceinline__ void dma_one(const DmaCtx& c, DmaLds& lds, int buf, int kb0,
                                        bool codes_on, int q, bool scales_on) {
  if (L < 16) {
    constexpr int op = L / 8, j = L % 8;
    const int lr = c.lane >> 3;
    uint32_t v = op == 0 ? c.vw[j & 1] : c.vx[j & 1];
    if (EDGE && (op == 0 ? c.i0 : c.t0) + c.wave * 64 + j * 8 + lr >= (op == 0 ? c.rows_w : c.rows_x))
      v = kOob;
    const __amdgpu_buffer_rsrc_t rs = codes_on ? (op == 0 ? c.rwc : c.rxc) : c.rnone;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_ptr_t)(lds.codes[buf][op] + (c.wave * 8 + j) * 1024), 16, (int)v,
        (int)(uint32_t)(j * 8 * c.ldb + kb0), 0, 0);
  } else {
    constexpr int op = L - 16;
    const __amdgpu_buffer_rsrc_t rs = scales_on ? (op == 0 ? c.rws : c.rxs) : c.rnone;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_ptr_t)(lds.scales[q & 1][op] + c.wave * 1024), 16,
        (int)(op == 0 ? c.sbw : c.sbx), (int)(uint32_t)(q * 16), 0, 0);
  }
}

// Fragment reads in the order the products use them: A0, B0..B3, A1..A3.
__device__ __forceinline__ void read_frags_ordered(const uint8_t* lw, const uint8_t* lx, int co,
                                                   u32x4 (&fa)[4], u32x4 (&fb)[4]) {
  fa[0] = *reinterpret_cast<const u32x4*>(lw + co);
#pragma unroll
  for (int n = 0; n < 4; n++) fb[n] = *reinterpret_cast<const u32x4*>(lx + n * 32 * kRowB + co);
#pragma unroll
  for (int m = 1; m < 4; m++) fa[m] = *reinterpret_cast<const u32x4*>(lw + m * 32 * kRowB + co);
}

// k step KS of a stage: its 16 products in the order (m, n), the next step's 8 fragment reads
// (KS < 3) and up to 8 of the next stage's NL loads (16: codes only; 18: codes and a scale
// period) placed between them, one instruction group at a time so that the matrix pipe never
// waits behind a batch of other work. A load that reads nothing still writes its (zero)
// bytes to LDS, so loads a stage does not need are not issued at all.
template <bool EDGE, int KS, int NL>
__device__ __forceinline__ void kstep(v16f (&acc)[4][4], const u32x4 (&fa)[4],
                                      const u32x4 (&fb)[4], u32x4 (&na)[4], u32x4 (&nb)[4],
                                      const uint8_t* lw, const uint8_t* lx, int sterm,
                                      const u32x2 (&sw)[4], const u32x2 (&sx)[4],
                                      const DmaCtx& c, DmaLds& lds, int nbuf, int kb0,
                                      bool codes_on, int q, bool scales_on) {
  const int co = ((2 * (KS + 1)) ^ sterm) * 16;
#pragma unroll
  for (int t = 0; t < 16; t++) {
    const int m = t / 4, n = t % 4;
    mfma_one<KS>(acc[m][n], fa[m], fb[n], sw[m], sx[n]);
    if (KS < 3 && t % 2 == 0) {  // next step's fragment t / 2 (A0, B0..B3, A1..A3)
      const int f = t / 2;
      if (f == 0) na[0] = *reinterpret_cast<const u32x4*>(lw + co);
      else if (f <= 4) nb[f - 1] = *reinterpret_cast<const u32x4*>(lx + (f - 1) * 32 * kRowB + co);
      else na[f - 4] = *reinterpret_cast<const u32x4*>(lw + (f - 4) * 32 * kRowB + co);
    }
    if (KS < 3 && t % 2 == 1 && KS * 8 + t / 2 < NL) {
      // loads KS * 8 + t / 2; the compiler folds the switch (everything is unrolled)
      switch (KS * 8 + t / 2) {
#define DQ_DMA_CASE(x) \
  case x: dma_one<EDGE, x>(c, lds, nbuf, kb0, codes_on, q, scales_on); break;
        DQ_DMA_CASE(0) DQ_DMA_CASE(1) DQ_DMA_CASE(2) DQ_DMA_CASE(3) DQ_DMA_CASE(4)
        DQ_DMA_CASE(5) DQ_DMA_CASE(6) DQ_DMA_CASE(7) DQ_DMA_CASE(8) DQ_DMA_CASE(9)
        DQ_DMA_CASE(10) DQ_DMA_CASE(11) DQ_DMA_CASE(12) DQ_DMA_CASE(13) DQ_DMA_CASE(14)
        DQ_DMA_CASE(15) DQ_DMA_CASE(16) DQ_DMA_CASE(17)
#undef DQ_DMA_CASE
        default: break;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool BF16, bool VECY, bool EDGE>
__device__ __forceinline__ void gemm_tile_dma(const GemmArgs& p, int i0, int t0, DmaLds& L) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const int ldb = p.K / 2, nkb = p.K / 32;
  const int nst = p.K / kBK;  // even: K % 512 == 0

  DmaCtx c;
  c.rwc = rsrc(p.wc, (uint32_t)p.out * (uint32_t)ldb);
  c.rxc = rsrc(p.xc, (uint32_t)p.tokens * (uint32_t)ldb);
  c.rws = rsrc(p.ws, (uint32_t)p.out * (uint32_t)nkb);
  c.rxs = rsrc(p.xs, (uint32_t)p.tokens * (uint32_t)nkb);
  // a descriptor that reads nothing: the loads of the stage after the last go there (the loop
  // body stays one basic block, so nothing can move across its barriers)
  c.rnone = rsrc(p.wc, 0u);
  c.i0 = i0;
  c.t0 = t0;
  c.rows_w = EDGE ? p.out : INT32_MAX;
  c.rows_x = EDGE ? p.tokens : INT32_MAX;
  c.ldb = ldb;
  c.nkb = nkb;
  c.wave = wave;
  c.lane = lane;
  {
    // lane j of a load writes LDS row 8 g + j / 8 at chunk position j % 8, which holds the
    // row's logical chunk (j % 8) ^ swizzle term (the term's bit 3 part flips with g)
    const int lr = lane >> 3;
    const uint32_t bw = (uint32_t)(i0 + wave * 64 + lr) * (uint32_t)ldb;
    const uint32_t bx = (uint32_t)(t0 + wave * 64 + lr) * (uint32_t)ldb;
    const uint32_t ce = (uint32_t)(((lane & 7) ^ lr) * 16), co = (uint32_t)(((lane & 7) ^ lr ^ 1) * 16);
    c.vw[0] = bw + ce;
    c.vw[1] = bw + co;
    c.vx[0] = bx + ce;
    c.vx[1] = bx + co;
    const int rw = i0 + wave * 64 + lane, rx = t0 + wave * 64 + lane;
    c.sbw = (EDGE && rw >= p.out) ? kOob : (uint32_t)rw * (uint32_t)nkb;
    c.sbx = (EDGE && rx >= p.tokens) ? kOob : (uint32_t)rx * (uint32_t)nkb;
  }

  v16f acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; m++)
#pragma unroll
    for (int n = 0; n < 4; n++) acc[m][n] = v16f{};

  const int rl = lane & 31;
  const int sterm = (rl & 7) ^ ((rl >> 3) & 1) ^ (lane >> 5);
  const int rw = (wi + rl) * kRowB, rx = (wt + rl) * kRowB;  // fragment row offsets
  const int sw_off = (wi + rl) * kScaleRowB, sx_off = (wt + rl) * kScaleRowB;

  // prologue: stage 0 into buffer 0 and the scales of period 0
  dma_one<EDGE, 0>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 1>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 2>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 3>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 4>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 5>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 6>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 7>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 8>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 9>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 10>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 11>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 12>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 13>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 14>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 15>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 16>(c, L, 0, 0, true, 0, true);
  dma_one<EDGE, 17>(c, L, 0, 0, true, 0, true);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  u32x2 sw[4], sx[4];
  u32x4 fa0[4], fb0[4], fa1[4], fb1[4];
  auto stage_scales = [&](int par, int half) {
    const uint8_t* bw = L.scales[par][0];
    const uint8_t* bx = L.scales[par][1];
#pragma unroll
    for (int m = 0; m < 4; m++) {
      sw[m] = lds_scales2(bw + sw_off + m * 32 * kScaleRowB, half, lane);
      sx[m] = lds_scales2(bx + sx_off + m * 32 * kScaleRowB, half, lane);
    }
  };
  // the stage in buffer `buf` (fa0 / fb0 holding its first k step), the next stage's loads
  // into buffer nbuf between its products
  auto stage = [&](auto nl, int buf, int nbuf, int kb0, bool codes_on, int q, bool scales_on) {
    constexpr int NL = decltype(nl)::value;
    const uint8_t* lw = L.codes[buf][0] + rw;
    const uint8_t* lx = L.codes[buf][1] + rx;
    __builtin_amdgcn_sched_barrier(0);
    kstep<EDGE, 0, NL>(acc, fa0, fb0, fa1, fb1, lw, lx, sterm, sw, sx, c, L, nbuf, kb0, codes_on, q, scales_on);
    kstep<EDGE, 1, NL>(acc, fa1, fb1, fa0, fb0, lw, lx, sterm, sw, sx, c, L, nbuf, kb0, codes_on, q, scales_on);
    kstep<EDGE, 2, NL>(acc, fa0, fb0, fa1, fb1, lw, lx, sterm, sw, sx, c, L, nbuf, kb0, codes_on, q, scales_on);
    kstep<EDGE, 3, NL>(acc, fa1, fb1, fa0, fb0, lw, lx, sterm, sw, sx, c, L, nbuf, kb0, codes_on, q, scales_on);
    // every wave's loads are in LDS after this
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  stage_scales(0, 0);
  read_frags_ordered(L.codes[0][0] + rw, L.codes[0][1] + rx, (0 ^ sterm) * 16, fa0, fb0);

  // two stages (one scale period) per trip: stage 2 q from buffer 0, stage 2 q + 1 from
  // buffer 1; the scales of period q + 1 load during stage 2 q
  for (int q = 0; q < nst / 2; q++) {
    const bool more = 2 * q + 2 < nst;
    const int par = q & 1;
    stage(std::integral_constant<int, 18>{}, 0, 1, (2 * q + 1) * kRowB, true, q + 1, more);
    stage_scales(par, 1);
    read_frags_ordered(L.codes[1][0] + rw, L.codes[1][1] + rx, (0 ^ sterm) * 16, fa0, fb0);
    stage(std::integral_constant<int, 16>{}, 1, 0, (2 * q + 2) * kRowB, more, q + 1, false);
    stage_scales(par ^ 1, 0);
    read_frags_ordered(L.codes[0][0] + rw, L.codes[0][1] + rx, (0 ^ sterm) * 16, fa0, fb0);
  }
  store_tile<BF16, VECY, EDGE>(p, acc, i0, t0, &L.codes[0][0][0]);
}

template <bool BF16, bool VECY>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx_dma(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) DmaLds lds;
  int i0, t0;
  tile_origin(p, i0, t0);
  if (i0 + kBM <= p.out && t0 + kBN <= p.tokens)
    gemm_tile_dma<BF16, VECY, false>(p, i0, t0, lds);
  else
    gemm_tile_dma<BF16, VECY, true>(p, i0, t0, lds);
}

// ------------------------------------------------------------ packed weights
// Weights are static, so they can be laid out once in the order the matrix instructions read
// them; the product then loads its weight fragments straight from global memory into
// registers (a wave instruction reads 1 KiB contiguously) and LDS serves only the token
// operand: with both operands' fragments read from LDS, the reads (512 bytes per product),
// not the matrix cores, set the pace.
//
// Within a stage the k values are assigned to the k steps so that a lane's share is
// contiguous: k step ks, lane half h, takes the stage's 32-value chunk 4 h + ks (the sum over
// the stage is the same; only the order of the fp32 additions differs). Packed codes: for
// each block of 32 rows rb, stage s and k step i, 1 KiB in which lane L holds 16 bytes: row
// 32 rb + L % 32, chunk 4 (L / 32) + i of stage s. Packed scales: for each rb and s, 256 bytes
// in which lane L holds the dword of k blocks 8 s + 4 (L / 32) .. + 3 of row 32 rb + L % 32
// (the matrix instruction selects byte ks). Rows past `out` up to the next multiple of 32
// hold zero codes and scale 2^0.
constexpr int kPackBlockB = 1024;                     // codes of (rb, s, i)
constexpr int kPackScaleB = 256;                      // scales of (rb, s)
constexpr int kXTileB = kBN * kRowB;                  // 32 KiB: the token operand's stage

__global__ void k_pack_codes(const uint8_t* __restrict__ wc, uint8_t* __restrict__ out_codes,
                             int out, int ldb, int nst, int64_t nchunks) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte output chunk
  if (g >= nchunks) return;
  const int L = (int)(g % 64);
  const int64_t blk = g / 64;  // (rb * nst + s) * 4 + i
  const int i = (int)(blk % 4);
  const int s = (int)((blk / 4) % nst);
  const int64_t rb = blk / 4 / nst;
  const int64_t row = rb * 32 + L % 32;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < out)
    v = *reinterpret_cast<const u32x4*>(wc + row * ldb + s * kRowB + (4 * (L / 32) + i) * 16);
  *reinterpret_cast<u32x4*>(out_codes + g * 16) = v;
}

__global__ void k_pack_scales(const uint8_t* __restrict__ ws, uint32_t* __restrict__ out_scales,
                              int out, int nkb, int nst, int64_t ndwords) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // output dword
  if (g >= ndwords) return;
  const int L = (int)(g % 64);
  const int s = (int)((g / 64) % nst);
  const int64_t rb = g / 64 / nst;
  const int64_t row = rb * 32 + L % 32;
  uint32_t v = 0x7F7F7F7Fu;
  if (row < out) v = *reinterpret_cast<const uint32_t*>(ws + row * nkb + 8 * s + 4 * (L / 32));
  out_scales[g] = v;
}

struct PackedLds {
  uint8_t x[3][kXTileB];                    // [stage % 3]: token stages, 96 KiB
  uint8_t xs[2][kScaleTileB];               // [period parity]: token scales, 8 KiB
};
// the epilogue stages fp32 results of 4 waves x 32 tokens in the same memory
static_assert(sizeof(PackedLds) >= kStageBytes, "epilogue staging does not fit");

// s_waitcnt operand: at most n vector-memory operations outstanding, the other counters free
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Per-wave state of the packed-weight tile loop.
struct PackedCtx {
  __amdgpu_buffer_rsrc_t rwc, rxc, rws, rxs, rnone;
  int t0, rows_x, ldb, nst, wave, lane;
  uint32_t va[4];     // packed-code offsets of this wave's row blocks m (+ lane), or kOob
  uint32_t vs[4];     // packed-scale offsets of the same, or kOob
  uint32_t vx[2];     // token-stage offsets of this lane's load rows, even / odd groups
  uint32_t sbx;       // token-scale offset of this lane's row in the scale loads
};

// Token stage load j (0..7) of this wave into stage buffer xb: LDS rows 8 (8 wave + j) .. + 7,
// lane j' writing row 8 g + j' / 8 at chunk position j' % 8, which holds the row's logical
// chunk (j' % 8) ^ swizzle term (the term's bit-3 part flips with the group's parity).
template <bool EDGE>
__device__ __forceinline__ void packed_load_x(const PackedCtx& c, uint8_t* xb, int j, int kb0,
                                              bool on) {
  uint32_t v = c.vx[j & 1];
  if (EDGE && c.t0 + c.wave * 64 + j * 8 + (c.lane >> 3) >= c.rows_x) v = kOob;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(on ? c.rxc : c.rnone,
                                           (lds_ptr_t)(xb + (c.wave * 8 + j) * 1024), 16, (int)v,
                                           (int)(uint32_t)(j * 8 * c.ldb + kb0), 0, 0);
}

// Token scale period q: rows 64 wave .. + 63, 16 bytes each.
__device__ __forceinline__ void packed_load_xs(const PackedCtx& c, PackedLds& lds, int q,
                                               bool on) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(on ? c.rxs : c.rnone,
                                           (lds_ptr_t)(lds.xs[q & 1] + c.wave * 1024), 16,
                                           (int)c.sbx, (int)(uint32_t)(q * 16), 0, 0);
}

template <int KS>
__device__ __forceinline__ void mfma_sel(v16f& acc, const u32x4& fa, const u32x4& fb, uint32_t sa,
                                         uint32_t sb) {
  const v8i A = {(int)fa[0], (int)fa[1], (int)fa[2], (int)fa[3], 0, 0, 0, 0};
  const v8i B = {(int)fb[0], (int)fb[1], (int)fb[2], (int)fb[3], 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, KS, (int)sa, KS, (int)sb);
}

// ------------------------------------------------- packed weights: the tile loop
// The four waves stack along the weight rows: wave w owns rows 64 w .. 64 w + 63 (two 32-row
// blocks m) and all 256 tokens (eight blocks n), 2 x 8 products per k step, so every weight
// fragment enters the CU once. Loads one stage issues (each lane): 8 weight fragments, 2
// weight scale dwords, 8 token loads, and on a period's first stage the token scales.
constexpr int kStageLoads = 8 + 2 + 8;

// k step KS of stage s: 16 products in the order (m, n). Between them: the next step's eight
// token fragments from LDS (at KS 3 the next stage's first fragments and its token scales,
// which the barrier before that step has made readable); after the last product of weight-row
// block m, that block's
// fragment of this step is reloaded with stage s + 2's, since its register is free from then on
// (and at KS 3 the block's scale dword as well); two of stage s + 2's eight token loads into
// its LDS buffer xb; and at KS 1 of a period's first stage (NX > 8) the next period's token
// scales. So every load has about two stages to land. Loads of stages past the last read
// nothing (a load to LDS that reads nothing still writes its zero bytes, into a buffer no
// longer read), and every stage issues the same number of them.
template <bool EDGE, int KS, int NX>
__device__ __forceinline__ void packed_kstep(v16f (&acc)[2][8], u32x4 (&fa)[2][4],
                                               const u32x4 (&fb)[8], u32x4 (&fb_next)[8],
                                               const uint8_t* lx, int xterm, uint32_t (&sw)[2],
                                               const uint32_t (&sx)[8], uint32_t (&sx_next)[8],
                                               const uint8_t* lx_next, const uint8_t* bx_next,
                                               const PackedCtx& c, PackedLds& lds, uint8_t* xb,
                                               int s2, bool on, int q, bool xs_on) {
#pragma unroll
  for (int t = 0; t < 16; t++) {
    const int m = t / 8, n = t % 8;
    mfma_sel<KS>(acc[m][n], fa[m][KS], fb[n], sw[m], sx[n]);
    if (t % 2 == 0 && KS < 3)
      fb_next[t / 2] =
          *reinterpret_cast<const u32x4*>(lx + (t / 2) * 32 * kRowB + (((KS + 1) ^ xterm) * 16));
    if (t % 2 == 0 && KS == 3)  // the next stage's first fragments
      fb_next[t / 2] =
          *reinterpret_cast<const u32x4*>(lx_next + (t / 2) * 32 * kRowB + ((0 ^ xterm) * 16));
    if (t % 2 == 1 && KS == 3)  // and its token scales
      sx_next[t / 2] = *reinterpret_cast<const uint32_t*>(bx_next + (t / 2) * 32 * kScaleRowB);
    if (n == 7) {
      fa[m][KS] = __builtin_amdgcn_raw_buffer_load_b128(
          on ? c.rwc : c.rnone, c.va[m], (uint32_t)((s2 * 4 + KS) * kPackBlockB), 0);
      if (KS == 3)
        sw[m] = __builtin_amdgcn_raw_buffer_load_b32(on ? c.rws : c.rnone, c.vs[m],
                                                     (uint32_t)(s2 * kPackScaleB), 0);
    }
    if (t == 1 || t == 9) packed_load_x<EDGE>(c, xb, KS * 2 + t / 8, s2 * kRowB, on);
    if (KS == 1 && t == 8 && NX > 8) packed_load_xs(c, lds, q, xs_on);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The packed kernel's epilogue: the wave's 64 x 256 results through LDS, 32 tokens at a time
// (rows of 64 fp32 channels, padded by 16 bytes); a lane reads back 4 channels of one row, 16
// lanes to a row, and each store instruction writes four rows of 128 (bf16) or 256 bytes.
constexpr int kRowStageRows = 64 * 4 + 16;
static_assert(4 * 32 * kRowStageRows <= (int)sizeof(PackedLds), "epilogue staging does not fit");

template <bool BF16, bool VECY, bool EDGE>
__device__ __forceinline__ void store_tile_rows(const GemmArgs& p, const v16f (&acc)[2][8], int i0,
                                             int t0, uint8_t* stage) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rl = lane & 31, h = lane >> 5;
  const int wi = wave * 64;
  uint8_t* region = stage + wave * 32 * kRowStageRows;
  const int ich = i0 + wi + (lane & 15) * 4;  // the 4 channels this lane stores
  f32x4 av = {1.0f, 1.0f, 1.0f, 1.0f};
  if (p.a) {
    if (!EDGE || ich + 3 < p.out) {
      av = *reinterpret_cast<const f32x4*>(p.a + ich);
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) av[e] = ich + e < p.out ? p.a[ich + e] : 1.0f;
    }
  }
  __syncthreads();  // every wave is done with the main loop's LDS

#pragma unroll
  for (int n = 0; n < 8; n++) {
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const f32x4 y = {acc[m][n][g * 4], acc[m][n][g * 4 + 1], acc[m][n][g * 4 + 2],
                         acc[m][n][g * 4 + 3]};
        *reinterpret_cast<f32x4*>(region + rl * kRowStageRows + (m * 32 + g * 8 + h * 4) * 4) = y;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int row = (lane >> 4) + 4 * r;
      f32x4 y = *reinterpret_cast<const f32x4*>(region + row * kRowStageRows + (lane & 15) * 16);
      const int t = t0 + n * 32 + row;
      if (EDGE && t >= p.tokens) continue;
#pragma unroll
      for (int e = 0; e < 4; e++) y[e] *= av[e];
      const bool vec = VECY && (!EDGE || ich + 3 < p.out);
      if (BF16) {
        __bf16* yp = static_cast<__bf16*>(p.y) + (int64_t)t * p.ldy + ich;
        const bf16x4 hv = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        if (vec) {
          __builtin_nontemporal_store(hv, reinterpret_cast<bf16x4*>(yp));
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (ich + e < p.out) yp[e] = hv[e];
        }
      } else {
        float* yp = static_cast<float*>(p.y) + (int64_t)t * p.ldy + ich;
        if (vec) {
          __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(yp));
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (ich + e < p.out) yp[e] = y[e];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next chunk's writes
  }
}

template <bool BF16, bool VECY, bool EDGE>
__device__ __forceinline__ void gemm_tile_packed(const GemmArgs& p, int i0, int t0,
                                                   PackedLds& L) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave * 64;
  const int ldb = p.K / 2, nkb = p.K / 32;
  const int nst = p.K / kBK;  // even: K % 512 == 0
  const int nrb = (p.out + 31) / 32;
  const int rl = lane & 31, h = lane >> 5;

  PackedCtx c;
  c.rwc = rsrc(p.wc, (uint32_t)nrb * (uint32_t)nst * 4u * kPackBlockB);
  c.rws = rsrc(p.ws, (uint32_t)nrb * (uint32_t)nst * kPackScaleB);
  c.rxc = rsrc(p.xc, (uint32_t)p.tokens * (uint32_t)ldb);
  c.rxs = rsrc(p.xs, (uint32_t)p.tokens * (uint32_t)nkb);
  c.rnone = rsrc(p.wc, 0u);  // reads nothing: the loads of stages after the last
  c.t0 = t0;
  c.rows_x = EDGE ? p.tokens : INT32_MAX;
  c.ldb = ldb;
  c.nst = nst;
  c.wave = wave;
  c.lane = lane;
#pragma unroll
  for (int m = 0; m < 2; m++) {
    const int rb = (i0 + wi) / 32 + m;
    const bool in = !EDGE || rb < nrb;
    c.va[m] = in ? (uint32_t)rb * (uint32_t)nst * 4u * kPackBlockB + (uint32_t)(lane * 16) : kOob;
    c.vs[m] = in ? (uint32_t)rb * (uint32_t)nst * kPackScaleB + (uint32_t)(lane * 4) : kOob;
  }
  {
    const int lr = lane >> 3;
    const uint32_t bx = (uint32_t)(t0 + wave * 64 + lr) * (uint32_t)ldb;
    c.vx[0] = bx + (uint32_t)(((lane & 7) ^ lr) * 16);
    c.vx[1] = bx + (uint32_t)(((lane & 7) ^ lr ^ 1) * 16);
    const int rx = t0 + wave * 64 + lane;
    c.sbx = (EDGE && rx >= p.tokens) ? kOob : (uint32_t)rx * (uint32_t)nkb;
  }

  v16f acc[2][8];
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int n = 0; n < 8; n++) acc[m][n] = v16f{};

  // token fragment reads: row 32 n + lane % 32 of the buffer, chunk 4 h + ks at its swizzled
  // position (4 h + ks) ^ term = ks ^ (term ^ 4 h)
  const int xterm = (rl & 7) ^ ((rl >> 3) & 1) ^ (4 * h);
  const int rx = rl * kRowB;
  const int sx_off = rl * kScaleRowB + 4 * h;

  u32x4 fa[2][2][4];  // [stage parity][m][ks]: the weight fragments of stages s and s + 1
  uint32_t sw[2][2];  // [stage parity][m]: their scale dwords
  u32x4 fb0[8], fb1[8];
  uint32_t sx[2][8];  // [stage parity][n]: token scale dwords of stages s and s + 1

  // prologue: stage 0 (weights and their scales into registers, tokens into buffer 0) and
  // token scale period 0, then stage 1; only the first two have to land before the loop starts
#pragma unroll
  for (int st = 0; st < 2; st++) {
#pragma unroll
    for (int m = 0; m < 2; m++) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        fa[st][m][i] = __builtin_amdgcn_raw_buffer_load_b128(
            c.rwc, c.va[m], (uint32_t)((st * 4 + i) * kPackBlockB), 0);
      sw[st][m] = __builtin_amdgcn_raw_buffer_load_b32(c.rws, c.vs[m],
                                                       (uint32_t)(st * kPackScaleB), 0);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) packed_load_x<EDGE>(c, L.x[st], j, st * kRowB, true);
    if (st == 0) packed_load_xs(c, L, 0, true);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStageLoads));  // stage 1's loads may be in flight
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // stage 0's token scales and first fragments
  {
    const uint8_t* bx = L.xs[0] + sx_off;
#pragma unroll
    for (int n = 0; n < 8; n++)
      sx[0][n] = *reinterpret_cast<const uint32_t*>(bx + n * 32 * kScaleRowB);
#pragma unroll
    for (int n = 0; n < 8; n++)
      fb0[n] = *reinterpret_cast<const u32x4*>(L.x[0] + rx + n * 32 * kRowB + ((0 ^ xterm) * 16));
  }
  // stage s: products from registers fa[P] / sw[P] / sx[P] and token buffer s % 3, while stage
  // s + 2 loads into the slots they free and buffer (s + 2) % 3. Before its last k step, every
  // load issued before the stage (those of stage s + 1) is complete in this wave and its LDS
  // reads are done, and after the barrier the same holds in every wave: the last step then
  // reads stage s + 1's first fragments and token scales (into fb0 and sx[P ^ 1]) under its own
  // products, so the matrix instructions run on across the stage boundary. The barrier also
  // orders every wave's reads of buffer (s - 1) % 3 before stage s + 1's loads into it.
  auto stage = [&](auto pc, auto nxc, int s, int q, bool xs_on) {
    constexpr int P = decltype(pc)::value, NX = decltype(nxc)::value;
    const uint8_t* lx = L.x[s % 3] + rx;
    uint8_t* xb = L.x[(s + 2) % 3];
    const int s2 = s + 2;
    const bool on = s2 < nst;
    // stage s + 1's scales: period (s + 1) / 2, half (s + 1) % 2 (past the last stage these
    // reads land in buffers that no load is writing, and their values go unused)
    const uint8_t* lxn = L.x[(s + 1) % 3] + rx;
    const uint8_t* bxn = L.xs[((s + 1) >> 1) & 1] + sx_off + (P ^ 1) * 8;
    __builtin_amdgcn_sched_barrier(0);
    packed_kstep<EDGE, 0, NX>(acc, fa[P], fb0, fb1, lx, xterm, sw[P], sx[P], sx[P ^ 1], lxn, bxn,
                              c, L, xb, s2, on, q, xs_on);
    packed_kstep<EDGE, 1, NX>(acc, fa[P], fb1, fb0, lx, xterm, sw[P], sx[P], sx[P ^ 1], lxn, bxn,
                              c, L, xb, s2, on, q, xs_on);
    packed_kstep<EDGE, 2, NX>(acc, fa[P], fb0, fb1, lx, xterm, sw[P], sx[P], sx[P ^ 1], lxn, bxn,
                              c, L, xb, s2, on, q, xs_on);
    // steps 0-2 issued 4 loads each (2 weight fragments, 2 token loads), and at a period's
    // first stage the token scales
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * 4 + (NX > 8 ? 1 : 0)) & ~(15 << 8));  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    packed_kstep<EDGE, 3, NX>(acc, fa[P], fb1, fb0, lx, xterm, sw[P], sx[P], sx[P ^ 1], lxn, bxn,
                              c, L, xb, s2, on, q, xs_on);
    __builtin_amdgcn_sched_barrier(0);
  };

  // two stages (one token scale period) per trip: stage 2 q (registers [0]) and stage 2 q + 1
  // (registers [1]); token scales of period q + 1 load during 2 q
  for (int q = 0; q < nst / 2; q++) {
    const bool more = 2 * q + 2 < nst;
    stage(std::integral_constant<int, 0>{}, std::integral_constant<int, 9>{}, 2 * q, q + 1, more);
    stage(std::integral_constant<int, 1>{}, std::integral_constant<int, 8>{}, 2 * q + 1, q + 1,
          false);
  }
  // the last stages' loads read nothing but still write their LDS buffers: drain them before
  // the epilogue reuses that memory
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  store_tile_rows<BF16, VECY, EDGE>(p, acc, i0, t0, reinterpret_cast<uint8_t*>(&L));
}

template <bool BF16, bool VECY>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx_packed(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) PackedLds lds;
  int i0, t0;
  tile_origin(p, i0, t0);
  if (i0 + kBM <= p.out && t0 + kBN <= p.tokens)
    gemm_tile_packed<BF16, VECY, false>(p, i0, t0, lds);
  else
    gemm_tile_packed<BF16, VECY, true>(p, i0, t0, lds);
}

template <bool BF16, bool VECY>
hipError_t launch_packed_t(const GemmArgs& p, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_mx_packed<BF16, VECY>), dim3(p.nti * p.ntt), dim3(kThreads), 0, s,
                     p);
  return hipGetLastError();
}

template <bool BF16, bool FULLK, bool VECY>
hipError_t launch_t(const GemmArgs& p, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_mx<BF16, FULLK, VECY>), dim3(p.nti * p.ntt), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, bool VECY>
hipError_t launch_dma_t(const GemmArgs& p, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_mx_dma<BF16, VECY>), dim3(p.nti * p.ntt), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch(const GemmArgs& p, bool bf16, bool fullk, bool dma, bool vecy,
                  hipStream_t s) {
  if (dma) {
    if (bf16) return vecy ? launch_dma_t<true, true>(p, s) : launch_dma_t<true, false>(p, s);
    return vecy ? launch_dma_t<false, true>(p, s) : launch_dma_t<false, false>(p, s);
  }
  if (bf16) {
    if (fullk) return vecy ? launch_t<true, true, true>(p, s) : launch_t<true, true, false>(p, s);
    return vecy ? launch_t<true, false, true>(p, s) : launch_t<true, false, false>(p, s);
  }
  if (fullk) return vecy ? launch_t<false, true, true>(p, s) : launch_t<false, true, false>(p, s);
  return vecy ? launch_t<false, false, true>(p, s) : launch_t<false, false, false>(p, s);
}

// The matrix cores' attainable rate: a stream of the scaled FP4 instruction on register
// operands only (eight independent accumulators per wave, nothing read or written in the loop),
// for comparison with the product's own rate at the clock the chip holds under that load. The
// sums are kept alive by a store that happens only if a lane's sum is exactly -1 (into a word
// of this module's own memory).
__device__ float g_mfma_sink[1];

__global__ __launch_bounds__(kThreads) void k_mfma_rate(int iters) {
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = v16f{};
  const int t = threadIdx.x;
  const v8i A = {t, t * 3, t * 5, t * 7, 0, 0, 0, 0};
  const v8i B = {t * 11, t * 13, t * 17, t * 19, 0, 0, 0, 0};
  const int unit = 0x7F7F7F7F;  // E8M0 2^0 in every byte
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 8; i++)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[i], 4, 4, 0, unit, 0, unit);
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int e = 0; e < 16; e++) sum += acc[i][e];
  if (sum == -1.0f) g_mfma_sink[0] = sum;
}

}  // namespace dqg

extern "C" {

dq_status dq_gemm_mx(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                     int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, const float* a,
                     int64_t out, dq_dtype yt, void* Y, hipStream_t stream) {
  using namespace dqg;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y) return DQ_ERR_ARG;
  if (tokens < 1 || out < 1 || K < 32 || K % 32 != 0) return DQ_ERR_ARG;
  if (yt != DQ_F32 && yt != DQ_BF16) return DQ_ERR_UNSUPPORTED;
  if (((uintptr_t)act_codes & 15u) || ((uintptr_t)w_codes & 15u) || ((uintptr_t)a & 15u))
    return DQ_ERR_ARG;
  // per launch, every buffer offset stays below 2^31: tokens (and output channels) are
  // split into chunks of whole tiles that keep it so
  const int64_t ldb = K / 2, nkb = K / 32;
  if (ldb * (kBM + 1) > (int64_t(1) << 30)) return DQ_ERR_ARG;  // K <= 2^22
  const int64_t lim = (int64_t(1) << 31) - ldb * (kBM + 1);
  const int64_t tchunk = std::max<int64_t>(kBN, (lim / ldb) / kBN * kBN);
  const int64_t ochunk = std::max<int64_t>(kBM, (lim / ldb) / kBM * kBM);
  const bool bf16 = yt == DQ_BF16;
  const size_t esz = bf16 ? 2 : 4;
  const bool fullk = K % kBK == 0 && ((uintptr_t)act_scales & 7u) == 0 &&
                     ((uintptr_t)w_scales & 7u) == 0;
  const bool vecy = out % 4 == 0 && ((uintptr_t)Y & (4 * esz - 1)) == 0;
  // the fast path loads 16 scale bytes per row at a time: K % 512 == 0, 16-byte aligned scales
  const bool dma = K % (2 * kBK) == 0 && ((uintptr_t)act_scales & 15u) == 0 &&
                   ((uintptr_t)w_scales & 15u) == 0;
  for (int64_t tb = 0; tb < tokens; tb += tchunk) {
    for (int64_t ob = 0; ob < out; ob += ochunk) {
      GemmArgs p{};
      p.xc = act_codes + tb * ldb;
      p.xs = act_scales + tb * nkb;
      p.wc = w_codes + ob * ldb;
      p.ws = w_scales + ob * nkb;
      p.a = a ? a + ob : nullptr;
      p.y = static_cast<char*>(Y) + (size_t)(tb * out + ob) * esz;
      p.tokens = (int)std::min(tchunk, tokens - tb);
      p.out = (int)std::min(ochunk, out - ob);
      p.K = (int)K;
      p.ldy = out;
      p.nti = (p.out + kBM - 1) / kBM;
      p.ntt = (p.tokens + kBN - 1) / kBN;
      if (launch(p, bf16, fullk, dma, vecy, stream) != hipSuccess) return DQ_ERR_HIP;
    }
  }
  return DQ_OK;
}

dq_status dq_gemm_pack_bytes(int64_t out, int64_t K, size_t* codes_bytes, size_t* scales_bytes) {
  using namespace dqg;
  if (!codes_bytes || !scales_bytes || out < 1 || K < 512 || K % 512 != 0 || K > (1 << 22))
    return DQ_ERR_ARG;
  const int64_t nrb = (out + 31) / 32, nst = K / kBK;
  *codes_bytes = (size_t)(nrb * nst * 4 * kPackBlockB);
  *scales_bytes = (size_t)(nrb * nst * kPackScaleB);
  return DQ_OK;
}

dq_status dq_gemm_pack_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t out,
                               int64_t K, uint8_t* packed_codes, uint8_t* packed_scales,
                               hipStream_t stream) {
  using namespace dqg;
  size_t cb = 0, sb = 0;
  if (dq_gemm_pack_bytes(out, K, &cb, &sb) != DQ_OK) return DQ_ERR_ARG;
  if (!w_codes || !w_scales || !packed_codes || !packed_scales) return DQ_ERR_ARG;
  if (((uintptr_t)w_codes & 15u) || ((uintptr_t)w_scales & 3u) || ((uintptr_t)packed_codes & 15u) ||
      ((uintptr_t)packed_scales & 3u))
    return DQ_ERR_ARG;
  const int nst = (int)(K / kBK);
  const int64_t nchunks = (int64_t)(cb / 16), ndw = (int64_t)(sb / 4);
  hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream,
                     w_codes, packed_codes, (int)out, (int)(K / 2), nst, nchunks);
  if (hipGetLastError() != hipSuccess) return DQ_ERR_HIP;
  hipLaunchKernelGGL(k_pack_scales, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, stream,
                     w_scales, reinterpret_cast<uint32_t*>(packed_scales), (int)out, (int)(K / 32),
                     nst, ndw);
  if (hipGetLastError() != hipSuccess) return DQ_ERR_HIP;
  return DQ_OK;
}

dq_status dq_gemm_mx_packed(const uint8_t* act_codes, const uint8_t* act_scales, int64_t tokens,
                            int64_t K, const uint8_t* packed_codes, const uint8_t* packed_scales,
                            const float* a, int64_t out, dq_dtype yt, void* Y,
                            hipStream_t stream) {
  using namespace dqg;
  if (!act_codes || !act_scales || !packed_codes || !packed_scales || !Y) return DQ_ERR_ARG;
  if (tokens < 1 || out < 1 || K < 512 || K % 512 != 0 || K > (1 << 22)) return DQ_ERR_ARG;
  if (yt != DQ_F32 && yt != DQ_BF16) return DQ_ERR_UNSUPPORTED;
  if (((uintptr_t)act_codes & 15u) || ((uintptr_t)act_scales & 15u) ||
      ((uintptr_t)packed_codes & 15u) || ((uintptr_t)packed_scales & 3u) ||
      ((uintptr_t)a & 15u))
    return DQ_ERR_ARG;
  // per launch, every buffer offset stays below 2^31: tokens and output channels are split
  // into chunks of whole tiles that keep it so (a chunk of channels is a whole number of
  // 32-row packed blocks)
  const int64_t ldb = K / 2, nkb = K / 32, nst = K / kBK;
  const int64_t lim = (int64_t(1) << 31) - ldb * (kBM + 1);
  const int64_t tchunk = std::max<int64_t>(kBN, (lim / ldb) / kBN * kBN);
  const int64_t ochunk = std::max<int64_t>(kBM, (lim / ldb) / kBM * kBM);
  const bool bf16 = yt == DQ_BF16;
  const size_t esz = bf16 ? 2 : 4;
  const bool vecy = out % 4 == 0 && ((uintptr_t)Y & (4 * esz - 1)) == 0;
  for (int64_t tb = 0; tb < tokens; tb += tchunk) {
    for (int64_t ob = 0; ob < out; ob += ochunk) {
      GemmArgs p{};
      p.xc = act_codes + tb * ldb;
      p.xs = act_scales + tb * nkb;
      p.wc = packed_codes + (ob / 32) * nst * 4 * kPackBlockB;
      p.ws = packed_scales + (ob / 32) * nst * kPackScaleB;
      p.a = a ? a + ob : nullptr;
      p.y = static_cast<char*>(Y) + (size_t)(tb * out + ob) * esz;
      p.tokens = (int)std::min(tchunk, tokens - tb);
      p.out = (int)std::min(ochunk, out - ob);
      p.K = (int)K;
      p.ldy = out;
      p.nti = (p.out + kBM - 1) / kBM;
      p.ntt = (p.tokens + kBN - 1) / kBN;
      const hipError_t e = bf16 ? (vecy ? launch_packed_t<true, true>(p, stream)
                                        : launch_packed_t<true, false>(p, stream))
                                : (vecy ? launch_packed_t<false, true>(p, stream)
                                        : launch_packed_t<false, false>(p, stream));
      if (e != hipSuccess) return DQ_ERR_HIP;
    }
  }
  return DQ_OK;
}

dq_status dq_bench_fp4_mfma_rate(int iters, hipStream_t stream, double* tflops) {
  if (iters < 1 || iters > (1 << 20) || !tflops) return DQ_ERR_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return DQ_ERR_HIP;
  const dim3 grid((unsigned)(4 * cus));  // four 4-wave workgroups per CU
  using namespace dqg;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  dq_status st = DQ_ERR_HIP;
  float ms = 0.0f;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    hipLaunchKernelGGL(k_mfma_rate, grid, dim3(kThreads), 0, stream, iters);  // warm-up
    hipEventRecord(e0, stream);
    hipLaunchKernelGGL(k_mfma_rate, grid, dim3(kThreads), 0, stream, iters);
    hipEventRecord(e1, stream);
    if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.0f) {
      const double flops = 2.0 * 32 * 32 * 64 * 8.0 * iters * (double)grid.x * (kThreads / 64);
      *tflops = flops / (ms * 1e-3) / 1e12;
      st = DQ_OK;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return st;
}

}  // extern "C"
