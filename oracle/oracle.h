/*
 * oracle.h -- plain, slow CPU oracle for the NVFP4 linear-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this code; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no source, table or helper with the GPU implementation.
 *
 * What it computes (sources, by page title and section):
 *  - NVFP4 element format: E2M1 codes in 16-element micro-blocks, one E4M3
 *    scale per block ("Nemotron 3 Super" summary at gkm0120.cn/p/20617,
 *    pretraining-recipe table, training-precision row).
 *  - 1D block scaling for activations and gradients, 2D block scaling for
 *    weights, Random Hadamard Transform on the wgrad inputs, stochastic
 *    rounding on gradients (same page, Infra table, quantization-scheme row;
 *    "Nemotron 3 Ultra" report, section 2.2 "NVFP4 pretraining").
 *  - Philox counter-based random bits for stochastic rounding, with five
 *    rounds as the accuracy/overhead balance point ("Nemotron 3 Super"
 *    report summary at papers.lianghsun.dev/paper/2604.12374v1, section 4.3).
 *  - fprop/dgrad/wgrad GEMMs on the quantized operands (Super summary, Infra
 *    table, training-precision row; Ultra report section 2.2).
 * Where the pages leave a choice open (16x16 2D blocks, 16-point RHT, the
 * per-tensor fp32 scale, the Philox key/counter layout, tie rules) the
 * reading used is stated at the function that implements it.
 *
 * Parity status: every function here is pinned by a CPU test against
 * something other than itself (value tables from the pages, library casts,
 * rocRAND's Philox, scipy's Hadamard matrix, brute force, closed forms and
 * invariants).  None is "parity unpinned".
 *
 * Arithmetic: every float operation is IEEE binary32 round-to-nearest-even
 * (written RN32 below), no FMA contraction (built with -ffp-contract=off),
 * subnormals kept.  The GEMM reference is fp64.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_ROW = 0, ORACLE_COL = 1, ORACLE_2D = 2 };
enum { ORACLE_RNE = 0, ORACLE_SR = 1 };

/* ---- element formats ---------------------------------------------------- */
float   oracle_e2m1_decode(uint8_t code);          /* 4-bit code -> value   */
uint8_t oracle_e2m1_encode_rne(float y);           /* nearest, ties to even */
uint8_t oracle_e2m1_encode_sr(float y, uint32_t u16);
float   oracle_e4m3_decode(uint8_t e);             /* byte -> value (NaN for 0x7F/0xFF) */
uint8_t oracle_e4m3_encode_rne_sat(float s);       /* s >= 0 finite -> byte */
/* Element-wise over arrays of n values (for exhaustive sweeps). */
void oracle_e2m1_encode_rne_n(const float* y, int64_t n, uint8_t* out);
void oracle_e4m3_encode_rne_sat_n(const float* s, int64_t n, uint8_t* out);

/* ---- Philox4x32 ---------------------------------------------------------- */
void oracle_philox4x32(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t rounds, uint32_t out[4]);
/* 16-bit random slot for element e (0..15) of block b. */
uint32_t oracle_sr_bits(uint64_t seed, uint64_t offset, uint32_t rounds,
                        uint64_t block, int e);

/* ---- 16-point randomized Hadamard transform ------------------------------ */
void oracle_rht16_vec(float v[16], uint32_t sign_mask);

/* ---- per-tensor scales --------------------------------------------------- */
void oracle_global_scales(float amax, float* S, float* k, float* g);

/* ---- whole-tensor operations --------------------------------------------
 * x: bf16 (x_is_bf16 = 1, raw uint16 bits) or fp32, row-major
 *    [batch][rows][cols].
 * block: ORACLE_ROW (1x16 along cols), ORACLE_COL (16x1 along rows),
 *        ORACLE_2D (16x16).
 * rht_mask: -1 for none, else a 16-bit sign mask (ROW/COL only).
 * amax_in: NULL to compute the per-slice amax, else [batch] given values.
 * Outputs: codes [batch][rows][cols/2] (low nibble = even column),
 *          scales ROW [rows][cols/16], COL [rows/16][cols],
 *          2D [rows/16][cols/16] (each per slice),
 *          amax_out [batch], global_dec [batch].
 * Returns 0, or -2 on a shape that the blocks do not tile, -5 on an
 * unsupported combination (SR or RHT with 2D blocks).
 */
int oracle_quantize(const void* x, int x_is_bf16, int64_t batch, int64_t rows,
                    int64_t cols, int block, int rounding, uint64_t seed,
                    uint64_t offset, uint32_t rounds, int32_t rht_mask,
                    const float* amax_in, uint8_t* codes, uint8_t* scales,
                    float* amax_out, float* global_dec);

/* Same, restricted to rows [row_begin, row_end) of every slice (multiples
 * of 16 for COL and 2D): only the codes and scales of blocks inside the
 * window are written, all others are left untouched.  Block ids stay those of
 * the whole slice, so stochastic rounding matches the full call.  A window
 * other than the whole slice requires amax_in. */
int oracle_quantize_rows(const void* x, int x_is_bf16, int64_t batch,
                         int64_t rows, int64_t cols, int block, int rounding,
                         uint64_t seed, uint64_t offset, uint32_t rounds,
                         int32_t rht_mask, const float* amax_in,
                         int64_t row_begin, int64_t row_end, uint8_t* codes,
                         uint8_t* scales, float* amax_out, float* global_dec);

/* Per-slice amax of |v| (after the RHT when rht_mask >= 0). */
int oracle_amax(const void* x, int x_is_bf16, int64_t batch, int64_t rows,
                int64_t cols, int block, int32_t rht_mask, float* amax_out);

/* Standalone transform: y[r][c] fp32 = RHT of x along the block axis. */
int oracle_rht16(const void* x, int x_is_bf16, int64_t rows, int64_t cols,
                 int block, uint32_t sign_mask, float* y);

/* x_hat = RN32(RN32(val(code) * val(scale)) * g), fp32 [rows][cols]. */
int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, float g,
                      int64_t rows, int64_t cols, int block, float* y);

/* Unscaled-by-g decoded element val(code)*val(scale) of a stored operand. */
double oracle_operand_value(const uint8_t* codes, const uint8_t* scales,
                            int64_t rows, int64_t cols, int block,
                            int64_t r, int64_t c);

/* GEMM reference in fp64.  C[M][N] = op(A) op(B) with row-major semantics:
 *   opA 'N': A stored [M][K]; 'T': A stored [K][M].
 *   opB 'T': B stored [N][K]; 'N': B stored [K][N].
 * For each requested (i, j):
 *   R = gA*gB*sum_k a(i,k) b(k,j);  D = gA*gB*sum_k |a(i,k) b(k,j)|.
 * a_block / b_block give the block kind each operand was quantized with.
 * Returns 0, or -2/-4 on a shape or layout mismatch.
 */
int oracle_gemm_entries(char opA, char opB, int64_t M, int64_t N, int64_t K,
                        const uint8_t* a_codes, const uint8_t* a_scales,
                        int a_block, float gA,
                        const uint8_t* b_codes, const uint8_t* b_scales,
                        int b_block, float gB,
                        const int64_t* ii, const int64_t* jj, int64_t n,
                        double* R, double* D);

/* Threads of the OpenMP loops above (the fp64 GEMM references and the
 * array encoders): n > 0 sets them for later calls from this host thread,
 * n <= 0 leaves them.  Returns the count now in force.  Used to time the
 * reference on one core and on all of them; results do not depend on it. */
int oracle_set_threads(int n);

/* Whole-matrix fp64 reference (R and D both [M][N]); threads over rows. */
int oracle_gemm_full(char opA, char opB, int64_t M, int64_t N, int64_t K,
                     const uint8_t* a_codes, const uint8_t* a_scales,
                     int a_block, float gA,
                     const uint8_t* b_codes, const uint8_t* b_scales,
                     int b_block, float gB, double* R, double* D);

/* PTQ weight quantization with MSE-calibrated block scales (Super report
 * summary, section 4.2: NVFP4 PTQ picks each weight block's scale by
 * minimizing the weight's MSE instead of taking the max-based one).
 * ROW blocks (1x16 along cols), RNE elements, per-tensor S, k, g from amax
 * (computed, or amax_in when non-NULL) exactly as the max-based quantizer.
 * Each block's E4M3 scale code is the one, of all 127 finite codes
 * 0 .. 126, whose encoding of the block has the smallest squared error.  A
 * code e encodes the block as the max-based quantizer would with scale e
 * (r = RN32(S / val(e)), y = RN32(x r), RNE) and its error is the fp64 sum,
 * in index order, of (x_i - xh_i)^2 with xh_i = RN32(RN32(val(code_i)
 * val(e)) g) the dequantized value.  Ties: the max-based code e0 =
 * E4M3(RN32(a k)) if it reaches the minimum, else the smallest code that
 * does.
 * Outputs as oracle_quantize (codes, scales [rows x cols/16], amax, g). */
int oracle_quantize_mse(const void* x, int x_is_bf16, int64_t rows, int64_t cols,
                        const float* amax_in, uint8_t* codes, uint8_t* scales,
                        float* amax_out, float* g_out);

/* fp32 -> fp16 with stochastic rounding, the SSM-state cache recipe (Super
 * report summary, section 4.3: FP16 with Philox<5> stochastic rounding, no
 * block scales).  lo = the largest finite fp16 <= |x| (found in a table of
 * every finite fp16 value), hi = the next one; the magnitude rounds up to hi
 * iff u < 65536 * (|x| - lo) / (hi - lo), evaluated in fp64 (exact).
 * Readings: |x| >= 65504 (infinities included) saturates to 65504; NaN gives
 * 0x7E00 with x's sign; the sign bit is kept (so -0 stays -0).
 * Element i draws the 16-bit slot i % 8 of Philox call i / 8 (the same
 * word/half order as the block quantizers).  Returns the fp16 bit pattern. */
uint16_t oracle_sr_fp16_one(float x, uint32_t u16);
void oracle_sr_fp16(const float* x, int64_t n, uint64_t seed, uint64_t offset,
                    uint32_t rounds, uint16_t* y);

#ifdef __cplusplus
}
#endif
#endif
