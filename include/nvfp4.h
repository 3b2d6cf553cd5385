/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 quantizers and GEMMs for AMD MI355X
 * (gfx950).
 *
 * What the library computes comes from the pages on the Nemotron 3 NVFP4
 * pretraining recipe:
 *  - NVFP4 = E2M1 elements in 16-element micro-blocks, each block with one
 *    E4M3 scale ("Nemotron 3 Super" summary, gkm0120.cn/p/20617,
 *    pretraining-recipe table, training-precision row);
 *  - fprop, dgrad and wgrad GEMMs all run in NVFP4; weights use 2D block
 *    scaling, activations and gradients 1D block scaling; the wgrad inputs
 *    get a Random Hadamard Transform and gradients stochastic rounding (same
 *    page, Infra table; "Nemotron 3 Ultra" report, section 2.2);
 *  - stochastic rounding draws Philox random bits, five rounds balancing
 *    quality and cost ("Nemotron 3 Super" report summary at
 *    papers.lianghsun.dev/paper/2604.12374v1, section 4.3);
 *  - routed-expert GEMMs run in NVFP4 (same summary, section 2.2).
 * The pages leave the 2D block size, the transform size, the per-tensor
 * scale, the random-bit layout and all tie rules open; the readings used are
 * stated at each call below and are the same as the CPU oracle's.
 *
 * Conventions for every call:
 *  - Every pointer argument except the nvfp4_operand / nvfp4_philox structs
 *    themselves is DEVICE memory owned by the caller.  The library allocates
 *    nothing and never synchronizes the device (except in the debug mode of
 *    nvfp4_set_debug_checks).  Its only state is two process-wide settings
 *    (nvfp4_set_single_pass_wait, nvfp4_set_debug_checks), the host counters
 *    that hand out its scratch slots, and that scratch itself: static device
 *    arrays (about 1.8 MB per device) through which the quantizers' workgroups
 *    combine a tensor's maximum; each call leaves them ready for the next.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and the call returns; outputs are valid in stream
 *    order.
 *  - Return value: NVFP4_OK (0) or a negative nvfp4_status.  Argument errors
 *    are reported before anything is launched; NVFP4_ERR_DEVICE means a HIP
 *    launch failed.  No C++ exception crosses this interface.
 *  - Inputs must be finite.  Results are bit-identical for identical
 *    arguments (no atomics whose order could change a value).
 *  - Matrices are row-major: "[R x C]" means C is the contiguous dimension.
 *
 * Encoding reading (identical in the CPU oracle):
 *   A   = max |v| over the tensor (over each slice when batched), v being the
 *         input in fp32 after the optional Hadamard transform;
 *   S   = RN32(2688 / A)   (1 if A == 0, FLT_MAX if it overflows),
 *   k   = RN32(S / 6),  g = RN32(A / 2688)        (2688 = 6 * 448);
 *   per 16-element block: a = max |v|, scale byte e = E4M3(RN32(a * k)) with
 *   round-to-nearest-even and saturation at 448, d = value(e),
 *   r = RN32(S / d) (0 when d == 0, FLT_MAX on overflow);
 *   per element: y = RN32(v * r), rounded onto the E2M1 grid
 *   {0, .5, 1, 1.5, 2, 3, 4, 6} (nearest-even, or stochastic), saturating at
 *   6; code = sign << 3 | magnitude index (-0 keeps its sign: code 0x8).
 *   Dequantized value = RN32(RN32(val(code) * d) * g).
 * Storage: codes two per byte along the contiguous dimension, even element in
 * the low nibble ([R x C/2] bytes).  Scale bytes: ROW blocks [R x C/16], COL
 * blocks [R/16 x C], 2D blocks [R/16 x C/16].
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_ERR_NULL (-1)        /* a required pointer is NULL            */
#define NVFP4_ERR_SHAPE (-2)       /* sizes the blocks or tiles cannot take */
#define NVFP4_ERR_ALIGN (-3)       /* a pointer misses its alignment        */
#define NVFP4_ERR_LAYOUT (-4)      /* op letters / block kind do not fit    */
#define NVFP4_ERR_UNSUPPORTED (-5) /* a valid-looking but unsupported mode  */
#define NVFP4_ERR_DEVICE (-6)      /* a HIP launch failed                   */
#define NVFP4_ERR_NONFINITE (-7)   /* debug checks only: an input holds an
                                      infinity or a NaN                       */

/* Element types of unquantized tensors. */
#define NVFP4_BF16 0
#define NVFP4_FP32 1
/* GEMM output only: fp32 C that the product is added to, C = RN32(C +
 * result) (gradient accumulation into an fp32 main-grad buffer; Ultra report
 * section 2.7 traces a divergence to local gradient accumulation in bf16
 * instead of fp32). */
#define NVFP4_FP32_ACCUMULATE 2

/* Rounding of elements onto the E2M1 grid. */
#define NVFP4_RNE 0 /* nearest, ties to the even code (activations, weights) */
#define NVFP4_SR 1  /* stochastic rounding (gradients)                       */

/* Block kinds (16 elements along the contraction dimension K). */
#define NVFP4_BLOCK_ROW 0 /* 1x16 along the contiguous dimension       */
#define NVFP4_BLOCK_COL 1 /* 16x1 along the row dimension              */
#define NVFP4_BLOCK_2D 2  /* 16x16                                     */

/* Philox4x32 stream for stochastic rounding (host struct, read at the call).
 * Reading of the pages' "Philox" with five rounds: key = (lo32(seed),
 * hi32(seed)); block id b makes two calls j = 0, 1 with counter
 * (lo32(2b+j), hi32(2b+j), lo32(offset), hi32(offset)); element e of the
 * block (0..15 along the block axis) uses call e>>3, output word (e>>1)&3,
 * low 16 bits for even e, high for odd; it rounds up iff
 * u16 < 65536 * (m - lo) / (hi - lo) with lo <= m < hi neighbouring grid
 * values.  Block ids: ROW b = r*(C/16) + c/16; COL b = c*(R/16) + r/16. */
typedef struct {
  uint64_t seed;
  uint64_t offset;
  uint32_t rounds; /* 1..16; 5 is the recipe's value, 10 matches cuRAND/rocRAND */
  uint32_t reserved;
} nvfp4_philox;

/* A quantized operand: device pointers to its codes, its scale bytes and its
 * fp32 decode scale g, with the stored shape [rows x cols] and block kind.
 * As a GEMM operand (kernels address it with 32-bit offsets): cols < 2^24
 * when K is its contiguous dimension (any number of rows: each tile's loads
 * cover at most 256 rows), rows * cols < 2^32 when K is its row dimension
 * (else NVFP4_ERR_SHAPE). */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global_dec;
  int64_t rows;
  int64_t cols;
  int32_t block; /* NVFP4_BLOCK_* */
  int32_t reserved;
} nvfp4_operand;

/* Version of this ABI (NVFP4_ABI_VERSION). */
int32_t nvfp4_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* nvfp4_status_string(int32_t status);

/*
 * 1D block quantization of activations and gradients (Super summary, Infra
 * table; Ultra report section 2.2), with the optional 16-point Random
 * Hadamard Transform of the wgrad inputs and stochastic rounding of
 * gradients.
 *   x        [rows x cols] input, NVFP4_BF16 or NVFP4_FP32 (x_dtype).
 *   axis     NVFP4_BLOCK_ROW (blocks along cols) or NVFP4_BLOCK_COL (blocks
 *            along rows, used for the token dimension of wgrad inputs).
 *   rounding NVFP4_RNE, or NVFP4_SR with `rng` (host struct) non-NULL.
 *   rht_sign_mask  -1 for no transform, else a 16-bit mask: each block v is
 *            replaced by (1/4) H16 diag(s) v, H16 the Sylvester Hadamard
 *            matrix, s_i = -1 where bit i is set; evaluated as butterflies of
 *            stride 1, 2, 4, 8 (RN32 sums/differences) then an exact * 1/4.
 *            Both wgrad operands must use the same mask.
 *   amax     device float: read when amax_is_input != 0, else written with
 *            the tensor amax (after the transform).
 *   codes    [rows x cols/2] bytes out;  scales ROW [rows x cols/16] or COL
 *            [rows/16 x cols] bytes out;  global_dec: device float out (g).
 * Shapes: cols % 32 == 0; COL also rows % 16 == 0; rows == 0 is a no-op.
 * Alignment: x, codes 16 bytes; scales 4 bytes.
 */
int32_t nvfp4_quantize_1d(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                          int32_t axis, int32_t rounding, const nvfp4_philox* rng,
                          int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                          uint8_t* codes, uint8_t* scales, float* global_dec, void* stream);

/*
 * Both 1D quantizations of one gradient tensor (dY), with both tensor
 * maxima taken in one read of it (Super summary, Infra table; Ultra report
 * section 2.2: dgrad and wgrad
 * both consume dY in NVFP4, stochastically rounded, the wgrad operand after
 * the Random Hadamard Transform), plus the count of zero-valued codes, the
 * health signal of the Super report summary, section 2.2 (NVFP4
 * pretraining: the share of zero-valued gradient elements).
 * Results are bit-identical to the two calls
 *   nvfp4_quantize_1d(x, ROW, SR, rng_row, -1,            amax[0], ...row outputs)
 *   nvfp4_quantize_1d(x, COL, SR, rng_col, rht_sign_mask, amax[1], ...col outputs)
 * with the same amax_is_input, so dgrad takes the ROW operand (blocks along
 * the output features) and wgrad the COL one (blocks along the tokens).
 *   x          [rows x cols], NVFP4_BF16 or NVFP4_FP32.
 *   rng_row, rng_col  host structs, both required (two independent streams).
 *   rht_sign_mask     -1 or a 16-bit mask, for the COL output only.
 *   amax       device float[2]: ROW tensor amax, COL tensor amax (after the
 *              transform); read when amax_is_input != 0, else written.
 *   row_codes [rows x cols/2], row_scales [rows x cols/16], row_global_dec;
 *   col_codes [rows x cols/2], col_scales [rows/16 x cols], col_global_dec.
 *   zero_codes NULL, or device uint64[2] overwritten with the number of
 *              codes of magnitude zero (0x0 or 0x8) in the ROW and in the
 *              COL output.
 * The two encodes then run as the two 1D quantizers' encode kernels (both are
 * ALU-bound: an encode reading x once for both outputs was slower), which
 * count the zero codes as they write them.
 * Shapes: rows % 16 == 0, cols % 32 == 0; rows == 0 or cols == 0 is a no-op
 * (nothing is written, zero_codes included).  Alignment: x and codes 16
 * bytes, scales and amax 4, zero_codes 8.
 */
int32_t nvfp4_quantize_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                            const nvfp4_philox* rng_row, const nvfp4_philox* rng_col,
                            int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                            uint8_t* row_codes, uint8_t* row_scales, float* row_global_dec,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_global_dec,
                            uint64_t* zero_codes, void* stream);

/*
 * Quantization fused with the MoE token dispatch (Super report summary,
 * section 2.1: LatentMoE routes each token to 22 of 512 experts; section 2.2:
 * the routed-expert GEMMs run in NVFP4).  The tensor quantized is
 *   G [rows x cols], row r of G = row row_index[r] of x [src_rows x cols],
 * and an index outside [0, src_rows) makes row r a row of zeros (the padding
 * that keeps each expert's rows a multiple of 16 for COL blocks).  The result
 * (codes, scales, amax, g, and for the dual form the zero counts) is bit for
 * bit that of nvfp4_quantize_1d / nvfp4_quantize_dual on G materialized, so
 * the gathered bf16/fp32 copy of the activations is never written.
 *   row_index  device int64 [rows], 8-byte aligned, read only.
 *   src_rows   >= 1; x is [src_rows x cols] as in the plain call.
 * Other arguments, shapes and errors as the plain calls, plus: src_rows < 1
 * or rows * cols / 8 >= 2^32 -> NVFP4_ERR_SHAPE; a NULL row_index with a
 * non-empty G -> NVFP4_ERR_NULL.
 */
int32_t nvfp4_quantize_1d_gather(const void* x, int32_t x_dtype, int64_t src_rows,
                                 const int64_t* row_index, int64_t rows, int64_t cols,
                                 int32_t axis, int32_t rounding, const nvfp4_philox* rng,
                                 int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                                 uint8_t* codes, uint8_t* scales, float* global_dec,
                                 void* stream);
int32_t nvfp4_quantize_dual_gather(const void* x, int32_t x_dtype, int64_t src_rows,
                                   const int64_t* row_index, int64_t rows, int64_t cols,
                                   const nvfp4_philox* rng_row, const nvfp4_philox* rng_col,
                                   int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                                   uint8_t* row_codes, uint8_t* row_scales,
                                   float* row_global_dec, uint8_t* col_codes,
                                   uint8_t* col_scales, float* col_global_dec,
                                   uint64_t* zero_codes, void* stream);

/*
 * Post-training weight quantization with MSE-calibrated block scales (Super
 * report summary, section 4.2, NVFP4 PTQ: each weight block's scale is chosen
 * to minimize the weight's MSE rather than from the block max; activations
 * keep the dynamic max-based nvfp4_quantize_1d).  ROW blocks (1x16 along
 * cols, i.e. along K of a weight stored [N x K]), RNE elements, per-tensor
 * scales as nvfp4_quantize_1d.  Each block's E4M3 scale is the one, of all
 * 127 finite codes, whose encoding of the block (as nvfp4_quantize_1d would
 * encode it with that scale) has the smallest error, the fp64 sum in index
 * order of (x - dequantized x)^2; on a tie the max-based code is kept if it
 * is a minimum, else the smallest code wins.  The search runs on the
 * device, offline (once per weight).
 * The result is a ROW operand for nvfp4_gemm (e.g. B of an NT GEMM).
 *   w [rows x cols] NVFP4_BF16 or NVFP4_FP32; amax as nvfp4_quantize_1d;
 *   codes [rows x cols/2], scales [rows x cols/16], global_dec out.
 * Shapes: cols % 32 == 0; rows == 0 is a no-op.  Alignment as
 * nvfp4_quantize_1d.
 */
int32_t nvfp4_quantize_mse(const void* w, int32_t w_dtype, int64_t rows, int64_t cols,
                           float* amax, int32_t amax_is_input, uint8_t* codes, uint8_t* scales,
                           float* global_dec, void* stream);

/*
 * 2D (16x16) block quantization of weights (Super summary, Infra table: 2D
 * block scaling for weights; the 16x16 size is the reading).  Round to
 * nearest even, no transform.  A batch of `batch` independent slices
 * [rows x cols] (e.g. the routed experts' weights) each gets its own amax and
 * g.  Because the blocks are square, the same codes and scales serve W and
 * W^T.
 *   w [batch x rows x cols]; amax, global_dec: [batch] device floats;
 *   codes [batch x rows x cols/2]; scales [batch x rows/16 x cols/16].
 * Shapes: rows % 16 == 0, cols % 32 == 0.  Alignment as nvfp4_quantize_1d.
 */
int32_t nvfp4_quantize_2d(const void* w, int32_t w_dtype, int64_t batch, int64_t rows,
                          int64_t cols, float* amax, int32_t amax_is_input, uint8_t* codes,
                          uint8_t* scales, float* global_dec, void* stream);

/*
 * The 16-point Random Hadamard Transform alone, fp32 out (Super summary,
 * Infra table; the size is the reading): y = (1/4) H16 diag(s) x on every
 * 16-element block along `axis` (ROW or COL), same evaluation order as in
 * nvfp4_quantize_1d.  x [rows x cols] bf16/fp32, y [rows x cols] fp32.
 * Shapes: cols % 32 == 0; COL also rows % 16 == 0.  Alignment 16 bytes.
 */
int32_t nvfp4_rht16(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t axis,
                    uint32_t sign_mask, float* y, void* stream);

/*
 * Dequantize one operand (one slice): y[r][c] = RN32(RN32(val(code) * d) * g)
 * as fp32 [rows x cols].  `q` is a host struct of device pointers.
 */
int32_t nvfp4_dequantize(const nvfp4_operand* q, float* y, void* stream);

/*
 * NVFP4 GEMM (Super summary, Infra table: fprop, dgrad and wgrad GEMMs in
 * NVFP4; Ultra report section 2.2).  C [M x N] = op(A) op(B) * gA * gB with
 * row-major op letters:
 *   opA 'N': A stored [M x K];  'T': A stored [K x M];
 *   opB 'T': B stored [N x K];  'N': B stored [K x N].
 * Supported: NT (fprop Y = X W^T), NN (dgrad dX = dY W), TN (wgrad
 * dW = dY^T X).  TT returns NVFP4_ERR_UNSUPPORTED.  Each operand's blocks
 * must lie along K: ROW iff K is its contiguous dimension, COL iff K is its
 * row dimension, 2D either way.
 * Arithmetic: every decoded element val(code) * d is exact in fp16 (at most
 * 6 significant bits, range 2^-10 .. 2688); products are summed by MFMA with
 * fp32 accumulation (the pages trace a divergence to bf16 accumulation,
 * Ultra report section 2.7); epilogue C = RN32(acc * RN32(gA * gB)), then
 * bf16 (RNE) or fp32 per c_dtype; with NVFP4_FP32_ACCUMULATE, C (fp32) is
 * read and C = RN32(C + that fp32 result) is written.  The grouped GEMMs
 * take the same c_dtype values.
 * Shapes: K % 64 == 0 and K > 0 (one pipeline stage is 64 k); M, N >= 0;
 * the contiguous dimension of a stored operand is a multiple of 32 and a COL
 * or 2D operand has rows % 16 == 0; N % 8 == 0 and N < 2^21 (else
 * NVFP4_ERR_SHAPE).  M == 0 or N == 0 is a no-op.  Alignment: codes 16
 * bytes, scales 4, C 16 bytes.
 * NT with M <= 64 (decode-like shapes), or M <= 512 when 256 x 256 tiles
 * would leave CUs idle, runs a split-K kernel: K is divided among the waves
 * of a workgroup and their partial sums are added in a fixed order, so C is
 * deterministic but rounds differently from the tiled kernel's product
 * (within the same error bound).
 */
int32_t nvfp4_gemm(char opA, char opB, int64_t M, int64_t N, int64_t K, const nvfp4_operand* A,
                   const nvfp4_operand* B, void* C, int32_t c_dtype, void* stream);

/*
 * Grouped NVFP4 GEMM for the routed experts (Super report summary, sections
 * 2.1 and 2.2: routed-expert GEMMs in NVFP4, 512 experts with 22 active).
 * For every group e: C[o_e : o_{e+1}] = A[o_e : o_{e+1}] B_e^T * gA * gB_e,
 * with o = row_offsets (device int64 [groups + 1], o_0 = 0, non-decreasing,
 * o_groups = total_rows; ragged, empty groups allowed).
 *   A: [total_rows x K], ROW blocks, one g.
 *   B: `groups` slices [N x K] (B->rows = N, B->cols = K), 2D or ROW blocks,
 *      codes/scales consecutive per slice, global_dec [groups].
 *   C: [total_rows x N], bf16 or fp32.
 * Shapes: K % 64 == 0, K > 0, N % 16 == 0, N < 2^21, groups <= 4096.  A
 * row_offsets entry outside
 * [0, total_rows] or decreasing is a precondition violation (rows outside
 * [0, total_rows) are never touched).
 */
int32_t nvfp4_grouped_gemm(int64_t groups, const int64_t* row_offsets, int64_t total_rows,
                           int64_t N, int64_t K, const nvfp4_operand* A, const nvfp4_operand* B,
                           void* C, int32_t c_dtype, void* stream);

/*
 * Grouped dgrad for the routed experts (Super report summary, section 2.2:
 * the routed-expert GEMMs run in NVFP4; Ultra report section 2.2: dgrad in
 * NVFP4 with stochastically rounded gradients).  For every group e:
 * C[o_e : o_{e+1}] = A[o_e : o_{e+1}] B_e * gA * gB_e, with
 *   A: dY [total_rows x K], ROW blocks (nvfp4_quantize_1d / _dual, SR), one g;
 *   B: `groups` slices stored [K x N] (B->rows = K, B->cols = N), 2D or COL
 *      blocks, global_dec [groups] -- the same 2D codes as the fprop's
 *      [N x K] slices when the fprop weight is W_e^T (square blocks);
 *   C: [total_rows x N] bf16 or fp32; row_offsets as nvfp4_grouped_gemm.
 * Shapes: K % 64 == 0, K > 0, N % 32 == 0, N < 2^21, groups <= 4096.
 */
int32_t nvfp4_grouped_gemm_nn(int64_t groups, const int64_t* row_offsets, int64_t total_rows,
                              int64_t N, int64_t K, const nvfp4_operand* A,
                              const nvfp4_operand* B, void* C, int32_t c_dtype, void* stream);

/*
 * Grouped wgrad for the routed experts (Ultra report section 2.2: wgrad in
 * NVFP4 on Random-Hadamard-transformed inputs, gradients stochastically
 * rounded; section 2.7: fp32 accumulation).  The contraction runs over each
 * group's own tokens: for every group e,
 *   C[e] [M x N] fp32 = A[k_e : k_{e+1}]^T B[k_e : k_{e+1}] * gA * gB,
 * with k = k_offsets (device int64 [groups + 1], k_0 = 0, non-decreasing,
 * every entry a multiple of 16, k_groups = total_k), so a group with no
 * tokens gets C[e] = 0.
 *   A: dY rows gathered per group, each group's rows padded with zero rows
 *      to a multiple of 16, stored [total_k x M], COL blocks (so no block
 *      spans two groups), one g;
 *   B: X gathered and padded the same way, [total_k x N], COL blocks, one g;
 *   C: [groups x M x N] fp32.
 * Shapes: M % 32 == 0, N % 32 == 0, N < 2^21, total_k % 16 == 0,
 * groups <= 4096.  Offsets that break these rules are a precondition
 * violation (rows outside [0, total_k) are never read).
 */
int32_t nvfp4_grouped_gemm_tn(int64_t groups, const int64_t* k_offsets, int64_t total_k,
                              int64_t M, int64_t N, const nvfp4_operand* A,
                              const nvfp4_operand* B, float* C, void* stream);

/*
 * nvfp4_grouped_gemm_tn accumulating into fp32 main-grad buffers (Ultra
 * report section 2.7: local gradient accumulation must stay fp32): for every
 * group e, C[e] = RN32(C[e] + P_e) with P_e the product nvfp4_grouped_gemm_tn
 * writes (a group with no tokens adds +0).  Same arguments, shapes and
 * errors; C is read and written.
 */
int32_t nvfp4_grouped_gemm_tn_accumulate(int64_t groups, const int64_t* k_offsets,
                                         int64_t total_k, int64_t M, int64_t N,
                                         const nvfp4_operand* A, const nvfp4_operand* B,
                                         float* C, void* stream);

/*
 * fp32 -> fp16 with stochastic rounding, for an SSM (Mamba) state cache
 * (Super report summary, section 4.3: an fp16 cache rounded to nearest even
 * drifts through the recurrence; the recipe is fp16 with Philox<5>
 * stochastic rounding and no block scales).  With lo the largest fp16 <=
 * |x| and hi the next one, the magnitude rounds up iff
 * u < 65536 (|x| - lo) / (hi - lo), u the element's 16-bit slot: element i
 * uses slot i % 8 (word (i % 8) / 2, low half for even i) of Philox call
 * i / 8, counter (i / 8, offset), key seed.  |x| >= 65504 (and +-inf)
 * saturates to +-65504, NaN gives NaN (0x7E00 with x's sign), the sign is
 * kept (so -0 stays -0).
 *   x  device fp32 [n];  y  device fp16 bit patterns [n] out.
 * Shapes: any n >= 0 (n == 0 is a no-op).  Alignment: x and y 16 bytes.
 */
int32_t nvfp4_sr_fp16(const float* x, int64_t n, const nvfp4_philox* rng, uint16_t* y,
                      void* stream);

/*
 * Tuning of the single-pass quantizers (a performance setting: results are
 * the same either way).  A bf16 tensor of at most 1 GiB quantized with ROW
 * blocks and no transform (RNE or stochastic rounding) or with COL blocks
 * and RNE (with or without the transform), or bf16
 * 16x16-blocked matrices of at most 1 GiB each (one, or a batch), is
 * quantized in one launch: its workgroups keep what the registers hold,
 * stream the rest for its maximum, and meet at a grid barrier to combine the
 * tensor amax before encoding (the streamed part is read again); a batch is
 * split over groups of workgroups that each take one matrix at a time and
 * meet at the group's barrier.  They wait there at most wait_us microseconds (default
 * 2000); a workgroup that gives up, which only happens when other kernels
 * hold CUs (e.g. on concurrent streams), reads the whole tensor to take the
 * amax itself, so the results are unchanged but slower.  wait_us < 0 turns
 * the single-pass kernels off (every call then takes the two-pass path:
 * amax, then encode).  Applies to calls made after it, process-wide.
 * Returns the previous setting (-1 when off).
 */
int32_t nvfp4_set_single_pass_wait(int32_t wait_us);

/*
 * Debug checks.  The method quantizes finite tensors: every block scale and
 * code above is defined for finite inputs only, and a single infinity or NaN
 * makes the tensor amax, and with it every code of the tensor, meaningless
 * (the pages trace training divergences back through the numerics, "Nemotron
 * 3 Ultra" report, section 2.7).  With on != 0, every quantizer entry point
 * (nvfp4_quantize_1d, _2d, _dual, _mse and the gathering variants) first
 * scans its whole input on the caller's stream for infinities and NaNs,
 * waits for the result (a host synchronization), and returns
 * NVFP4_ERR_NONFINITE, writing nothing, if it finds one; a gathering call
 * scans all src_rows rows of x.  Off (the default), inputs are not checked
 * and a non-finite input is the caller's error.  The flag a scan sets lives
 * in a slot of device memory that the library owns; calls that overlap on
 * one device use different slots unless more than 256 are in flight.
 * Process-wide; returns the previous setting (0 or 1).
 */
int32_t nvfp4_set_debug_checks(int32_t on);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
