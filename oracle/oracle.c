/*
 * oracle.c -- plain, slow CPU oracle for the NVFP4 linear-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): the product path never includes,
 * links or calls it.  Every routine takes the method's steps one element or
 * one block at a time, in the order the spec states them, without blocking,
 * fusion or reordering.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 *        (x86-64 SSE arithmetic: every float op is IEEE binary32 RNE).
 */
#include "oracle.h"

#include <math.h>
#include <float.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ========================================================================
 * Element formats
 * ======================================================================== */

/* E2M1 (1 sign, 2 exponent, 1 mantissa bit) magnitudes by the 3-bit code.
 * NVFP4 stores elements as E2M1 ("Nemotron 3 Super" summary, gkm0120.cn,
 * pretraining-recipe table, training-precision row); the representable
 * magnitudes of that format are these eight values. */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float oracle_e2m1_decode(uint8_t code) {
  float m = (float)kE2M1Mag[code & 7];
  return (code & 8) ? -m : m; /* code 0x8 decodes to -0.0 */
}

/* Round-to-nearest onto the E2M1 grid, ties to the even code, saturating at
 * 6.  Reading: the pages name E2M1 but give no tie rule; IEEE's default
 * (nearest, ties to even) is used.  Written as a brute-force nearest search
 * over the eight magnitudes: |m - grid| is exact in double for fp32 m. */
uint8_t oracle_e2m1_encode_rne(float y) {
  uint8_t sign = signbit(y) ? 8 : 0;
  double m = fabs((double)y);
  if (m >= 6.0) return (uint8_t)(sign | 7); /* saturate (also avoids huge-m
                                               distance ties in double) */
  int best = 0;
  double best_d = fabs(m - kE2M1Mag[0]);
  for (int i = 1; i < 8; i++) {
    double d = fabs(m - kE2M1Mag[i]);
    if (d < best_d || (d == best_d && (i % 2) == 0)) {
      best = i;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* Stochastic rounding onto the E2M1 grid with a 16-bit uniform u16.
 * The pages: round-to-nearest-even has a biased expected error while
 * stochastic rounding is unbiased ("Nemotron 3 Super" report summary,
 * section 4.3), and gradients use stochastic rounding (Ultra report,
 * section 2.2).  Reading: with lo <= m < hi the neighbouring grid values and
 * f = (m - lo)/(hi - lo) (exact in fp32), round up iff u16 < f * 65536;
 * magnitudes >= 6 saturate to 6.  Values on the grid have f = 0 and never
 * move. */
uint8_t oracle_e2m1_encode_sr(float y, uint32_t u16) {
  uint8_t sign = signbit(y) ? 8 : 0;
  float m = fabsf(y);
  if (m >= 6.0f) return (uint8_t)(sign | 7);
  int lo = 0;
  for (int i = 0; i < 7; i++)
    if ((double)m >= kE2M1Mag[i]) lo = i;
  float lo_v = (float)kE2M1Mag[lo];
  float hi_v = (float)kE2M1Mag[lo + 1];
  float f = (m - lo_v) / (hi_v - lo_v); /* exact: Sterbenz, power-of-2 divisor */
  int up = (float)u16 < f * 65536.0f;
  return (uint8_t)(sign | (lo + up));
}

/* E4M3 (bias 7, 3 mantissa bits, no infinities, 0x7F = NaN, max 448).
 * Block scales are E4M3 (Super summary, pretraining-recipe table). */
float oracle_e4m3_decode(uint8_t e) {
  int s = e >> 7, ex = (e >> 3) & 15, mt = e & 7;
  float v;
  if (ex == 15 && mt == 7) return NAN;
  if (ex == 0)
    v = ldexpf((float)mt, -9); /* subnormal: mt * 2^-9 */
  else
    v = ldexpf(1.0f + (float)mt / 8.0f, ex - 7);
  return s ? -v : v;
}

/* Non-negative finite s -> nearest of the 127 finite non-negative E4M3
 * values, ties to the even code; anything at or above 448 gives 448 (0x7E).
 * Reading: saturate rather than produce NaN, since a block scale must stay a
 * finite number.  Brute force over all candidate codes. */
static double e4m3_value_table[0x7F];
static int e4m3_table_ready = 0;

static const double* e4m3_values(void) {
  if (!e4m3_table_ready) {
    for (int c = 0; c < 0x7F; c++)
      e4m3_value_table[c] = (double)oracle_e4m3_decode((uint8_t)c);
    e4m3_table_ready = 1;
  }
  return e4m3_value_table;
}

uint8_t oracle_e4m3_encode_rne_sat(float s) {
  const double* val = e4m3_values();
  if (s >= 448.0f) return 0x7E;
  int best = 0;
  double best_d = fabs((double)s - val[0]);
  for (int c = 1; c <= 0x7E; c++) {
    double d = fabs((double)s - val[c]);
    if (d < best_d || (d == best_d && (c % 2) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)best;
}

/* The two encoders above applied to arrays (threads split the elements;
 * each element is the scalar encoder's result). */
void oracle_e2m1_encode_rne_n(const float* y, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode_rne(y[i]);
}

void oracle_e4m3_encode_rne_sat_n(const float* s, int64_t n, uint8_t* out) {
  (void)e4m3_values(); /* fill the value table before the threads */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode_rne_sat(s[i]);
}

/* ========================================================================
 * Philox4x32-R (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011).  The pages use Philox with five rounds for
 * stochastic rounding ("Nemotron 3 Super" report summary, section 4.3).
 * ======================================================================== */
void oracle_philox4x32(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t rounds, uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (uint32_t r = 0; r < rounds; r++) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0; /* multiplier of word 0 */
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2; /* multiplier of word 2 */
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u; /* Weyl key schedule */
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Reading (the pages fix no layout): key = (lo32(seed), hi32(seed)); block b
 * makes two calls j = 0, 1 with counter (lo32(2b+j), hi32(2b+j), lo32(offset),
 * hi32(offset)).  Element e (0..15, position along the block axis) takes
 * call e>>3, word (e>>1)&3, and the low (e even) or high (e odd) 16 bits. */
uint32_t oracle_sr_bits(uint64_t seed, uint64_t offset, uint32_t rounds,
                        uint64_t block, int e) {
  uint64_t n = 2 * block + (uint64_t)(e >> 3);
  uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), (uint32_t)offset,
                     (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32(ctr, key, rounds, out);
  uint32_t w = out[(e >> 1) & 3];
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* ========================================================================
 * Randomized Hadamard transform, 16 points (Super summary, Infra table,
 * quantization row; Ultra report section 2.2: applied to the wgrad inputs).
 * Reading: v = (1/4) H16 diag(s) x, H16 the Sylvester Hadamard matrix
 * H[i][j] = (-1)^popcount(i & j), s_i = -1 where bit i of the mask is set.
 * Evaluated as sign flips, then butterflies with strides 1, 2, 4, 8 (each
 * sum and difference RN32), then an exact multiply by 1/4.
 * ======================================================================== */
void oracle_rht16_vec(float v[16], uint32_t sign_mask) {
  for (int i = 0; i < 16; i++)
    if ((sign_mask >> i) & 1u) v[i] = -v[i];
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; i++) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  for (int i = 0; i < 16; i++) v[i] = v[i] * 0.25f;
}

/* ========================================================================
 * Per-tensor second-level scale (not on the pages; the reading): the tensor
 * amax A maps onto the largest encodable magnitude 6 * 448 = 2688.
 *   S = RN32(2688 / A) (FLT_MAX if that overflows; 1 if A == 0)
 *   k = RN32(S / 6)     block-scale multiplier
 *   g = RN32(A / 2688)  decode scale used by dequantize and the GEMM
 * ======================================================================== */
void oracle_global_scales(float amax, float* S, float* k, float* g) {
  float s;
  if (amax == 0.0f) {
    s = 1.0f;
  } else {
    s = 2688.0f / amax;
    if (isinf(s)) s = FLT_MAX;
  }
  *S = s;
  *k = s / 6.0f;
  *g = amax / 2688.0f;
}

/* ========================================================================
 * Tensor quantization
 * ======================================================================== */
static float load_elem(const void* x, int is_bf16, int64_t idx) {
  if (is_bf16) {
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16; /* exact */
    float f;
    memcpy(&f, &bits, 4);
    return f;
  }
  return ((const float*)x)[idx];
}

/* Block ids, for one [rows x cols] slice (they seed the Philox counter):
 * ROW: block (r, c/16), id r*(cols/16) + c/16.
 * COL: block (r/16, c), id c*(rows/16) + r/16  (fiber-major, so COL of X
 *      equals the transpose of ROW of X^T, random bits included).
 * 2D : block (r/16, c/16), id (r/16)*(cols/16) + c/16.                 */
static int64_t block_id(int block, int64_t rows, int64_t cols, int64_t r,
                        int64_t c) {
  if (block == ORACLE_ROW) return r * (cols / 16) + c / 16;
  if (block == ORACLE_COL) return c * (rows / 16) + r / 16;
  return (r / 16) * (cols / 16) + c / 16;
}

/* Position of element (r, c) inside its block along the block axis. */
static int pos_in_block(int block, int64_t r, int64_t c) {
  if (block == ORACLE_COL) return (int)(r % 16);
  return (int)(c % 16);
}

/* Where the scale of element (r, c) is stored. */
static int64_t scale_index(int block, int64_t rows, int64_t cols, int64_t r,
                           int64_t c) {
  (void)rows;
  if (block == ORACLE_ROW) return r * (cols / 16) + c / 16;
  if (block == ORACLE_COL) return (r / 16) * cols + c;
  return (r / 16) * (cols / 16) + c / 16;
}

static int64_t scale_count(int block, int64_t rows, int64_t cols) {
  if (block == ORACLE_ROW) return rows * (cols / 16);
  if (block == ORACLE_COL) return (rows / 16) * cols;
  return (rows / 16) * (cols / 16);
}

static int check_shape(int block, int64_t rows, int64_t cols) {
  if (block < 0 || block > 2) return -4;
  if (rows < 0 || cols < 0) return -2;
  if (cols % 2) return -2; /* two codes per byte */
  if (block == ORACLE_ROW && cols % 16) return -2;
  if (block == ORACLE_COL && rows % 16) return -2;
  if (block == ORACLE_2D && (rows % 16 || cols % 16)) return -2;
  return 0;
}

/* v = the slice as fp32, with the 16-point RHT applied along the block axis
 * of every 16-element block when rht_mask >= 0 (rows [r0, r1) only). */
static void transform_slice(const void* x, int is_bf16, int64_t base,
                            int64_t rows, int64_t cols, int block,
                            int32_t rht_mask, int64_t r0, int64_t r1,
                            float* v) {
  (void)rows;
  for (int64_t r = r0; r < r1; r++)
    for (int64_t c = 0; c < cols; c++)
      v[r * cols + c] = load_elem(x, is_bf16, base + r * cols + c);
  if (rht_mask < 0) return;
  float t[16];
  if (block == ORACLE_ROW) {
    for (int64_t r = r0; r < r1; r++)
      for (int64_t c = 0; c < cols; c += 16) {
        for (int i = 0; i < 16; i++) t[i] = v[r * cols + c + i];
        oracle_rht16_vec(t, (uint32_t)rht_mask);
        for (int i = 0; i < 16; i++) v[r * cols + c + i] = t[i];
      }
  } else { /* ORACLE_COL */
    for (int64_t r = r0; r < r1; r += 16)
      for (int64_t c = 0; c < cols; c++) {
        for (int i = 0; i < 16; i++) t[i] = v[(r + i) * cols + c];
        oracle_rht16_vec(t, (uint32_t)rht_mask);
        for (int i = 0; i < 16; i++) v[(r + i) * cols + c] = t[i];
      }
  }
}

int oracle_quantize_rows(const void* x, int x_is_bf16, int64_t batch,
                         int64_t rows, int64_t cols, int block, int rounding,
                         uint64_t seed, uint64_t offset, uint32_t rounds,
                         int32_t rht_mask, const float* amax_in,
                         int64_t row_begin, int64_t row_end, uint8_t* codes,
                         uint8_t* scales, float* amax_out,
                         float* global_dec) {
  int rc = check_shape(block, rows, cols);
  if (rc) return rc;
  if (block == ORACLE_2D && (rounding != ORACLE_RNE || rht_mask >= 0))
    return -5;
  if (rht_mask > 0xFFFF || rht_mask < -1) return -5;
  if (rounding != ORACLE_RNE && rounding != ORACLE_SR) return -5;
  if (row_begin < 0 || row_end > rows || row_begin > row_end) return -2;
  if (block != ORACLE_ROW && (row_begin % 16 || row_end % 16)) return -2;
  if (!amax_in && (row_begin != 0 || row_end != rows)) return -2;

  int64_t nscale = scale_count(block, rows, cols);
  int64_t plane = rows * cols;
  float* v = (float*)malloc(sizeof(float) * (size_t)(plane > 0 ? plane : 1));
  float* blk_amax =
      (float*)malloc(sizeof(float) * (size_t)(nscale > 0 ? nscale : 1));
  if (!v || !blk_amax) {
    free(v);
    free(blk_amax);
    return -6;
  }

  for (int64_t s = 0; s < batch; s++) {
    int64_t base = s * plane;
    transform_slice(x, x_is_bf16, base, rows, cols, block, rht_mask, row_begin,
                    row_end, v);

    /* Step 1: tensor (slice) amax, after the transform. */
    float A = 0.0f;
    if (amax_in) {
      A = amax_in[s];
    } else {
      for (int64_t i = 0; i < plane; i++)
        if (fabsf(v[i]) > A) A = fabsf(v[i]);
    }
    /* Step 2: second-level scales. */
    float S, k, g;
    oracle_global_scales(A, &S, &k, &g);
    amax_out[s] = A;
    global_dec[s] = g;

    /* Step 3: per block: a_b = max |v|, s_b = RN32(a_b k), E4M3 scale. */
    for (int64_t i = 0; i < nscale; i++) blk_amax[i] = 0.0f;
    for (int64_t r = row_begin; r < row_end; r++)
      for (int64_t c = 0; c < cols; c++) {
        int64_t si = scale_index(block, rows, cols, r, c);
        float a = fabsf(v[r * cols + c]);
        if (a > blk_amax[si]) blk_amax[si] = a;
      }
    uint8_t* sc = scales + s * nscale;
    for (int64_t r = row_begin; r < row_end; r++)
      for (int64_t c = 0; c < cols; c++) {
        int64_t si = scale_index(block, rows, cols, r, c);
        float sb = blk_amax[si] * k;
        sc[si] = oracle_e4m3_encode_rne_sat(sb);
      }

    /* Step 4: per element: r_b = RN32(S / d_b) (0 when d_b = 0),
     * y = RN32(v r_b), then RNE or SR onto E2M1, two codes per byte. */
    uint8_t* cd = codes + s * (plane / 2);
    for (int64_t r = row_begin; r < row_end; r++)
      for (int64_t c = 0; c < cols; c++) {
        int64_t si = scale_index(block, rows, cols, r, c);
        float d = oracle_e4m3_decode(sc[si]);
        float rb = 0.0f;
        if (d != 0.0f) {
          rb = S / d;
          if (isinf(rb)) rb = FLT_MAX;
        }
        float y = v[r * cols + c] * rb;
        uint8_t q;
        if (rounding == ORACLE_SR) {
          int64_t b = block_id(block, rows, cols, r, c);
          uint32_t u = oracle_sr_bits(seed, offset, rounds, (uint64_t)b,
                                      pos_in_block(block, r, c));
          q = oracle_e2m1_encode_sr(y, u);
        } else {
          q = oracle_e2m1_encode_rne(y);
        }
        int64_t byte = (r * cols + c) / 2;
        if (c % 2 == 0)
          cd[byte] = (uint8_t)((cd[byte] & 0xF0) | q);
        else
          cd[byte] = (uint8_t)((cd[byte] & 0x0F) | (q << 4));
      }
  }
  free(v);
  free(blk_amax);
  return 0;
}

int oracle_quantize(const void* x, int x_is_bf16, int64_t batch, int64_t rows,
                    int64_t cols, int block, int rounding, uint64_t seed,
                    uint64_t offset, uint32_t rounds, int32_t rht_mask,
                    const float* amax_in, uint8_t* codes, uint8_t* scales,
                    float* amax_out, float* global_dec) {
  return oracle_quantize_rows(x, x_is_bf16, batch, rows, cols, block,
                              rounding, seed, offset, rounds, rht_mask,
                              amax_in, 0, rows, codes, scales, amax_out,
                              global_dec);
}

int oracle_amax(const void* x, int x_is_bf16, int64_t batch, int64_t rows,
                int64_t cols, int block, int32_t rht_mask, float* amax_out) {
  int rc = check_shape(block, rows, cols);
  if (rc) return rc;
  if (block == ORACLE_2D && rht_mask >= 0) return -5;
  int64_t plane = rows * cols;
  float* v = (float*)malloc(sizeof(float) * (size_t)(plane > 0 ? plane : 1));
  if (!v) return -6;
  for (int64_t s = 0; s < batch; s++) {
    transform_slice(x, x_is_bf16, s * plane, rows, cols, block, rht_mask, 0,
                    rows, v);
    float A = 0.0f;
    for (int64_t i = 0; i < plane; i++)
      if (fabsf(v[i]) > A) A = fabsf(v[i]);
    amax_out[s] = A;
  }
  free(v);
  return 0;
}

int oracle_rht16(const void* x, int x_is_bf16, int64_t rows, int64_t cols,
                 int block, uint32_t sign_mask, float* y) {
  if (block != ORACLE_ROW && block != ORACLE_COL) return -4;
  int rc = check_shape(block, rows, cols);
  if (rc) return rc;
  if (sign_mask > 0xFFFF) return -5;
  transform_slice(x, x_is_bf16, 0, rows, cols, block, (int32_t)sign_mask, 0,
                  rows, y);
  return 0;
}

static uint8_t code_at(const uint8_t* codes, int64_t cols, int64_t r,
                       int64_t c) {
  uint8_t byte = codes[(r * cols + c) / 2];
  return (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, float g,
                      int64_t rows, int64_t cols, int block, float* y) {
  int rc = check_shape(block, rows, cols);
  if (rc) return rc;
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++) {
      float e = oracle_e2m1_decode(code_at(codes, cols, r, c));
      float d = oracle_e4m3_decode(scales[scale_index(block, rows, cols, r, c)]);
      float ed = e * d; /* exact: <= 6 significant bits */
      y[r * cols + c] = ed * g;
    }
  return 0;
}

double oracle_operand_value(const uint8_t* codes, const uint8_t* scales,
                            int64_t rows, int64_t cols, int block, int64_t r,
                            int64_t c) {
  double e = (double)oracle_e2m1_decode(code_at(codes, cols, r, c));
  double d =
      (double)oracle_e4m3_decode(scales[scale_index(block, rows, cols, r, c)]);
  return e * d;
}

/* ========================================================================
 * GEMM reference (fp64).  Decoded operands are exact with <= 6 significant
 * bits, so every product is exact in fp64; only the sum rounds.
 * ======================================================================== */
static int gemm_check(char opA, char opB, int64_t M, int64_t N, int64_t K,
                      int a_block, int b_block) {
  if (!((opA == 'N' || opA == 'T') && (opB == 'N' || opB == 'T'))) return -4;
  if (M < 0 || N < 0 || K < 0) return -2;
  /* Quantization blocks must lie along K for the operand. */
  int a_kcontig = opA == 'N'; /* A stored [M][K] */
  int b_kcontig = opB == 'T'; /* B stored [N][K] */
  if (a_block == ORACLE_ROW && !a_kcontig) return -4;
  if (a_block == ORACLE_COL && a_kcontig) return -4;
  if (b_block == ORACLE_ROW && !b_kcontig) return -4;
  if (b_block == ORACLE_COL && b_kcontig) return -4;
  return 0;
}

static double a_val(char opA, int64_t M, int64_t K, const uint8_t* codes,
                    const uint8_t* scales, int blk, int64_t i, int64_t k) {
  if (opA == 'N') return oracle_operand_value(codes, scales, M, K, blk, i, k);
  return oracle_operand_value(codes, scales, K, M, blk, k, i);
}

static double b_val(char opB, int64_t N, int64_t K, const uint8_t* codes,
                    const uint8_t* scales, int blk, int64_t k, int64_t j) {
  if (opB == 'T') return oracle_operand_value(codes, scales, N, K, blk, j, k);
  return oracle_operand_value(codes, scales, K, N, blk, k, j);
}

int oracle_gemm_entries(char opA, char opB, int64_t M, int64_t N, int64_t K,
                        const uint8_t* a_codes, const uint8_t* a_scales,
                        int a_block, float gA, const uint8_t* b_codes,
                        const uint8_t* b_scales, int b_block, float gB,
                        const int64_t* ii, const int64_t* jj, int64_t n,
                        double* R, double* D) {
  int rc = gemm_check(opA, opB, M, N, K, a_block, b_block);
  if (rc) return rc;
  double gg = (double)gA * (double)gB;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; t++) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; k++) {
      double p = a_val(opA, M, K, a_codes, a_scales, a_block, ii[t], k) *
                 b_val(opB, N, K, b_codes, b_scales, b_block, k, jj[t]);
      acc += p;
      mag += fabs(p);
    }
    R[t] = gg * acc;
    D[t] = gg * mag;
  }
  return 0;
}

int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

int oracle_gemm_full(char opA, char opB, int64_t M, int64_t N, int64_t K,
                     const uint8_t* a_codes, const uint8_t* a_scales,
                     int a_block, float gA, const uint8_t* b_codes,
                     const uint8_t* b_scales, int b_block, float gB,
                     double* R, double* D) {
  int rc = gemm_check(opA, opB, M, N, K, a_block, b_block);
  if (rc) return rc;
  double gg = (double)gA * (double)gB;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; i++) {
    for (int64_t j = 0; j < N; j++) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double p = a_val(opA, M, K, a_codes, a_scales, a_block, i, k) *
                   b_val(opB, N, K, b_codes, b_scales, b_block, k, j);
        acc += p;
        mag += fabs(p);
      }
      R[i * N + j] = gg * acc;
      D[i * N + j] = gg * mag;
    }
  }
  return 0;
}

/* ========================================================================
 * fp32 -> fp16 stochastic rounding (SSM-state cache)
 * ======================================================================== */
static double fp16_values[0x7C00]; /* fp16 0x0000 .. 0x7BFF: ascending */
static int fp16_ready = 0;

static const double* fp16_table(void) {
  if (!fp16_ready) {
    for (int h = 0; h < 0x7C00; h++) {
      int e = h >> 10, m = h & 0x3FF;
      /* subnormal m * 2^-24; normal (1024 + m) * 2^(e - 25) */
      fp16_values[h] = e == 0 ? ldexp((double)m, -24) : ldexp(1024.0 + m, e - 25);
    }
    fp16_ready = 1;
  }
  return fp16_values;
}

uint16_t oracle_sr_fp16_one(float x, uint32_t u16) {
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7E00);
  const double a = fabs((double)x);
  if (a >= 65504.0) return (uint16_t)(sign | 0x7BFF);
  const double* V = fp16_table();
  int lo = 0, hi = 0x7BFE; /* the largest index with V[index] <= a */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (V[mid] <= a) lo = mid; else hi = mid - 1;
  }
  const double frac = (a - V[lo]) / (V[lo + 1] - V[lo]);
  const int up = (double)u16 < frac * 65536.0;
  return (uint16_t)(sign | (lo + up));
}

void oracle_sr_fp16(const float* x, int64_t n, uint64_t seed, uint64_t offset,
                    uint32_t rounds, uint16_t* y) {
  fp16_table();
  for (int64_t i = 0; i < n; i++) {
    /* call i/8 is call 2*(i/16) + (i%16)/8 of block i/16, slot i%8 */
    const uint32_t u = oracle_sr_bits(seed, offset, rounds, (uint64_t)(i >> 4), (int)(i & 15));
    y[i] = oracle_sr_fp16_one(x[i], u);
  }
}

/* ========================================================================
 * PTQ: MSE-calibrated block scales (ROW blocks, RNE)
 * ======================================================================== */
/* Squared error of block xb encoded with scale code e, as the max-based
 * quantizer would encode it with that scale: r = RN32(S / val(e)) (0 for a
 * zero scale), y = RN32(x r), RNE code, then the dequantized value
 * xh = RN32(RN32(val(code) val(e)) g).  The 16 terms (x - xh)^2 are summed
 * in fp64 in index order, one running sum. */
static double mse_candidate(const float* xb, uint8_t e, float S, float g, uint8_t* q) {
  const float d = oracle_e4m3_decode(e);
  float rb = 0.0f;
  if (d != 0.0f) {
    rb = S / d;
    if (isinf(rb)) rb = FLT_MAX;
  }
  double sum = 0.0;
  for (int i = 0; i < 16; i++) {
    q[i] = oracle_e2m1_encode_rne(xb[i] * rb);
    const float xh = (oracle_e2m1_decode(q[i]) * d) * g;
    const double err = (double)xb[i] - (double)xh;
    sum += err * err;
  }
  return sum;
}

int oracle_quantize_mse(const void* x, int x_is_bf16, int64_t rows, int64_t cols,
                        const float* amax_in, uint8_t* codes, uint8_t* scales,
                        float* amax_out, float* g_out) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return -2;
  float A = 0.0f;
  if (amax_in) {
    A = *amax_in;
  } else {
    for (int64_t i = 0; i < rows * cols; i++) {
      float a = fabsf(load_elem(x, x_is_bf16, i));
      if (a > A) A = a;
    }
  }
  float S, k, g;
  oracle_global_scales(A, &S, &k, &g);
  *amax_out = A;
  *g_out = g;
  (void)oracle_e4m3_encode_rne_sat(0.0f); /* fill the value table before the threads */
  /* Blocks are independent: threads split the rows. */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c0 = 0; c0 < cols; c0 += 16) {
      float xb[16];
      float a = 0.0f;
      for (int i = 0; i < 16; i++) {
        xb[i] = load_elem(x, x_is_bf16, r * cols + c0 + i);
        if (fabsf(xb[i]) > a) a = fabsf(xb[i]);
      }
      /* Start from the max-based scale; then every finite E4M3 code in
       * ascending order, replacing the choice only when strictly better.  So
       * the result is the argmin over all 127 codes; on a tie the max-based
       * code is kept if it is among the minima, else the smallest code. */
      const int e0 = oracle_e4m3_encode_rne_sat(a * k);
      uint8_t best_q[16], q[16];
      int best = e0;
      double best_err = mse_candidate(xb, (uint8_t)e0, S, g, best_q);
      for (int e = 0; e <= 126; e++) {
        if (e == e0) continue;
        const double err = mse_candidate(xb, (uint8_t)e, S, g, q);
        if (err < best_err) {
          best_err = err;
          best = e;
          memcpy(best_q, q, 16);
        }
      }
      scales[r * (cols / 16) + c0 / 16] = (uint8_t)best;
      for (int i = 0; i < 16; i += 2)
        codes[(r * cols + c0 + i) / 2] = (uint8_t)(best_q[i] | (best_q[i + 1] << 4));
    }
  return 0;
}
