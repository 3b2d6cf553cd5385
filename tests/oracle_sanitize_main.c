/* Drives every entry point of the CPU oracle on small inputs held in buffers
 * of exactly the documented sizes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py): an access
 * past a buffer, an overflow of a signed type or a bad shift aborts the run.
 * Exit status 0 when every call returned its documented status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

static uint32_t rng = 12345u;
static float frand(void) {
  rng = rng * 1664525u + 1013904223u;
  return ((int32_t)(rng >> 8) - (1 << 23)) / (float)(1 << 21);
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) exit(2);
  return p;
}

int main(void) {
  const int64_t B = 2, R = 48, C = 64; /* batch, rows, cols */
  const int64_t n = B * R * C;
  float* xf = xmalloc(n * sizeof(float));
  uint16_t* xb = xmalloc(n * sizeof(uint16_t));
  for (int64_t i = 0; i < n; i++) {
    xf[i] = frand();
    uint32_t bits;
    memcpy(&bits, &xf[i], 4);
    xb[i] = (uint16_t)(bits >> 16);
  }
  xf[5] = 0.0f;
  xf[7] = -0.0f;
  uint8_t* codes = xmalloc(n / 2);
  float* amax = xmalloc(B * sizeof(float));
  float* g = xmalloc(B * sizeof(float));
  const int blocks[3] = {ORACLE_ROW, ORACLE_COL, ORACLE_2D};
  for (int bi = 0; bi < 3; bi++) {
    const int blk = blocks[bi];
    const int64_t ns = blk == ORACLE_ROW ? R * (C / 16) : blk == ORACLE_COL ? (R / 16) * C
                                                                            : (R / 16) * (C / 16);
    uint8_t* scales = xmalloc(B * ns);
    for (int bf = 0; bf < 2; bf++)
      for (int rnd = 0; rnd < 2; rnd++)
        for (int rht = 0; rht < 2; rht++) {
          const int expect = (blk == ORACLE_2D && (rnd || rht)) ? -5 : 0;
          int rc = oracle_quantize(bf ? (const void*)xb : (const void*)xf, bf, B, R, C, blk, rnd,
                                   7, 3, 5, rht ? 0xA5C3 : -1, NULL, codes, scales, amax, g);
          CHECK(rc == expect);
          if (rc == 0) {
            rc = oracle_quantize_rows(bf ? (const void*)xb : (const void*)xf, bf, B, R, C, blk,
                                      rnd, 7, 3, 5, rht ? 0xA5C3 : -1, amax, 16, 32, codes,
                                      scales, amax, g);
            CHECK(rc == 0);
            float* y = xmalloc(R * C * sizeof(float));
            CHECK(oracle_dequantize(codes, scales, g[0], R, C, blk, y) == 0);
            free(y);
          }
        }
    CHECK(oracle_amax(xf, 0, B, R, C, blk, blk == ORACLE_2D ? -1 : 0x00FF, amax) == 0);
    free(scales);
  }
  {
    float* y = xmalloc(R * C * sizeof(float));
    CHECK(oracle_rht16(xb, 1, R, C, ORACLE_ROW, 0x1234, y) == 0);
    CHECK(oracle_rht16(xf, 0, R, C, ORACLE_COL, 0xFFFF, y) == 0);
    free(y);
  }
  {
    /* MSE scales: ROW blocks, computed and given amax */
    uint8_t* sc = xmalloc(R * (C / 16));
    float a_in = 3.5f;
    CHECK(oracle_quantize_mse(xb, 1, R, C, NULL, codes, sc, amax, g) == 0);
    CHECK(oracle_quantize_mse(xf, 0, R, C, &a_in, codes, sc, amax, g) == 0);
    free(sc);
  }
  {
    /* GEMM references: NT (A ROW, B 2D), NN (B COL), TN (both COL) */
    const int64_t M = 32, N = 48, K = 64;
    float* a = xmalloc(M * K * sizeof(float));
    float* b = xmalloc(N * K * sizeof(float));
    for (int64_t i = 0; i < M * K; i++) a[i] = frand();
    for (int64_t i = 0; i < N * K; i++) b[i] = frand();
    uint8_t* ac = xmalloc(M * K / 2);
    uint8_t* as = xmalloc(M * K / 16);
    uint8_t* bc = xmalloc(N * K / 2);
    uint8_t* bs = xmalloc(N * K / 16);
    float ga, gb, aa, ab;
    double* R_ = xmalloc(M * N * sizeof(double));
    double* D_ = xmalloc(M * N * sizeof(double));
    int64_t ii[3] = {0, 5, M - 1}, jj[3] = {N - 1, 7, 0};
    double Re[3], De[3];
    CHECK(oracle_quantize(a, 0, 1, M, K, ORACLE_ROW, 0, 0, 0, 5, -1, NULL, ac, as, &aa, &ga) == 0);
    CHECK(oracle_quantize(b, 0, 1, N, K, ORACLE_2D, 0, 0, 0, 5, -1, NULL, bc, bs, &ab, &gb) == 0);
    CHECK(oracle_gemm_full('N', 'T', M, N, K, ac, as, ORACLE_ROW, ga, bc, bs, ORACLE_2D, gb, R_,
                           D_) == 0);
    CHECK(oracle_gemm_entries('N', 'T', M, N, K, ac, as, ORACLE_ROW, ga, bc, bs, ORACLE_2D, gb,
                              ii, jj, 3, Re, De) == 0);
    for (int t = 0; t < 3; t++) CHECK(Re[t] == R_[ii[t] * N + jj[t]]);
    /* One thread: the same values (the thread count only splits the outputs) */
    const int threads = oracle_set_threads(0);
    CHECK(threads >= 1);
    CHECK(oracle_set_threads(1) == 1);
    CHECK(oracle_gemm_entries('N', 'T', M, N, K, ac, as, ORACLE_ROW, ga, bc, bs, ORACLE_2D, gb,
                              ii, jj, 3, Re, De) == 0);
    for (int t = 0; t < 3; t++) CHECK(Re[t] == R_[ii[t] * N + jj[t]]);
    CHECK(oracle_set_threads(threads) == threads);
    /* B stored [K][N] with COL blocks (NN), A stored [K][M] with COL (TN) */
    float* bt = xmalloc(K * N * sizeof(float));
    float* at = xmalloc(K * M * sizeof(float));
    for (int64_t k = 0; k < K; k++) {
      for (int64_t j = 0; j < N; j++) bt[k * N + j] = b[j * K + k];
      for (int64_t i = 0; i < M; i++) at[k * M + i] = a[i * K + k];
    }
    uint8_t* bsc = xmalloc((K / 16) * N);
    uint8_t* asc = xmalloc((K / 16) * M);
    CHECK(oracle_quantize(bt, 0, 1, K, N, ORACLE_COL, 1, 9, 0, 5, 0x0F0F, NULL, bc, bsc, &ab,
                          &gb) == 0);
    CHECK(oracle_gemm_full('N', 'N', M, N, K, ac, as, ORACLE_ROW, ga, bc, bsc, ORACLE_COL, gb, R_,
                           D_) == 0);
    CHECK(oracle_quantize(at, 0, 1, K, M, ORACLE_COL, 0, 0, 0, 5, 0x0F0F, NULL, ac, asc, &aa,
                          &ga) == 0);
    CHECK(oracle_gemm_full('T', 'N', M, N, K, ac, asc, ORACLE_COL, ga, bc, bsc, ORACLE_COL, gb, R_,
                           D_) == 0);
    CHECK(oracle_gemm_entries('T', 'T', M, N, K, ac, asc, ORACLE_COL, ga, bc, bsc, ORACLE_COL, gb,
                              ii, jj, 3, Re, De) != 0);
    free(a); free(b); free(ac); free(as); free(bc); free(bs); free(R_); free(D_);
    free(bt); free(at); free(bsc); free(asc);
  }
  {
    /* fp16 stochastic rounding, scalar encoders, Philox */
    uint16_t* y = xmalloc(n * sizeof(uint16_t));
    oracle_sr_fp16(xf, n, 1, 2, 5, y);
    (void)oracle_sr_fp16_one(70000.0f, 3);
    uint8_t e[16];
    float v[16];
    for (int i = 0; i < 16; i++) v[i] = frand() * 100.0f;
    oracle_e2m1_encode_rne_n(v, 16, e);
    oracle_e4m3_encode_rne_sat_n(v, 16, e);
    for (int i = 0; i < 16; i++) (void)oracle_e2m1_encode_sr(v[i], (uint32_t)i * 4099u);
    oracle_rht16_vec(v, 0xBEEF);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    oracle_philox4x32(ctr, key, 10, out);
    (void)oracle_sr_bits(~0ull, ~0ull, 16, ~0ull >> 4, 15);
    float S, k, gg;
    oracle_global_scales(0.0f, &S, &k, &gg);
    oracle_global_scales(1e-38f, &S, &k, &gg);
    free(y);
  }
  free(xf); free(xb); free(codes); free(amax); free(g);
  puts("oracle sanitizer run: ok");
  return 0;
}
