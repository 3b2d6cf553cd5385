// launch.hpp -- internal interface between the C ABI (api.cpp) and the
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kBlockRow = 0;
constexpr int kBlockCol = 1;
constexpr int kBlock2d = 2;

struct QuantArgs {
  const void* x;
  bool x_fp32;
  int64_t rows, cols;
  int axis;  // kBlockRow / kBlockCol
  bool sr, rht;
  uint32_t mask;
  uint64_t seed, offset;
  uint32_t rounds;
  float* amax;
  bool amax_is_input;
  uint8_t* codes;
  uint8_t* scales;
  float* gdec;
  const int64_t* ridx;  // null, or row r of the input is row ridx[r] of x (MoE gather)
  int64_t src_rows;     // rows of x when gathering; other indices read as zero rows
};

// Both 1D quantizations of one gradient tensor from one read: ROW blocks with
// stochastic rounding (no transform) and COL blocks with stochastic rounding
// and, when rht, the transform.  amax[0] is the ROW tensor amax, amax[1] the
// COL one; zeros (nullable) receives the zero-magnitude code counts.
struct QuantDualArgs {
  const void* x;
  bool x_fp32;
  int64_t rows, cols;
  bool rht;
  uint32_t mask;
  uint64_t seed_r, offset_r, seed_c, offset_c;
  uint32_t rounds_r, rounds_c;
  float* amax;  // [2]
  bool amax_is_input;
  uint8_t *row_codes, *row_scales;
  float* row_gdec;
  uint8_t *col_codes, *col_scales;
  float* col_gdec;
  unsigned long long* zeros;  // [2] or null
  const int64_t* ridx;        // as QuantArgs
  int64_t src_rows;
};

struct Quant2dArgs {
  const void* w;
  bool w_fp32;
  int64_t batch, rows, cols;
  float* amax;
  bool amax_is_input;
  uint8_t* codes;
  uint8_t* scales;
  float* gdec;
};

// One GEMM operand as the kernels see it.  kmajor: stored [MN][K] (K
// contiguous), else stored [K][MN].  block: kBlockRow/kBlockCol/kBlock2d.
struct DevOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gdec;
  int block;
};

struct GemmArgs {
  bool a_kmajor, b_kmajor;  // NT: true,true  NN: true,false  TN: false,false
  int64_t M, N, K;
  DevOperand A, B;
  void* C;
  bool c_bf16;
  bool c_acc;  // fp32 C is added to: C = RN32(C + result)
};

struct GroupedArgs {
  int64_t groups;
  const int64_t* offsets;  // device [groups + 1]
  int64_t total_rows, N, K;
  DevOperand A;   // [total_rows x K] ROW
  DevOperand B;   // groups x [N x K] (b_kmajor; 2D or ROW) or [K x N] (2D or COL); gdec [groups]
  bool b_kmajor;  // NT (fprop) when true, NN (dgrad) when false
  void* C;
  bool c_bf16;
  bool c_acc;
};

// Grouped wgrad: C[e] [M x N] fp32 = A[k_e : k_{e+1}]^T B[k_e : k_{e+1}].
struct WgradArgs {
  int64_t groups;
  const int64_t* k_offsets;  // device [groups + 1], multiples of 16
  int64_t total_k, M, N;
  DevOperand A;  // [total_k x M] COL (or 2D)
  DevOperand B;  // [total_k x N] COL (or 2D)
  float* C;      // [groups x M x N]
  bool c_acc;    // C[e] += the product instead of C[e] = it
};

hipError_t launch_quantize_1d(const QuantArgs& a, hipStream_t st);
// Sets the single-pass kernels' barrier wait (microseconds; negative: do not
// use them) and returns the previous setting.
int set_single_pass_wait_us(int us);
// Debug check: *finite = false when any of the n elements (a multiple of 32)
// of the bf16 / fp32 tensor x is an infinity or a NaN.  Synchronizes st.
hipError_t check_finite(const void* x, bool x_fp32, int64_t n, hipStream_t st, bool* finite);
hipError_t launch_quantize_2d(const Quant2dArgs& a, hipStream_t st);
hipError_t launch_quantize_dual(const QuantDualArgs& a, hipStream_t st);
hipError_t launch_quantize_mse(const void* x, bool x_fp32, int64_t rows, int64_t cols,
                               float* amax, bool amax_is_input, uint8_t* codes, uint8_t* scales,
                               float* gdec, hipStream_t st);
hipError_t launch_rht16(const void* x, bool x_fp32, int64_t rows, int64_t cols, int axis,
                        uint32_t mask, float* y, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gdec,
                             int64_t rows, int64_t cols, int block, float* y, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_sr_fp16(const float* x, int64_t n, uint64_t seed, uint64_t offset,
                          uint32_t rounds, uint16_t* y, hipStream_t st);
hipError_t launch_grouped_gemm(const GroupedArgs& a, hipStream_t st);
hipError_t launch_grouped_wgrad(const WgradArgs& a, hipStream_t st);

}  // namespace nvfp4
