// api.cpp -- the C ABI of libnvfp4 (declared in include/nvfp4.h): argument
// validation, then kernel launches on the caller's stream.  Validation runs
// entirely on the host before any HIP call, so a rejected call launches
// nothing and touches no device state.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include <cstdint>

#include "launch.hpp"

namespace {

using nvfp4::DevOperand;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t device_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE; }

// Debug mode (nvfp4_set_debug_checks): the quantizers first check their
// input for infinities and NaNs.
std::atomic<int> g_debug_checks{0};

// NVFP4_OK, NVFP4_ERR_NONFINITE, or NVFP4_ERR_DEVICE; a no-op unless debug
// checks are on.
int32_t debug_finite(const void* x, bool x_fp32, int64_t n, void* stream) {
  if (!g_debug_checks.load(std::memory_order_relaxed)) return NVFP4_OK;
  bool finite = true;
  const hipError_t e =
      nvfp4::check_finite(x, x_fp32, n, static_cast<hipStream_t>(stream), &finite);
  if (e != hipSuccess) return NVFP4_ERR_DEVICE;
  return finite ? NVFP4_OK : NVFP4_ERR_NONFINITE;
}

bool valid_dtype(int32_t t) { return t == NVFP4_BF16 || t == NVFP4_FP32; }

// GEMM outputs may also accumulate into an fp32 C.
bool valid_out(int32_t t) { return valid_dtype(t) || t == NVFP4_FP32_ACCUMULATE; }

// The stored shape an operand must have, and the block kinds that tile K.
struct Expect {
  int64_t rows, cols;
  bool kmajor;
};

int32_t check_operand(const nvfp4_operand* q, const Expect& e) {
  if (!q || !q->codes || !q->scales || !q->global_dec) return NVFP4_ERR_NULL;
  if (q->rows != e.rows || q->cols != e.cols) return NVFP4_ERR_SHAPE;
  if (q->block == NVFP4_BLOCK_ROW && !e.kmajor) return NVFP4_ERR_LAYOUT;
  if (q->block == NVFP4_BLOCK_COL && e.kmajor) return NVFP4_ERR_LAYOUT;
  if (q->block != NVFP4_BLOCK_ROW && q->block != NVFP4_BLOCK_COL && q->block != NVFP4_BLOCK_2D)
    return NVFP4_ERR_LAYOUT;
  if (q->cols % 32 != 0) return NVFP4_ERR_SHAPE;  // contiguous dim: 16-byte code rows
  if ((q->block == NVFP4_BLOCK_COL || q->block == NVFP4_BLOCK_2D) && q->rows % 16 != 0)
    return NVFP4_ERR_SHAPE;
  // The kernels address operands through 32-bit buffer offsets: a K-major
  // operand through ranges over one tile's rows (at most 256 rows, so
  // cols < 2^24 keeps them under 2^31 bytes whatever the row count), an
  // MN-major one through one range over all of it.
  if (e.kmajor ? q->cols >= (int64_t(1) << 24) : q->rows * (q->cols / 2) >= (int64_t(1) << 31))
    return NVFP4_ERR_SHAPE;
  if (!aligned(q->codes, 16) || !aligned(q->scales, 4) || !aligned(q->global_dec, 4))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

DevOperand dev(const nvfp4_operand* q) {
  return DevOperand{q->codes, q->scales, q->global_dec, q->block};
}

// Output rows of a GEMM tile (at most 256 of them, 4-byte elements) must span
// fewer than 2^31 bytes: the epilogue's store offsets are 31-bit.
constexpr int64_t kMaxN = int64_t(1) << 21;

// Shared by the NT (fprop) and NN (dgrad) grouped GEMMs: B slices stored
// [N x K] (b_kmajor) or [K x N].
int32_t grouped_gemm(bool b_kmajor, int64_t groups, const int64_t* row_offsets,
                     int64_t total_rows, int64_t N, int64_t K, const nvfp4_operand* A,
                     const nvfp4_operand* B, void* C, int32_t c_dtype, void* stream) {
  if (!valid_out(c_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (groups < 0 || total_rows < 0 || N < 0 || K < 0) return NVFP4_ERR_SHAPE;
  if (groups > 4096) return NVFP4_ERR_SHAPE;
  if (K % 64 != 0 || N % 16 != 0 || K == 0 || N >= kMaxN) return NVFP4_ERR_SHAPE;
  if (!b_kmajor && N % 32 != 0) return NVFP4_ERR_SHAPE;  // B's contiguous dimension
  if (!row_offsets || !A || !B || !C) return NVFP4_ERR_NULL;
  if (!aligned(row_offsets, 8) || !aligned(C, 16)) return NVFP4_ERR_ALIGN;
  int32_t s = check_operand(A, Expect{total_rows, K, true});
  if (s != NVFP4_OK) return s;
  if (A->block != NVFP4_BLOCK_ROW) return NVFP4_ERR_LAYOUT;
  s = check_operand(B, b_kmajor ? Expect{N, K, true} : Expect{K, N, false});
  if (s != NVFP4_OK) return s;
  if (groups == 0 || total_rows == 0 || N == 0) return NVFP4_OK;
  nvfp4::GroupedArgs a{};
  a.groups = groups;
  a.offsets = row_offsets;
  a.total_rows = total_rows;
  a.N = N;
  a.K = K;
  a.A = dev(A);
  a.B = dev(B);
  a.b_kmajor = b_kmajor;
  a.C = C;
  a.c_bf16 = c_dtype == NVFP4_BF16;
  a.c_acc = c_dtype == NVFP4_FP32_ACCUMULATE;
  return device_status(nvfp4::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)));
}


}  // namespace

extern "C" {

int32_t nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int32_t s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "shape not supported by the block or tile sizes";
    case NVFP4_ERR_ALIGN: return "pointer misaligned";
    case NVFP4_ERR_LAYOUT: return "operand layout or block kind does not fit the op letters";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported mode";
    case NVFP4_ERR_DEVICE: return "HIP launch failed";
    case NVFP4_ERR_NONFINITE: return "input holds an infinity or a NaN (debug check)";
    default: return "unknown status";
  }
}

namespace {

// Gathering (row_index != null): row r of the quantized tensor is row
// row_index[r] of x's src_rows rows.  The flat chunk index of a ROW kernel is
// split into (row, chunk) with 32-bit arithmetic, hence rows * cols / 8 < 2^32.
int32_t gather_check(const void* x, int64_t src_rows, const int64_t* row_index, int64_t rows,
                     int64_t cols) {
  if (src_rows < 1) return NVFP4_ERR_SHAPE;
  if (rows * (cols / 8) >= (int64_t(1) << 32)) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (!row_index || !x)) return NVFP4_ERR_NULL;
  if (!aligned(row_index, 8)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int32_t quantize_1d(const void* x, int32_t x_dtype, const int64_t* row_index, int64_t src_rows,
                    int64_t rows, int64_t cols, int32_t axis, int32_t rounding,
                    const nvfp4_philox* rng, int32_t rht_sign_mask, float* amax,
                    int32_t amax_is_input, uint8_t* codes, uint8_t* scales, float* global_dec,
                    void* stream) {
  if (!valid_dtype(x_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (axis != NVFP4_BLOCK_ROW && axis != NVFP4_BLOCK_COL) return NVFP4_ERR_LAYOUT;
  if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_UNSUPPORTED;
  if (rht_sign_mask < -1 || rht_sign_mask > 0xFFFF) return NVFP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
  if (cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (axis == NVFP4_BLOCK_COL && rows % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rounding == NVFP4_SR && !rng) return NVFP4_ERR_NULL;
  if (rng && rounding == NVFP4_SR && (rng->rounds < 1 || rng->rounds > 16))
    return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!x || !amax || !codes || !scales || !global_dec) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(amax, 4) ||
      !aligned(global_dec, 4))
    return NVFP4_ERR_ALIGN;
  const int32_t fin =
      debug_finite(x, x_dtype == NVFP4_FP32, (row_index ? src_rows : rows) * cols, stream);
  if (fin != NVFP4_OK) return fin;
  nvfp4::QuantArgs a{};
  a.x = x;
  a.x_fp32 = x_dtype == NVFP4_FP32;
  a.rows = rows;
  a.cols = cols;
  a.axis = axis == NVFP4_BLOCK_ROW ? nvfp4::kBlockRow : nvfp4::kBlockCol;
  a.sr = rounding == NVFP4_SR;
  a.rht = rht_sign_mask >= 0;
  a.mask = a.rht ? (uint32_t)rht_sign_mask : 0u;
  a.seed = a.sr ? rng->seed : 0;
  a.offset = a.sr ? rng->offset : 0;
  a.rounds = a.sr ? rng->rounds : 0;
  a.amax = amax;
  a.amax_is_input = amax_is_input != 0;
  a.codes = codes;
  a.scales = scales;
  a.gdec = global_dec;
  a.ridx = row_index;
  a.src_rows = src_rows;
  return device_status(nvfp4::launch_quantize_1d(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int32_t nvfp4_quantize_1d(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                          int32_t axis, int32_t rounding, const nvfp4_philox* rng,
                          int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                          uint8_t* codes, uint8_t* scales, float* global_dec, void* stream) {
  return quantize_1d(x, x_dtype, nullptr, 0, rows, cols, axis, rounding, rng, rht_sign_mask, amax,
                     amax_is_input, codes, scales, global_dec, stream);
}

int32_t nvfp4_quantize_1d_gather(const void* x, int32_t x_dtype, int64_t src_rows,
                                 const int64_t* row_index, int64_t rows, int64_t cols,
                                 int32_t axis, int32_t rounding, const nvfp4_philox* rng,
                                 int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                                 uint8_t* codes, uint8_t* scales, float* global_dec,
                                 void* stream) {
  if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
  const int32_t g = gather_check(x, src_rows, row_index, rows, cols);
  if (g != NVFP4_OK) return g;
  return quantize_1d(x, x_dtype, row_index, src_rows, rows, cols, axis, rounding, rng,
                     rht_sign_mask, amax, amax_is_input, codes, scales, global_dec, stream);
}

namespace {

int32_t quantize_dual(const void* x, int32_t x_dtype, const int64_t* row_index, int64_t src_rows,
                      int64_t rows, int64_t cols, const nvfp4_philox* rng_row,
                      const nvfp4_philox* rng_col, int32_t rht_sign_mask, float* amax,
                      int32_t amax_is_input, uint8_t* row_codes, uint8_t* row_scales,
                      float* row_global_dec, uint8_t* col_codes, uint8_t* col_scales,
                      float* col_global_dec, uint64_t* zero_codes, void* stream) {
  if (!valid_dtype(x_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (rht_sign_mask < -1 || rht_sign_mask > 0xFFFF) return NVFP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (!rng_row || !rng_col) return NVFP4_ERR_NULL;
  if (rng_row->rounds < 1 || rng_row->rounds > 16 || rng_col->rounds < 1 || rng_col->rounds > 16)
    return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!x || !amax || !row_codes || !row_scales || !row_global_dec || !col_codes || !col_scales ||
      !col_global_dec)
    return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(row_codes, 16) || !aligned(col_codes, 16) ||
      !aligned(row_scales, 4) || !aligned(col_scales, 4) || !aligned(amax, 4) ||
      !aligned(row_global_dec, 4) || !aligned(col_global_dec, 4) || !aligned(zero_codes, 8))
    return NVFP4_ERR_ALIGN;
  const int32_t fin =
      debug_finite(x, x_dtype == NVFP4_FP32, (row_index ? src_rows : rows) * cols, stream);
  if (fin != NVFP4_OK) return fin;
  nvfp4::QuantDualArgs a{};
  a.x = x;
  a.x_fp32 = x_dtype == NVFP4_FP32;
  a.rows = rows;
  a.cols = cols;
  a.rht = rht_sign_mask >= 0;
  a.mask = a.rht ? (uint32_t)rht_sign_mask : 0u;
  a.seed_r = rng_row->seed;
  a.offset_r = rng_row->offset;
  a.rounds_r = rng_row->rounds;
  a.seed_c = rng_col->seed;
  a.offset_c = rng_col->offset;
  a.rounds_c = rng_col->rounds;
  a.amax = amax;
  a.amax_is_input = amax_is_input != 0;
  a.row_codes = row_codes;
  a.row_scales = row_scales;
  a.row_gdec = row_global_dec;
  a.col_codes = col_codes;
  a.col_scales = col_scales;
  a.col_gdec = col_global_dec;
  a.zeros = reinterpret_cast<unsigned long long*>(zero_codes);
  a.ridx = row_index;
  a.src_rows = src_rows;
  return device_status(nvfp4::launch_quantize_dual(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int32_t nvfp4_quantize_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                            const nvfp4_philox* rng_row, const nvfp4_philox* rng_col,
                            int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                            uint8_t* row_codes, uint8_t* row_scales, float* row_global_dec,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_global_dec,
                            uint64_t* zero_codes, void* stream) {
  return quantize_dual(x, x_dtype, nullptr, 0, rows, cols, rng_row, rng_col, rht_sign_mask, amax,
                       amax_is_input, row_codes, row_scales, row_global_dec, col_codes,
                       col_scales, col_global_dec, zero_codes, stream);
}

int32_t nvfp4_quantize_dual_gather(const void* x, int32_t x_dtype, int64_t src_rows,
                                   const int64_t* row_index, int64_t rows, int64_t cols,
                                   const nvfp4_philox* rng_row, const nvfp4_philox* rng_col,
                                   int32_t rht_sign_mask, float* amax, int32_t amax_is_input,
                                   uint8_t* row_codes, uint8_t* row_scales,
                                   float* row_global_dec, uint8_t* col_codes,
                                   uint8_t* col_scales, float* col_global_dec,
                                   uint64_t* zero_codes, void* stream) {
  if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
  const int32_t g = gather_check(x, src_rows, row_index, rows, cols);
  if (g != NVFP4_OK) return g;
  return quantize_dual(x, x_dtype, row_index, src_rows, rows, cols, rng_row, rng_col,
                       rht_sign_mask, amax, amax_is_input, row_codes, row_scales, row_global_dec,
                       col_codes, col_scales, col_global_dec, zero_codes, stream);
}

int32_t nvfp4_quantize_mse(const void* w, int32_t w_dtype, int64_t rows, int64_t cols,
                           float* amax, int32_t amax_is_input, uint8_t* codes, uint8_t* scales,
                           float* global_dec, void* stream) {
  if (!valid_dtype(w_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!w || !amax || !codes || !scales || !global_dec) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(amax, 4) ||
      !aligned(global_dec, 4))
    return NVFP4_ERR_ALIGN;
  const int32_t fin = debug_finite(w, w_dtype == NVFP4_FP32, rows * cols, stream);
  if (fin != NVFP4_OK) return fin;
  return device_status(nvfp4::launch_quantize_mse(w, w_dtype == NVFP4_FP32, rows, cols, amax,
                                                  amax_is_input != 0, codes, scales, global_dec,
                                                  static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_quantize_2d(const void* w, int32_t w_dtype, int64_t batch, int64_t rows,
                          int64_t cols, float* amax, int32_t amax_is_input, uint8_t* codes,
                          uint8_t* scales, float* global_dec, void* stream) {
  if (!valid_dtype(w_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (batch < 0 || rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
  if (rows % 16 != 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (batch > 65535) return NVFP4_ERR_SHAPE;
  if (batch == 0 || rows == 0 || cols == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!w || !amax || !codes || !scales || !global_dec) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(amax, 4) ||
      !aligned(global_dec, 4))
    return NVFP4_ERR_ALIGN;
  const int32_t fin = debug_finite(w, w_dtype == NVFP4_FP32, batch * rows * cols, stream);
  if (fin != NVFP4_OK) return fin;
  nvfp4::Quant2dArgs a{};
  a.w = w;
  a.w_fp32 = w_dtype == NVFP4_FP32;
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.amax = amax;
  a.amax_is_input = amax_is_input != 0;
  a.codes = codes;
  a.scales = scales;
  a.gdec = global_dec;
  return device_status(nvfp4::launch_quantize_2d(a, static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_rht16(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t axis,
                    uint32_t sign_mask, float* y, void* stream) {
  if (!valid_dtype(x_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (axis != NVFP4_BLOCK_ROW && axis != NVFP4_BLOCK_COL) return NVFP4_ERR_LAYOUT;
  if (sign_mask > 0xFFFFu) return NVFP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (axis == NVFP4_BLOCK_COL && rows % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!x || !y) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
  return device_status(nvfp4::launch_rht16(x, x_dtype == NVFP4_FP32, rows, cols,
                                           axis == NVFP4_BLOCK_ROW ? nvfp4::kBlockRow
                                                                   : nvfp4::kBlockCol,
                                           sign_mask, y, static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_dequantize(const nvfp4_operand* q, float* y, void* stream) {
  if (!q || !y) return NVFP4_ERR_NULL;
  if (q->rows < 0 || q->cols < 0) return NVFP4_ERR_SHAPE;
  Expect e{q->rows, q->cols, q->block != NVFP4_BLOCK_COL};
  int32_t s = check_operand(q, e);
  if (s != NVFP4_OK) return s;
  if (!aligned(y, 16)) return NVFP4_ERR_ALIGN;
  if (q->rows == 0 || q->cols == 0) return NVFP4_OK;
  return device_status(nvfp4::launch_dequantize(q->codes, q->scales, q->global_dec, q->rows,
                                                q->cols, q->block, y,
                                                static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_gemm(char opA, char opB, int64_t M, int64_t N, int64_t K, const nvfp4_operand* A,
                   const nvfp4_operand* B, void* C, int32_t c_dtype, void* stream) {
  if ((opA != 'N' && opA != 'T') || (opB != 'N' && opB != 'T')) return NVFP4_ERR_LAYOUT;
  if (opA == 'T' && opB == 'T') return NVFP4_ERR_UNSUPPORTED;
  if (!valid_out(c_dtype)) return NVFP4_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_SHAPE;
  if (K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (!A || !B || !C) return NVFP4_ERR_NULL;
  const bool a_k = opA == 'N', b_k = opB == 'T';
  Expect ea = a_k ? Expect{M, K, true} : Expect{K, M, false};
  Expect eb = b_k ? Expect{N, K, true} : Expect{K, N, false};
  int32_t s = check_operand(A, ea);
  if (s != NVFP4_OK) return s;
  s = check_operand(B, eb);
  if (s != NVFP4_OK) return s;
  if (N % 8 != 0 || N >= kMaxN) return NVFP4_ERR_SHAPE;
  if (!aligned(C, 16)) return NVFP4_ERR_ALIGN;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (K == 0) return NVFP4_ERR_SHAPE;  // nothing to contract: caller should fill C
  nvfp4::GemmArgs a{};
  a.a_kmajor = a_k;
  a.b_kmajor = b_k;
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = dev(A);
  a.B = dev(B);
  a.C = C;
  a.c_bf16 = c_dtype == NVFP4_BF16;
  a.c_acc = c_dtype == NVFP4_FP32_ACCUMULATE;
  return device_status(nvfp4::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_grouped_gemm(int64_t groups, const int64_t* row_offsets, int64_t total_rows,
                           int64_t N, int64_t K, const nvfp4_operand* A, const nvfp4_operand* B,
                           void* C, int32_t c_dtype, void* stream) {
  return grouped_gemm(true, groups, row_offsets, total_rows, N, K, A, B, C, c_dtype, stream);
}

int32_t nvfp4_grouped_gemm_nn(int64_t groups, const int64_t* row_offsets, int64_t total_rows,
                              int64_t N, int64_t K, const nvfp4_operand* A,
                              const nvfp4_operand* B, void* C, int32_t c_dtype, void* stream) {
  return grouped_gemm(false, groups, row_offsets, total_rows, N, K, A, B, C, c_dtype, stream);
}

namespace {

int32_t grouped_tn(bool accumulate, int64_t groups, const int64_t* k_offsets, int64_t total_k,
                   int64_t M, int64_t N, const nvfp4_operand* A, const nvfp4_operand* B, float* C,
                   void* stream) {
  if (groups < 0 || total_k < 0 || M < 0 || N < 0) return NVFP4_ERR_SHAPE;
  if (groups > 4096) return NVFP4_ERR_SHAPE;
  if (M % 32 != 0 || N % 32 != 0 || total_k % 16 != 0 || N >= kMaxN) return NVFP4_ERR_SHAPE;
  if (!k_offsets || !A || !B || !C) return NVFP4_ERR_NULL;
  if (!aligned(k_offsets, 8) || !aligned(C, 16)) return NVFP4_ERR_ALIGN;
  int32_t s = check_operand(A, Expect{total_k, M, false});
  if (s != NVFP4_OK) return s;
  s = check_operand(B, Expect{total_k, N, false});
  if (s != NVFP4_OK) return s;
  if (groups == 0 || M == 0 || N == 0) return NVFP4_OK;
  nvfp4::WgradArgs a{};
  a.groups = groups;
  a.k_offsets = k_offsets;
  a.total_k = total_k;
  a.M = M;
  a.N = N;
  a.A = dev(A);
  a.B = dev(B);
  a.C = C;
  a.c_acc = accumulate;
  return device_status(nvfp4::launch_grouped_wgrad(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int32_t nvfp4_grouped_gemm_tn(int64_t groups, const int64_t* k_offsets, int64_t total_k,
                              int64_t M, int64_t N, const nvfp4_operand* A,
                              const nvfp4_operand* B, float* C, void* stream) {
  return grouped_tn(false, groups, k_offsets, total_k, M, N, A, B, C, stream);
}

int32_t nvfp4_grouped_gemm_tn_accumulate(int64_t groups, const int64_t* k_offsets,
                                         int64_t total_k, int64_t M, int64_t N,
                                         const nvfp4_operand* A, const nvfp4_operand* B,
                                         float* C, void* stream) {
  return grouped_tn(true, groups, k_offsets, total_k, M, N, A, B, C, stream);
}

int32_t nvfp4_sr_fp16(const float* x, int64_t n, const nvfp4_philox* rng, uint16_t* y,
                      void* stream) {
  if (n < 0) return NVFP4_ERR_SHAPE;
  if (!rng) return NVFP4_ERR_NULL;
  if (rng->rounds < 1 || rng->rounds > 16) return NVFP4_ERR_UNSUPPORTED;
  if (n == 0) return NVFP4_OK;  // empty: pointers may be NULL
  if (!x || !y) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
  return device_status(nvfp4::launch_sr_fp16(x, n, rng->seed, rng->offset, rng->rounds, y,
                                             static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_set_debug_checks(int32_t on) {
  return g_debug_checks.exchange(on != 0 ? 1 : 0, std::memory_order_relaxed);
}

int32_t nvfp4_set_single_pass_wait(int32_t wait_us) {
  return nvfp4::set_single_pass_wait_us(wait_us);
}

}  // extern "C"
