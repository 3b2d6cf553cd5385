// quantize.hip -- NVFP4 quantizers, Hadamard transform and dequantizer for
// gfx950 (bandwidth-bound passes).
//
// Work mapping (wave64):
//  * ROW blocks (1x16 along the contiguous dim): the tensor is a flat stream
//    of 16-element blocks.  Each lane owns 8 consecutive elements (one 16-byte
//    bf16 load), so lanes 2t and 2t+1 share a block: its max takes one DPP
//    exchange, the 16-point transform's stride-8 stage one exchange of 8
//    values.  A lane stores one dword of codes; even lanes store the scale.
//  * COL blocks (16x1 along rows) and 2D blocks (16x16): each lane owns 8
//    columns x 16 rows, loading one 16-byte row segment per row, so each load
//    instruction reads 1 KiB of a row contiguously across the wave.  COL
//    blocks live entirely in one lane; 2D blocks span lanes 2t and 2t+1.
//  * The per-tensor amax runs first: a fill kernel zeroes it (no memset, so
//    the sequence can be captured in a graph), then every workgroup does one
//    atomicMax on the fp32 bits (non-negative floats order like integers, so
//    the result does not depend on the order).  For bf16 input the max of
//    |x| is taken on the 15 magnitude bits with packed 16-bit integer max.
//
// Arithmetic of the encoders (identical results to the element-wise
// definitions in nvfp4_device.hpp, which the oracle also follows):
//  * E2M1 round-to-nearest-even: v_cvt_scalef32_pk_fp4_f32 with scale 1,
//    which rounds every finite fp32 input exactly like the nearest-even
//    definition (ties to the even code, saturation at 6, signed zero);
//  * E4M3 block scale: v_cvt_scalef32_pk_fp8_f32 with scale 1 on
//    min(s, 448): the instruction rounds to nearest even but gives NaN
//    instead of saturating above 464, which the clamp removes;
//  * block reciprocal RN32(S / d) for all 127 E4M3 values d, computed once
//    per workgroup into an LDS table by IEEE division, then looked up.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

typedef short short2v __attribute__((ext_vector_type(2)));

// ---- loads ---------------------------------------------------------------------------
template <typename T>
struct In;

template <>
struct In<uint16_t> {  // bf16 bits
  static constexpr bool kBf16 = true;
  static __device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ uint4 raw(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
};

template <>
struct In<float> {
  static constexpr bool kBf16 = false;
  static __device__ __forceinline__ void load8(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ float max8(const float v[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) m = fmaxf(m, __builtin_fabsf(v[i]));
  return m;
}

// Max of |x| over 8 bf16 values given as 4 raw dwords, exact: non-negative
// bf16 bit patterns order like integers.
__device__ __forceinline__ float max8_bf16_bits(uint4 q) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 a = __builtin_bit_cast(u16x2, q.x & 0x7FFF7FFFu);
  u16x2 b = __builtin_bit_cast(u16x2, q.y & 0x7FFF7FFFu);
  u16x2 c = __builtin_bit_cast(u16x2, q.z & 0x7FFF7FFFu);
  u16x2 d = __builtin_bit_cast(u16x2, q.w & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
  uint32_t hi = m[0] > m[1] ? m[0] : m[1];
  return __uint_as_float(hi << 16);
}

// Value of the partner lane (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Stride-8 butterfly across the lane pair (2t holds positions 0..7, 2t+1
// positions 8..15), then the exact * 1/4.
__device__ __forceinline__ void rht_pair_stage8(float v[8], int odd) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float other = xor1(v[i]);
    float lo = odd ? other : v[i];
    float hi = odd ? v[i] : other;
    v[i] = (odd ? (lo - hi) : (lo + hi)) * 0.25f;
  }
}

// ---- block scale and reciprocal ---------------------------------------------------------
// LDS table of r = RN32(S / value(e)) (0 for e = 0, FLT_MAX on overflow) for
// the E4M3 codes e = 0..127; entry 127 (NaN code) is never looked up.
__device__ __forceinline__ void build_recip_table(float* tab, float S) {
  for (int e = threadIdx.x; e < 128; e += blockDim.x)
    tab[e] = block_recip(S, e4m3_decode((uint32_t)e));
  __syncthreads();
}

// E4M3 code of the block scale s = RN32(a * k): hardware RNE on min(s, 448).
__device__ __forceinline__ uint32_t block_code(float a, float k) {
  float s = fminf(a * k, 448.0f);
  short2v z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, s, s, 1.0f, false)) &
         0xFFu;
}

// 8 values (already multiplied by the block reciprocal) -> 8 RNE codes.
__device__ __forceinline__ uint32_t pack8_rne(const float y[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// ---- workgroup max -> atomicMax ---------------------------------------------------------
// Same-address atomics serialize in L2 (several ns each), so the amax passes
// run few, large workgroups (kAmaxThreads) and one atomic per workgroup.
constexpr int kAmaxThreads = 1024;

// m0 -> out0 and, when out1 is given, m1 -> out1 (one reduction pass).
__device__ __forceinline__ void block_max_to(float m0, float* out0, float m1 = 0.0f,
                                             float* out1 = nullptr) {
  __shared__ float red[2][kAmaxThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, o));
    m1 = fmaxf(m1, __shfl_xor(m1, o));
  }
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = m0;
    red[1][w] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 0; k < (out1 ? 2 : 1); k++) {
      float r = red[k][0];
      for (int i = 1; i < (int)(blockDim.x >> 6); i++) r = fmaxf(r, red[k][i]);
      // Thousands of workgroups target one address: skip the atomic when the
      // value already there is at least ours (it only grows, and the max of
      // the atomics performed is the same), which removes most of the
      // contention.
      unsigned int* p = reinterpret_cast<unsigned int*>(k ? out1 : out0);
      if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < __float_as_uint(r))
        atomicMax(p, __float_as_uint(r));
    }
  }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---- amax over flat 8-element chunks (ROW blocks, or no transform) -----------------------
// chunks: number of 8-element chunks per slice; slice = blockIdx.y.  A grid-
// stride loop in which each thread issues all its loads of a trip (U 16-byte
// loads, strided by the workgroup size so each load instruction is
// contiguous across the wave) before reducing them.
constexpr int kAmaxUnroll = 4;

// ---- input rows, optionally gathered (the MoE dispatch) ---------------------------------------
// Row r of the tensor being quantized is row r of x or, gathering, row idx[r]
// of x (src_rows rows); an index outside [0, src_rows) reads as a row of
// zeros, which is how per-expert padding rows are expressed.
template <bool kGather>
struct RowSrc {
  const int64_t* idx = nullptr;
  int64_t src_rows = 0;
  // Source row of row r, or -1 for a row of zeros.
  __device__ __forceinline__ int64_t at(int64_t r) const {
    if constexpr (!kGather) {
      return r;
    } else {
      const int64_t s = idx[r];
      return s >= 0 && s < src_rows ? s : -1;
    }
  }
  // Element offset of flat chunk i (8 elements, cpr chunks per row) and
  // whether it is read (false: zeros).  Gathering needs i < 2^32.
  __device__ __forceinline__ int64_t chunk(int64_t i, uint32_t cpr, bool& ok) const {
    if constexpr (!kGather) {
      ok = true;
      return i * 8;
    } else {
      const uint32_t r = (uint32_t)i / cpr, c = (uint32_t)i - r * cpr;
      const int64_t sr = at(r);
      ok = sr >= 0;
      return ((ok ? sr : 0) * cpr + c) * 8;
    }
  }
};

// p always points at readable data (a zero row reads source row 0, which
// exists: src_rows >= 1), so the load needs no branch; !ok selects zeros.
template <typename T>
__device__ __forceinline__ void load8_or_zero(const T* p, bool ok, float v[8]) {
  In<T>::load8(p, v);
#pragma unroll
  for (int t = 0; t < 8; t++) v[t] = ok ? v[t] : 0.0f;
}

// amax2 (nullable): a second target that receives the same maximum.
template <typename T, bool kRHT, bool kGather = false>
__global__ __launch_bounds__(kAmaxThreads) void amax_flat_kernel(const T* __restrict__ x,
                                                                 int64_t chunks, uint32_t mask,
                                                                 float* __restrict__ amax,
                                                                 float* __restrict__ amax2,
                                                                 RowSrc<kGather> rs = {},
                                                                 uint32_t cpr = 1) {
  const T* xs = x + (int64_t)blockIdx.y * chunks * 8;
  float m = 0.0f;
  constexpr int U = (In<T>::kBf16 && !kRHT) ? kAmaxUnroll : 2;
  constexpr int NT = kAmaxThreads;
  for (int64_t b = blockIdx.x; b * NT * U < chunks; b += gridDim.x) {
    const int64_t base = b * NT * U + threadIdx.x;
    if (In<T>::kBf16 && !kRHT) {
      uint4 q[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        int64_t i = base + (int64_t)u * NT;
        bool ok;
        const int64_t off = rs.chunk(i < chunks ? i : 0, cpr, ok);
        q[u] = i < chunks ? *reinterpret_cast<const uint4*>(xs + off) : make_uint4(0, 0, 0, 0);
        if (!ok) q[u] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; u++) m = fmaxf(m, max8_bf16_bits(q[u]));
    } else {
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; u++) {
        int64_t i = base + (int64_t)u * NT;
        // Past the end: zeros (a duplicated chunk would not change a plain
        // max, but its transform, paired with its partner, could).
        bool ok;
        const int64_t off = rs.chunk(i < chunks ? i : chunks - 1, cpr, ok);
        load8_or_zero(xs + off, ok, v[u]);
        if (i >= chunks)
#pragma unroll
          for (int q = 0; q < 8; q++) v[u][q] = 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (kRHT) {
          const int odd = (int)((base + (int64_t)u * NT) & 1);
          rht_signs_and_low_stages(v[u], mask, odd * 8);
          rht_pair_stage8(v[u], odd);
        }
        m = fmaxf(m, max8(v[u]));
      }
    }
  }
  block_max_to(m, amax + blockIdx.y, m, amax2);
}

// ---- amax of COL blocks with the transform (lane: 8 cols x 16 rows) ---------------------
// 256-thread workgroups: each lane holds a 16 x 8 tile and its transform,
// too many registers for the large amax workgroups.  kPlain: also the max of
// |x| itself (into amax_plain), from the same loads.
template <typename T, bool kPlain, bool kGather = false>
__global__ __launch_bounds__(kThreads) void amax_col_rht_kernel(const T* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                uint32_t mask,
                                                                float* __restrict__ amax,
                                                                float* __restrict__ amax_plain,
                                                                RowSrc<kGather> rs = {}) {
  const int64_t cg = cols / 8;
  const int64_t units = (rows / 16) * cg;
  float m = 0.0f, mp = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
    int64_t g = u / cg, c0 = (u % cg) * 8;
    float v[16][8];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t sr = rs.at(g * 16 + r);
      load8_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0, v[r]);
    }
    if (kPlain)
#pragma unroll
      for (int r = 0; r < 16; r++) mp = fmaxf(mp, max8(v[r]));
#pragma unroll
    for (int c = 0; c < 8; c++) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; r++) col[r] = v[r][c];
      rht16_inreg(col, mask);
#pragma unroll
      for (int r = 0; r < 16; r++) m = fmaxf(m, __builtin_fabsf(col[r]));
    }
  }
  if (kPlain)
    block_max_to(m, amax, mp, amax_plain);
  else
    block_max_to(m, amax);
}

// ---- ROW quantizer ---------------------------------------------------------------------------
// Lane chunk i (8 elements) belongs to block i >> 1; with stochastic rounding
// its Philox counter is 2 * block + (i & 1) = i.
constexpr int kRowUnroll = 4;

template <typename T, bool kSR, bool kRHT, bool kGather = false>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(
    const T* __restrict__ x, int64_t chunks, const float* __restrict__ amax,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec,
    uint32_t mask, uint64_t seed, uint64_t offset, uint32_t rounds, RowSrc<kGather> rs = {},
    uint32_t cpr = 1) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kRowUnroll + threadIdx.x;
  // Loads first (kRowUnroll 16-byte loads in flight), then the table.
  float v[kRowUnroll][8];
  float bm[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; u++) {
    int64_t i = base + (int64_t)u * kThreads;
    int64_t ic = i < chunks ? i : chunks - 1;  // chunks is even: pairs agree
    bool ok;
    const int64_t off = rs.chunk(ic, cpr, ok);
    load8_or_zero(x + off, ok, v[u]);
  }
  build_recip_table(rtab, ts.S);
#pragma unroll
  for (int u = 0; u < kRowUnroll; u++) {
    int64_t i = base + (int64_t)u * kThreads;
    const int odd = (int)(i & 1);
    if (kRHT) {
      rht_signs_and_low_stages(v[u], mask, odd * 8);
      rht_pair_stage8(v[u], odd);
    }
    float m = max8(v[u]);
    bm[u] = fmaxf(m, xor1(m));
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; u++) {
    int64_t i = base + (int64_t)u * kThreads;
    if (i >= chunks) continue;  // chunks is even: both lanes of a pair agree
    const int odd = (int)(i & 1);
    uint32_t e = block_code(bm[u], ts.k);
    float r = rtab[e];
    float y[8];
#pragma unroll
    for (int t = 0; t < 8; t++) y[t] = v[u][t] * r;
    uint32_t packed = 0;
    if (kSR) {
      Philox4 p = sr_call((uint64_t)i, seed, offset, rounds);
#pragma unroll
      for (int t = 0; t < 8; t++) packed |= e2m1_sr(y[t], sr_slot(p, t)) << (4 * t);
    } else {
      packed = pack8_rne(y);
    }
    codes[i] = packed;
    if (!odd) scales[i >> 1] = (uint8_t)e;
  }
}

// ---- small tensors: ROW quantization in one workgroup --------------------------------------------
// A decode step quantizes activations of a few rows per layer; three launches
// (clear, tensor amax, encode) would cost more than the data.  One workgroup
// takes the tensor amax (max of |x|: exact, whatever the order), publishes it
// through LDS and then encodes exactly as quant_row_kernel does (same block
// code, reciprocal table and rounding), so the outputs are bit-identical.
// Each thread takes kSmallUnroll chunks (all its loads in flight at once):
// the launch takes at most kSmallChunks chunks.
constexpr int kSmallThreads = 1024;
constexpr int kSmallUnroll = 8;         // chunks in flight per thread
constexpr int64_t kSmallChunks = kSmallThreads * kSmallUnroll;  // 8-element chunks (64 Ki elements)

template <typename T, bool kSR, bool kGather = false>
__global__ __launch_bounds__(kSmallThreads) void quant_row_small_kernel(
    const T* __restrict__ x, int64_t chunks, float* __restrict__ amax, bool amax_is_input,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec,
    uint64_t seed, uint64_t offset, uint32_t rounds, RowSrc<kGather> rs = {}, uint32_t cpr = 1) {
  __shared__ float rtab[128];
  __shared__ float red[kSmallThreads / 64];
  const int tid = threadIdx.x;
  float a;
  if (amax_is_input) {
    a = *amax;
  } else {
    float m = 0.0f;
    float v[kSmallUnroll][8];
#pragma unroll
    for (int u = 0; u < kSmallUnroll; u++) {  // all loads first (past the end: zeros)
      const int64_t i = tid + (int64_t)u * kSmallThreads;
      bool ok = false;
      const int64_t off = i < chunks ? rs.chunk(i, cpr, ok) : 0;
      if (i < chunks) {
        load8_or_zero(x + off, ok, v[u]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; t++) v[u][t] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kSmallUnroll; u++) m = fmaxf(m, max8(v[u]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int w = 1; w < kSmallThreads / 64; w++) a = fmaxf(a, red[w]);
    if (tid == 0) *amax = a;
  }
  const TensorScales ts = tensor_scales(a);
  if (tid == 0) *gdec = ts.g;
  build_recip_table(rtab, ts.S);
  // The stride is even and chunks is even: the two lanes of a block are
  // active together, so the pair exchange always finds its partner.
  float v[kSmallUnroll][8];
#pragma unroll
  for (int u = 0; u < kSmallUnroll; u++) {
    const int64_t i = tid + (int64_t)u * kSmallThreads;
    if (i < chunks) {
      bool ok;
      const int64_t off = rs.chunk(i, cpr, ok);
      load8_or_zero(x + off, ok, v[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kSmallUnroll; u++) {
    const int64_t i = tid + (int64_t)u * kSmallThreads;
    if (i >= chunks) break;
    const float mm = max8(v[u]);
    const float bm = fmaxf(mm, xor1(mm));
    const uint32_t e = block_code(bm, ts.k);
    const float r = rtab[e];
    float y[8];
#pragma unroll
    for (int t = 0; t < 8; t++) y[t] = v[u][t] * r;
    uint32_t packed = 0;
    if (kSR) {
      Philox4 p = sr_call((uint64_t)i, seed, offset, rounds);
#pragma unroll
      for (int t = 0; t < 8; t++) packed |= e2m1_sr(y[t], sr_slot(p, t)) << (4 * t);
    } else {
      packed = pack8_rne(y);
    }
    codes[i] = packed;
    if (!(i & 1)) scales[i >> 1] = (uint8_t)e;
  }
}

// ---- PTQ weights: ROW blocks with MSE-calibrated scales ----------------------------------------
// As the ROW quantizer (lane: 8 elements, lanes 2t and 2t+1: one block), but
// each block's E4M3 scale is the candidate with the smallest squared error
// of the dequantized block: the max-based code e0 first, then e0 + 1, e0 - 1,
// ..., e0 - 15 (within 0 .. 126), a candidate winning only when strictly
// better.  A lane sums its 8 squared errors in fp64 in index order; the pair
// adds its two halves (even lane's first), so both lanes hold the same error
// and make the same choice.  xh = RN32(RN32(val(code) d) g), the value the
// dequantizer gives.  The pair's two lanes agree on every branch here (the
// candidate list depends only on e0, the pair's), so the exchanges always
// find their partner active.
__device__ __forceinline__ double xor1_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0xB1, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0xB1, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Squared error (this lane's 8 elements) of the block quantized with scale
// code e; packed receives the 8 codes.
__device__ __forceinline__ double mse_half(const float v[8], uint32_t e, const float* rtab,
                                           float g, uint32_t& packed) {
  const float d = e4m3_decode(e);
  const float r = rtab[e];
  float y[8];
#pragma unroll
  for (int t = 0; t < 8; t++) y[t] = v[t] * r;
  packed = pack8_rne(y);
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    // codes 2q, 2q+1 (byte q) -> exact E2M1 values, by the fp16 conversion
    // (the one the GEMM decode uses), then exactly to fp32
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 h2;
    switch (q) {
      case 0: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0); break;
      case 1: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1); break;
      case 2: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2); break;
      default: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3); break;
    }
    const float val[2] = {(float)h2[0], (float)h2[1]};
    const float xh0 = (val[0] * d) * g, xh1 = (val[1] * d) * g;
    const double e0 = (double)v[2 * q] - (double)xh0, e1 = (double)v[2 * q + 1] - (double)xh1;
    acc = acc + e0 * e0;
    acc = acc + e1 * e1;
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_mse_row_kernel(
    const T* __restrict__ x, int64_t chunks, const float* __restrict__ amax,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const int64_t base = (int64_t)blockIdx.x * kThreads * 4 + threadIdx.x;
  float v[4][8];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int64_t i = base + (int64_t)u * kThreads;
    In<T>::load8(x + (i < chunks ? i : chunks - 1) * 8, v[u]);  // chunks is even: pairs agree
  }
  build_recip_table(rtab, ts.S);
#pragma unroll 1
  for (int u = 0; u < 4; u++) {
    const int64_t i = base + (int64_t)u * kThreads;
    const float m = max8(v[u]);
    const int e0 = (int)block_code(fmaxf(m, xor1(m)), ts.k);
    uint32_t best_q, q;
    double h = mse_half(v[u], (uint32_t)e0, rtab, ts.g, best_q);
    const bool odd = i & 1;
    // The pair's total: both lanes exchange halves outside any branch (a lane
    // shut off by a branch would be read as 0) and add them; the addition is
    // commutative, so both lanes get half0 + half1 exactly.
    double best_err = h + xor1_d(h);
    int best = e0;
#pragma unroll 1
    for (int t = 1; t <= 16; t++) {
      const int e = t == 1 ? e0 + 1 : e0 - (t - 1);
      if (e < 0 || e > 126) continue;  // the pair agrees (e0 is the pair's)
      h = mse_half(v[u], (uint32_t)e, rtab, ts.g, q);
      const double err = h + xor1_d(h);
      if (err < best_err) {
        best_err = err;
        best = e;
        best_q = q;
      }
    }
    if (i >= chunks) continue;
    codes[i] = best_q;
    if (!odd) scales[i >> 1] = (uint8_t)best;
  }
}

// ---- COL quantizer (lane: 8 cols x 16 rows = 8 blocks) ---------------------------------------
// The 16 rows stay as loaded (raw input words) and are worked one column pair
// at a time (the loop is kept rolled so that only one pair's transform and
// random bits are live): with stochastic rounding an unrolled lane would hold
// all 8 blocks' Philox output and its occupancy would drop to one wave per
// SIMD.
template <typename T>
struct RawRow;

template <>
struct RawRow<uint16_t> {  // 8 bf16 = 4 words; column pair p is word p
  uint4 q;
  __device__ __forceinline__ void load(const uint16_t* p) { q = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_or_zero(const uint16_t* p, bool ok) {  // p readable
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
    q = make_uint4(t.x & m, t.y & m, t.z & m, t.w & m);
  }
  __device__ __forceinline__ void pair(int p, float& a, float& b) const {
    const uint32_t w = p == 0 ? q.x : p == 1 ? q.y : p == 2 ? q.z : q.w;
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ __forceinline__ void all(float v[8]) const {
#pragma unroll
    for (int p = 0; p < 4; p++) pair(p, v[2 * p], v[2 * p + 1]);
  }
};

template <>
struct RawRow<float> {  // named words (no array, so selects stay in registers)
  uint4 lo, hi;         // elements 0..3, 4..7
  __device__ __forceinline__ void load(const float* p) {
    lo = reinterpret_cast<const uint4*>(p)[0];
    hi = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void load_or_zero(const float* p, bool ok) {  // p readable
    load(p);
    const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
    lo = make_uint4(lo.x & m, lo.y & m, lo.z & m, lo.w & m);
    hi = make_uint4(hi.x & m, hi.y & m, hi.z & m, hi.w & m);
  }
  __device__ __forceinline__ void pair(int p, float& a, float& b) const {
    const uint32_t wa = p == 0 ? lo.x : p == 1 ? lo.z : p == 2 ? hi.x : hi.z;
    const uint32_t wb = p == 0 ? lo.y : p == 1 ? lo.w : p == 2 ? hi.y : hi.w;
    a = __uint_as_float(wa);
    b = __uint_as_float(wb);
  }
  __device__ __forceinline__ void all(float v[8]) const {
#pragma unroll
    for (int p = 0; p < 4; p++) pair(p, v[2 * p], v[2 * p + 1]);
  }
};

// COL encode of one lane's 8 columns x 16 rows (8 blocks), from its raw
// rows: out[r] gets the 8 codes of row r, sc[0..1] the 8 scale bytes.
template <typename T, bool kSR, bool kRHT>
__device__ __forceinline__ void col_encode(const RawRow<T> (&raw)[16], int64_t rows, int64_t g,
                                           int64_t c0, const TensorScales& ts,
                                           const float* rtab, uint32_t mask, uint64_t seed,
                                           uint64_t offset, uint32_t rounds, uint32_t (&out)[16],
                                           uint32_t (&sc)[2]) {
#pragma unroll
  for (int r = 0; r < 16; r++) out[r] = 0;
  sc[0] = sc[1] = 0;
#pragma unroll 1
  for (int cp = 0; cp < 4; cp++) {  // column pairs (c, c+1) share one code byte per row
    float col[2][16];
#pragma unroll
    for (int r = 0; r < 16; r++) raw[r].pair(cp, col[0][r], col[1][r]);
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int c = 2 * cp + h;
      if (kRHT) rht16_inreg(col[h], mask);
      float bm = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r++) bm = fmaxf(bm, __builtin_fabsf(col[h][r]));
      const uint32_t e = block_code(bm, ts.k);
      const float rcp = rtab[e];
      sc[cp >> 1] |= e << (8 * (c & 3));
#pragma unroll
      for (int r = 0; r < 16; r++) col[h][r] = col[h][r] * rcp;
      if (kSR) {
        const uint64_t blk = (uint64_t)(c0 + c) * (uint64_t)(rows / 16) + (uint64_t)g;
        const Philox4 p0 = sr_call(2 * blk, seed, offset, rounds);
        const Philox4 p1 = sr_call(2 * blk + 1, seed, offset, rounds);
#pragma unroll
        for (int r = 0; r < 8; r++) out[r] |= e2m1_sr(col[h][r], sr_slot(p0, r)) << (4 * c);
#pragma unroll
        for (int r = 0; r < 8; r++)
          out[r + 8] |= e2m1_sr(col[h][r + 8], sr_slot(p1, r)) << (4 * c);
      }
    }
    if (!kSR) {
#pragma unroll
      for (int r = 0; r < 16; r++)
        out[r] |= __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, col[0][r], col[1][r], 1.0f, 0)
                  << (8 * cp);
    }
  }
}

template <typename T, bool kSR, bool kRHT, bool kGather = false>
__global__ __launch_bounds__(kThreads) void quant_col_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ amax,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec,
    uint32_t mask, uint64_t seed, uint64_t offset, uint32_t rounds, RowSrc<kGather> rs = {}) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const int64_t cg = cols / 8;
  const int64_t units = (rows / 16) * cg;
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t uc = u < units ? u : units - 1;
  const int64_t g = uc / cg, c0 = (uc % cg) * 8;
  RawRow<T> raw[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int64_t sr = rs.at(g * 16 + r);
    raw[r].load_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0);
  }
  build_recip_table(rtab, ts.S);
  if (u >= units) return;
  uint32_t out[16], sc[2];
  col_encode<T, kSR, kRHT>(raw, rows, g, c0, ts, rtab, mask, seed, offset, rounds, out, sc);
#pragma unroll
  for (int r = 0; r < 16; r++)
    *reinterpret_cast<uint32_t*>(codes + (g * 16 + r) * (cols / 2) + c0 / 2) = out[r];
  uint32_t* sp = reinterpret_cast<uint32_t*>(scales + g * cols + c0);
  sp[0] = sc[0];
  sp[1] = sc[1];
}

// ---- both 1D quantizations of a gradient from one read ---------------------------------------
// Zero-magnitude codes (0x0 or 0x8) among the 8 nibbles of w.
__device__ __forceinline__ uint32_t zero_nibbles(uint32_t w) {
  const uint32_t m = w & 0x77777777u;
  return 8u - (uint32_t)__builtin_popcount((m | (m >> 1) | (m >> 2)) & 0x11111111u);
}

// Lane: 8 columns x 16 rows, as the COL quantizer.  First its COL blocks,
// exactly as the COL quantizer (transform when kRHT).  Then the ROW blocks
// (1 x 16 along columns, no transform, stochastic rounding) of each of its 16
// rows, which span lanes 2t and 2t+1 (cols % 16 == 0 keeps the pairs in one
// row), exactly as the ROW quantizer forms them: block max across the pair,
// chunk i = (row * cols + c0) / 8 draws Philox call i of the ROW stream.  The
// ROW pass takes one row at a time and reads its 16 bytes again (a cache hit:
// the workgroup has just loaded them), which keeps it out of the COL pass's
// registers.  Both outputs are bit-identical to the two separate calls.
// zeros (nullable): the zero-magnitude codes of each output, summed per
// workgroup and added with one atomic each (an atomic per wave on the same
// two addresses serializes in L2 and doubled the kernel's time).
template <typename T, bool kRHT, bool kGather = false>
__global__ __launch_bounds__(kThreads) void quant_dual_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ amax,
    uint32_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    float* __restrict__ row_gdec, uint8_t* __restrict__ col_codes,
    uint8_t* __restrict__ col_scales, float* __restrict__ col_gdec, uint32_t mask,
    uint64_t seed_r, uint64_t offset_r, uint32_t rounds_r, uint64_t seed_c, uint64_t offset_c,
    uint32_t rounds_c, unsigned long long* __restrict__ zeros, RowSrc<kGather> rs = {}) {
  __shared__ float rtab_r[128], rtab_c[128];
  const TensorScales tr = tensor_scales(amax[0]), tc = tensor_scales(amax[1]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *row_gdec = tr.g;
    *col_gdec = tc.g;
  }
  const int64_t cg = cols / 8;
  const int64_t units = (rows / 16) * cg;  // even (cols % 16 == 0): lane pairs agree below
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool active = u < units;
  const int64_t uc = active ? u : units - 2 + (u & 1);  // the last pair, same parity
  const int64_t g = uc / cg, c0 = (uc % cg) * 8;
  RawRow<T> raw[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int64_t sr = rs.at(g * 16 + r);
    raw[r].load_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0);
  }
  for (int e = threadIdx.x; e < 128; e += blockDim.x) {
    const float d = e4m3_decode((uint32_t)e);
    rtab_r[e] = block_recip(tr.S, d);
    rtab_c[e] = block_recip(tc.S, d);
  }
  __syncthreads();
  uint32_t zr = 0, zc = 0;
  {
    uint32_t out[16], sc[2];
    col_encode<T, true, kRHT>(raw, rows, g, c0, tc, rtab_c, mask, seed_c, offset_c, rounds_c,
                              out, sc);
    if (active) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        *reinterpret_cast<uint32_t*>(col_codes + (g * 16 + r) * (cols / 2) + c0 / 2) = out[r];
        zc += zero_nibbles(out[r]);
      }
      uint32_t* sp = reinterpret_cast<uint32_t*>(col_scales + g * cols + c0);
      sp[0] = sc[0];
      sp[1] = sc[1];
    }
  }
  const bool even = (uc & 1) == 0;
#pragma unroll 1
  for (int r = 0; r < 16; r++) {
    RawRow<T> rr;  // this row's segment again (just loaded: a cache hit)
    const int64_t sr = rs.at(g * 16 + r);
    rr.load_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0);
    float v[8];
    rr.all(v);
    const float m = max8(v);
    const uint32_t e = block_code(fmaxf(m, xor1(m)), tr.k);
    const float rc = rtab_r[e];
    const int64_t chunk = (g * 16 + r) * cg + c0 / 8;
    const Philox4 p = sr_call((uint64_t)chunk, seed_r, offset_r, rounds_r);
    uint32_t packed = 0;
#pragma unroll
    for (int t = 0; t < 8; t++) packed |= e2m1_sr(v[t] * rc, sr_slot(p, t)) << (4 * t);
    if (active) {
      row_codes[chunk] = packed;
      if (even) row_scales[(g * 16 + r) * (cols / 16) + c0 / 16] = (uint8_t)e;
      zr += zero_nibbles(packed);
    }
  }
  if (zeros) {  // per workgroup: one atomic per output
    __shared__ uint32_t wz[2][kThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      zr += __shfl_xor(zr, o);
      zc += __shfl_xor(zc, o);
    }
    if ((threadIdx.x & 63) == 0) {
      wz[0][threadIdx.x >> 6] = zr;
      wz[1][threadIdx.x >> 6] = zc;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      unsigned long long t = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; w++) t += wz[threadIdx.x][w];
      if (t) atomicAdd(zeros + threadIdx.x, t);
    }
  }
}

// ---- 2D quantizer (lane: 8 cols x 16 rows; lanes 2t, 2t+1 = one 16x16 block) ------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void quant_2d_kernel(
    const T* __restrict__ w, int64_t rows, int64_t cols, const float* __restrict__ amax,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec) {
  __shared__ float rtab[128];
  const int64_t slice = blockIdx.y;
  const TensorScales ts = tensor_scales(amax[slice]);
  if (blockIdx.x == 0 && threadIdx.x == 0) gdec[slice] = ts.g;
  const T* ws = w + slice * rows * cols;
  uint8_t* cs = codes + slice * rows * (cols / 2);
  uint8_t* ss = scales + slice * (rows / 16) * (cols / 16);
  const int64_t cg = cols / 8;  // a multiple of 4, so pairs never straddle rows
  const int64_t units = (rows / 16) * cg;
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t uc = u < units ? u : units - 1;  // units is even: pairs agree
  const int64_t g = uc / cg, c0 = (uc % cg) * 8;
  float v[16][8];
  float bm = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    In<T>::load8(ws + (g * 16 + r) * cols + c0, v[r]);
    bm = fmaxf(bm, max8(v[r]));
  }
  bm = fmaxf(bm, xor1(bm));
  build_recip_table(rtab, ts.S);
  if (u >= units) return;
  uint32_t e = block_code(bm, ts.k);
  float rcp = rtab[e];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    float y[8];
#pragma unroll
    for (int t = 0; t < 8; t++) y[t] = v[r][t] * rcp;
    *reinterpret_cast<uint32_t*>(cs + (g * 16 + r) * (cols / 2) + c0 / 2) = pack8_rne(y);
  }
  if (((uc % cg) & 1) == 0) ss[g * (cols / 16) + c0 / 16] = (uint8_t)e;
}

// ---- standalone transform ------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void rht_row_kernel(const T* __restrict__ x, int64_t chunks,
                                                           uint32_t mask, float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= chunks) return;  // chunks even: lane pairs agree
  float v[8];
  In<T>::load8(x + i * 8, v);
  const int odd = (int)(i & 1);
  rht_signs_and_low_stages(v, mask, odd * 8);
  rht_pair_stage8(v, odd);
  float4* o = reinterpret_cast<float4*>(y + i * 8);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rht_col_kernel(const T* __restrict__ x, int64_t rows,
                                                           int64_t cols, uint32_t mask,
                                                           float* __restrict__ y) {
  const int64_t cg = cols / 8;
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= (rows / 16) * cg) return;
  const int64_t g = u / cg, c0 = (u % cg) * 8;
  float v[16][8];
#pragma unroll
  for (int r = 0; r < 16; r++) In<T>::load8(x + (g * 16 + r) * cols + c0, v[r]);
#pragma unroll
  for (int c = 0; c < 8; c++) {
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; r++) col[r] = v[r][c];
    rht16_inreg(col, mask);
#pragma unroll
    for (int r = 0; r < 16; r++) v[r][c] = col[r];
  }
#pragma unroll
  for (int r = 0; r < 16; r++) {
    float4* o = reinterpret_cast<float4*>(y + (g * 16 + r) * cols + c0);
    o[0] = make_float4(v[r][0], v[r][1], v[r][2], v[r][3]);
    o[1] = make_float4(v[r][4], v[r][5], v[r][6], v[r][7]);
  }
}

// ---- dequantize ------------------------------------------------------------------------------
// Lane: one dword of codes = 8 elements of one row.
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ gdec,
                                                          int64_t rows, int64_t cols, int block,
                                                          float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * cols / 8) return;
  const float g = *gdec;
  const int64_t r = (i * 8) / cols, c0 = (i * 8) % cols;
  const uint32_t q = codes[i];
  float out[8];
#pragma unroll
  for (int t = 0; t < 8; t++) {
    const int64_t c = c0 + t;
    int64_t si = block == kBlockRow ? r * (cols / 16) + c / 16
                 : block == kBlockCol ? (r / 16) * cols + c
                                      : (r / 16) * (cols / 16) + c / 16;
    const float d = e4m3_decode(scales[si]);
    const uint32_t code = (q >> (4 * t)) & 15u;
    const uint32_t mi = code & 7u;
    float mag = mi < 4u ? (float)mi * 0.5f : (mi < 6u ? (float)(mi - 2u) : (mi == 6u ? 4.0f : 6.0f));
    float val = (code & 8u) ? -mag : mag;
    float ed = val * d;  // exact
    out[t] = ed * g;
  }
  float4* o = reinterpret_cast<float4*>(y + i * 8);
  o[0] = make_float4(out[0], out[1], out[2], out[3]);
  o[1] = make_float4(out[4], out[5], out[6], out[7]);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups of an amax pass: one per kAmaxThreads * unroll units, capped
// near the CU count (the kernels loop over the rest) to keep the atomics few.
int amax_grid(int64_t units, int unroll, int64_t cap = 512) {
  int64_t g = cdiv(units, (int64_t)kAmaxThreads * unroll);
  return (int)(g < cap ? (g > 0 ? g : 1) : cap);
}

template <typename T, bool G>
hipError_t launch_quantize_1d_t(const QuantArgs& a, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  RowSrc<G> rs;
  if constexpr (G) {
    rs.idx = a.ridx;
    rs.src_rows = a.src_rows;
  }
  const uint32_t cpr = (uint32_t)(a.cols / 8);
  if (a.axis == kBlockRow && !a.rht && a.rows * a.cols / 8 <= kSmallChunks) {
    const int64_t chunks = a.rows * a.cols / 8;
    uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes);
    if (a.sr)
      quant_row_small_kernel<T, true, G><<<1, kSmallThreads, 0, st>>>(
          x, chunks, a.amax, a.amax_is_input, cd, a.scales, a.gdec, a.seed, a.offset, a.rounds,
          rs, cpr);
    else
      quant_row_small_kernel<T, false, G><<<1, kSmallThreads, 0, st>>>(
          x, chunks, a.amax, a.amax_is_input, cd, a.scales, a.gdec, 0, 0, 0, rs, cpr);
    return hipGetLastError();
  }
  if (!a.amax_is_input) {
    fill_zero_kernel<<<1, 64, 0, st>>>(a.amax, 1);
    if (a.axis == kBlockCol && a.rht) {
      int64_t units = (a.rows / 16) * (a.cols / 8);
      amax_col_rht_kernel<T, false, G>
          <<<(unsigned)std::min<int64_t>(cdiv(units, kThreads), 1024), kThreads, 0, st>>>(
              x, a.rows, a.cols, a.mask, a.amax, nullptr, rs);
    } else {
      int64_t chunks = a.rows * a.cols / 8;
      // ROW with the transform needs the pair exchange; COL amax without the
      // transform is the plain max.
      const int u = (!a.x_fp32 && !(a.rht && a.axis == kBlockRow)) ? kAmaxUnroll : 2;
      if (a.rht && a.axis == kBlockRow)
        amax_flat_kernel<T, true, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
            x, chunks, a.mask, a.amax, nullptr, rs, cpr);
      else
        amax_flat_kernel<T, false, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
            x, chunks, 0, a.amax, nullptr, rs, cpr);
    }
  }
  if (a.axis == kBlockRow) {
    int64_t chunks = a.rows * a.cols / 8;
    int grid = (int)cdiv(chunks, (int64_t)kThreads * kRowUnroll);
    uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes);
#define NVFP4_ROW(SR, RHT)                                                                     \
  quant_row_kernel<T, SR, RHT, G><<<grid, kThreads, 0, st>>>(x, chunks, a.amax, cd, a.scales, \
                                                             a.gdec, a.mask, a.seed, a.offset, \
                                                             a.rounds, rs, cpr)
    if (a.sr && a.rht) NVFP4_ROW(true, true);
    else if (a.sr) NVFP4_ROW(true, false);
    else if (a.rht) NVFP4_ROW(false, true);
    else NVFP4_ROW(false, false);
#undef NVFP4_ROW
  } else {
    int64_t units = (a.rows / 16) * (a.cols / 8);
    int grid = (int)cdiv(units, kThreads);
#define NVFP4_COL(SR, RHT)                                                                        \
  quant_col_kernel<T, SR, RHT, G><<<grid, kThreads, 0, st>>>(x, a.rows, a.cols, a.amax, a.codes, \
                                                             a.scales, a.gdec, a.mask, a.seed,   \
                                                             a.offset, a.rounds, rs)
    if (a.sr && a.rht) NVFP4_COL(true, true);
    else if (a.sr) NVFP4_COL(true, false);
    else if (a.rht) NVFP4_COL(false, true);
    else NVFP4_COL(false, false);
#undef NVFP4_COL
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_2d_t(const Quant2dArgs& a, hipStream_t st) {
  const T* w = static_cast<const T*>(a.w);
  if (!a.amax_is_input) {
    fill_zero_kernel<<<(unsigned)cdiv(a.batch, 256), 256, 0, st>>>(a.amax, a.batch);
    int64_t chunks = a.rows * a.cols / 8;
    const int u = a.w_fp32 ? 2 : kAmaxUnroll;
    // about 512 workgroups in all, at least one per slice
    const int64_t per = a.batch >= 512 ? 1 : 512 / a.batch;
    dim3 grid((unsigned)amax_grid(chunks, u, per), (unsigned)a.batch);
    amax_flat_kernel<T, false><<<grid, kAmaxThreads, 0, st>>>(w, chunks, 0, a.amax, nullptr);
  }
  int64_t units = (a.rows / 16) * (a.cols / 8);
  dim3 grid((unsigned)cdiv(units, kThreads), (unsigned)a.batch);
  quant_2d_kernel<T><<<grid, kThreads, 0, st>>>(w, a.rows, a.cols, a.amax, a.codes, a.scales,
                                                a.gdec);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rht16_t(const void* xv, int64_t rows, int64_t cols, int axis, uint32_t mask,
                          float* y, hipStream_t st) {
  const T* x = static_cast<const T*>(xv);
  if (axis == kBlockRow) {
    int64_t chunks = rows * cols / 8;
    rht_row_kernel<T><<<(unsigned)cdiv(chunks, kThreads), kThreads, 0, st>>>(x, chunks, mask, y);
  } else {
    int64_t units = (rows / 16) * (cols / 8);
    rht_col_kernel<T><<<(unsigned)cdiv(units, kThreads), kThreads, 0, st>>>(x, rows, cols, mask,
                                                                            y);
  }
  return hipGetLastError();
}

template <typename T, bool G>
hipError_t launch_quantize_dual_t(const QuantDualArgs& a, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  RowSrc<G> rs;
  if constexpr (G) {
    rs.idx = a.ridx;
    rs.src_rows = a.src_rows;
  }
  const int64_t units = (a.rows / 16) * (a.cols / 8);
  if (!a.amax_is_input) {
    fill_zero_kernel<<<1, 64, 0, st>>>(a.amax, 2);
    if (a.rht) {  // transform max for COL, plain max for ROW, one read
      amax_col_rht_kernel<T, true, G>
          <<<(unsigned)std::min<int64_t>(cdiv(units, kThreads), 1024), kThreads, 0, st>>>(
              x, a.rows, a.cols, a.mask, a.amax + 1, a.amax, rs);
    } else {  // the same plain max for both
      const int64_t chunks = a.rows * a.cols / 8;
      const int u = a.x_fp32 ? 2 : kAmaxUnroll;
      amax_flat_kernel<T, false, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
          x, chunks, 0, a.amax, a.amax + 1, rs, (uint32_t)(a.cols / 8));
    }
  }
  if (a.zeros) fill_zero_kernel<<<1, 64, 0, st>>>(reinterpret_cast<float*>(a.zeros), 4);
  const int grid = (int)cdiv(units, kThreads);
  uint32_t* rc = reinterpret_cast<uint32_t*>(a.row_codes);
#define NVFP4_DUAL(RHT)                                                                       \
  quant_dual_kernel<T, RHT, G><<<grid, kThreads, 0, st>>>(                                    \
      x, a.rows, a.cols, a.amax, rc, a.row_scales, a.row_gdec, a.col_codes, a.col_scales,     \
      a.col_gdec, a.mask, a.seed_r, a.offset_r, a.rounds_r, a.seed_c, a.offset_c, a.rounds_c, \
      a.zeros, rs)
  if (a.rht) NVFP4_DUAL(true);
  else NVFP4_DUAL(false);
#undef NVFP4_DUAL
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_mse_t(const void* xv, int64_t rows, int64_t cols, bool x_fp32,
                                 float* amax, bool amax_is_input, uint8_t* codes,
                                 uint8_t* scales, float* gdec, hipStream_t st) {
  const T* x = static_cast<const T*>(xv);
  const int64_t chunks = rows * cols / 8;
  if (!amax_is_input) {
    fill_zero_kernel<<<1, 64, 0, st>>>(amax, 1);
    const int u = x_fp32 ? 2 : kAmaxUnroll;
    amax_flat_kernel<T, false><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
        x, chunks, 0, amax, nullptr);
  }
  const int grid = (int)cdiv(chunks, (int64_t)kThreads * 4);
  quant_mse_row_kernel<T><<<grid, kThreads, 0, st>>>(x, chunks, amax,
                                                     reinterpret_cast<uint32_t*>(codes), scales,
                                                     gdec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mse(const void* x, bool x_fp32, int64_t rows, int64_t cols,
                               float* amax, bool amax_is_input, uint8_t* codes, uint8_t* scales,
                               float* gdec, hipStream_t st) {
  return x_fp32 ? launch_quantize_mse_t<float>(x, rows, cols, true, amax, amax_is_input, codes,
                                               scales, gdec, st)
                : launch_quantize_mse_t<uint16_t>(x, rows, cols, false, amax, amax_is_input,
                                                  codes, scales, gdec, st);
}

hipError_t launch_quantize_dual(const QuantDualArgs& a, hipStream_t st) {
  if (a.ridx)
    return a.x_fp32 ? launch_quantize_dual_t<float, true>(a, st)
                    : launch_quantize_dual_t<uint16_t, true>(a, st);
  return a.x_fp32 ? launch_quantize_dual_t<float, false>(a, st)
                  : launch_quantize_dual_t<uint16_t, false>(a, st);
}

hipError_t launch_quantize_1d(const QuantArgs& a, hipStream_t st) {
  if (a.ridx)
    return a.x_fp32 ? launch_quantize_1d_t<float, true>(a, st)
                    : launch_quantize_1d_t<uint16_t, true>(a, st);
  return a.x_fp32 ? launch_quantize_1d_t<float, false>(a, st)
                  : launch_quantize_1d_t<uint16_t, false>(a, st);
}

hipError_t launch_quantize_2d(const Quant2dArgs& a, hipStream_t st) {
  return a.w_fp32 ? launch_quantize_2d_t<float>(a, st) : launch_quantize_2d_t<uint16_t>(a, st);
}

hipError_t launch_rht16(const void* x, bool x_fp32, int64_t rows, int64_t cols, int axis,
                        uint32_t mask, float* y, hipStream_t st) {
  return x_fp32 ? launch_rht16_t<float>(x, rows, cols, axis, mask, y, st)
                : launch_rht16_t<uint16_t>(x, rows, cols, axis, mask, y, st);
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gdec,
                             int64_t rows, int64_t cols, int block, float* y, hipStream_t st) {
  int64_t n = rows * cols / 8;
  dequant_kernel<<<(unsigned)cdiv(n, kThreads), kThreads, 0, st>>>(
      reinterpret_cast<const uint32_t*>(codes), scales, gdec, rows, cols, block, y);
  return hipGetLastError();
}

}  // namespace nvfp4
