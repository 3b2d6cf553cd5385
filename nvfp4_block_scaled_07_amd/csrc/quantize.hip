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
#include <atomic>
#include <type_traits>

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
  uint32_t w = __float_as_uint(y[0]);  // any start value: the four conversions write every byte
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// ---- workgroup max -> tensor amax --------------------------------------------------------
// Same-address atomics serialize in L2 (several ns each), so the amax passes
// run few, large workgroups (kAmaxThreads) and one atomic per workgroup.
constexpr int kAmaxThreads = 1024;

// Per-call scratch of the amax passes.  A pass combines its workgroups'
// maxima in a slot of this array instead of in the caller's output, which
// would need an extra launch to clear it first: each workgroup raises the
// maxima (atomicMax on the fp32 bits: non-negative floats order like
// integers, so the result does not depend on the order) and counts itself
// in; the last one to arrive copies the maxima to the caller's outputs and
// clears the slot for its next use.  The host hands slots out round
// robin (next_slot), so calls in flight at the same time on different
// streams use different slots unless more than kSlots of them overlap.  The
// array starts zeroed when the code object loads and every completed use
// leaves it zeroed.
//
// Same-address atomics serialize (about 20-25 ns each here), so a slot is
// two-level: workgroup b counts in at group line b % 8 (the XCD it runs on),
// and the last of each group carries the group's maxima and counts up to the
// top line.  A line sees at most a few dozen atomics.
struct alignas(128) Line {
  unsigned int bits0;   // running maximum
  unsigned int arrive;  // workgroups counted in
  unsigned int bits1;   // second running maximum
};
constexpr int kGroups = 8;
struct Slot {
  Line group[kGroups];
  Line top;
};
constexpr int kSlots = 256;
__device__ Slot g_slots[kSlots];

constexpr int kAgent = __HIP_MEMORY_SCOPE_AGENT;

// All slot accesses are relaxed device-scope atomics, which are coherent
// across the XCDs on their own; acquire/release orderings would also write
// back and invalidate the XCD's L2 on every access, which slowed the passes
// by tens of microseconds.  Where one atomic must be performed before the
// next one is issued (a maximum before the arrival that announces it), the
// first returns its old value and the wave waits for it (done()).
__device__ __forceinline__ void done(unsigned int v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ unsigned int ld(const unsigned int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, kAgent);
}
__device__ __forceinline__ void st(unsigned int* p, unsigned int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, kAgent);
}

__device__ __forceinline__ void raise_max(unsigned int* p, unsigned int v) {
  // Most workgroups find the maximum already at least theirs: a relaxed load
  // first skips their atomic, which removes most of the contention.
  if (ld(p) < v) done(__hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, kAgent));
}

// Counts workgroup blockIdx.x (of `count`) in: at its group line, then, for
// the last of the group, at the top line.  Before counting in at a level,
// the maxima (nmax of them) are raised there: a workgroup's own at its group
// line, a group's at the top line.  Returns true in the one workgroup that
// completes the count; the top line then holds the maxima.  Thread 0 only.
__device__ __forceinline__ bool count_in(Slot& s, unsigned int count, int nmax,
                                         const unsigned int* mx) {
  const unsigned int g = blockIdx.x % kGroups;
  const unsigned int ng = (count - g + kGroups - 1) / kGroups;  // workgroups of group g
  Line& L = s.group[g];
  if (nmax > 0) raise_max(&L.bits0, mx[0]);
  if (nmax > 1) raise_max(&L.bits1, mx[1]);
  if (__hip_atomic_fetch_add(&L.arrive, 1u, __ATOMIC_RELAXED, kAgent) != ng - 1) return false;
  Line& T = s.top;
  if (nmax > 0) raise_max(&T.bits0, ld(&L.bits0));
  if (nmax > 1) raise_max(&T.bits1, ld(&L.bits1));
  const unsigned int groups = count < kGroups ? count : kGroups;
  return __hip_atomic_fetch_add(&T.arrive, 1u, __ATOMIC_RELAXED, kAgent) == groups - 1;
}

// Zeroes every line of a slot (by the workgroup that completed its use).
__device__ __forceinline__ void slot_clear(Slot& s) {
  Line* l = &s.group[0];
  for (int i = 0; i < kGroups + 1; i++) {
    st(&l[i].bits0, 0u);
    st(&l[i].arrive, 0u);
    st(&l[i].bits1, 0u);
  }
}

// Maxima of m0 and m1 over the workgroup, valid in thread 0.
__device__ __forceinline__ void block_max2(float& m0, float& m1) {
  __shared__ float red[2][kAmaxThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, o));
    m1 = fmaxf(m1, __shfl_xor(m1, o));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = m0;
    red[1][w] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < (int)(blockDim.x >> 6); i++) {
      m0 = fmaxf(m0, red[0][i]);
      m1 = fmaxf(m1, red[1][i]);
    }
  }
}

// m0 -> out0 and, when out1 is given, m1 -> out1.  slot < 0: atomicMax
// straight into the outputs (cleared beforehand by the caller; used for
// batched slices).  slot >= 0: through g_slots[slot], `count` workgroups in
// all, with no clearing needed.
__device__ __forceinline__ void block_max_to(float m0, float* out0, float m1, float* out1,
                                             int slot, unsigned int count) {
  block_max2(m0, m1);
  if (threadIdx.x != 0) return;
  if (slot < 0) {
    raise_max(reinterpret_cast<unsigned int*>(out0), __float_as_uint(m0));
    if (out1) raise_max(reinterpret_cast<unsigned int*>(out1), __float_as_uint(m1));
    return;
  }
  Slot& s = g_slots[slot];
  const unsigned int mx[2] = {__float_as_uint(m0), __float_as_uint(m1)};
  if (count_in(s, count, out1 ? 2 : 1, mx)) {
    *out0 = __uint_as_float(ld(&s.top.bits0));
    if (out1) *out1 = __uint_as_float(ld(&s.top.bits1));
    slot_clear(s);
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
                                                                 int slot,
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
  block_max_to(m, amax + blockIdx.y, m, amax2, slot, gridDim.x);
}

// ---- a lane's 16 x 8 tile, kept as loaded ------------------------------------------------------
// The COL+RHT amax pass holds 16 rows of 8 columns per lane as raw input
// words and works them one column pair at a time.
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
  // Negates every element when neg (one XOR per two elements).
  __device__ __forceinline__ void flip(bool neg) {
    const uint32_t m = neg ? 0x80008000u : 0u;
    q = make_uint4(q.x ^ m, q.y ^ m, q.z ^ m, q.w ^ m);
  }
  __device__ __forceinline__ float absmax() const { return max8_bf16_bits(q); }
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
  __device__ __forceinline__ void flip(bool neg) {
    const uint32_t m = neg ? 0x80000000u : 0u;
    lo = make_uint4(lo.x ^ m, lo.y ^ m, lo.z ^ m, lo.w ^ m);
    hi = make_uint4(hi.x ^ m, hi.y ^ m, hi.z ^ m, hi.w ^ m);
  }
  __device__ __forceinline__ float absmax() const {
    float v[8];
    all(v);
    return max8(v);
  }
};


// ---- amax of COL blocks with the transform (lane: 8 cols x 16 rows) ---------------------
// 256-thread workgroups, one 16 x 8 tile per lane at a time, kept as raw
// words; the compiler issues the next tile's loads before transforming the
// current one, so the grid is sized to two workgroups per CU (what fits in
// the registers) and each lane takes several tiles.  kPlain:
// also the max of |x| itself (into amax_plain), from the same loads.  The
// transform's sign flips are applied to the raw words (exact negations), and
// its final * 1/4 to the maximum instead of to every element: rounding is
// monotone, so max |RN32(c / 4)| = RN32(max |c| / 4).
template <typename T, bool kPlain, bool kGather = false>
__global__ __launch_bounds__(kThreads) void amax_col_rht_kernel(const T* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                uint32_t mask,
                                                                float* __restrict__ amax,
                                                                float* __restrict__ amax_plain,
                                                                int slot,
                                                                RowSrc<kGather> rs = {}) {
  const int64_t cg = cols / 8;
  const int64_t units = (rows / 16) * cg;
  float m = 0.0f, mp = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto load_tile = [&](int64_t u, RawRow<T> (&raw)[16]) __attribute__((always_inline)) {
    const int64_t g = u / cg, c0 = (u % cg) * 8;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t sr = rs.at(g * 16 + r);
      raw[r].load_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0);
    }
  };
  auto tile_max = [&](RawRow<T> (&raw)[16]) __attribute__((always_inline)) {
    if (kPlain)
#pragma unroll
      for (int r = 0; r < 16; r++) mp = fmaxf(mp, raw[r].absmax());
#pragma unroll
    for (int r = 0; r < 16; r++) raw[r].flip((mask >> r) & 1u);
#pragma unroll
    for (int cp = 0; cp < 4; cp++) {
      float col[2][16];
#pragma unroll
      for (int r = 0; r < 16; r++) raw[r].pair(cp, col[0][r], col[1][r]);
#pragma unroll
      for (int h = 0; h < 2; h++) {
        hadamard16_unscaled(col[h]);
#pragma unroll
        for (int r = 0; r < 16; r++) m = fmaxf(m, __builtin_fabsf(col[h][r]));
      }
    }
  };
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if constexpr (std::is_same<T, uint16_t>::value && !kPlain && !kGather) {
    // Two tiles per trip: the second tile's 16 loads are issued before the
    // first tile's transform (bf16 holds 64 registers per tile).  The loads
    // are unconditional (a lane past its last tile re-reads the tensor's last
    // one and drops it), so the waits before a transform cover only its own
    // tile.  Without this the compiler waited for every load of a tile right
    // after issuing them.  It still waits for all loads at the top of the
    // loop (the tile loaded at the end of a trip), so half of the tiles'
    // loads overlap a transform: the [8192 x 6144] COL+RHT+SR quantizer went
    // from 66.8 to 65.1 us.
    // The tile to load next is kept as (block row g, column group c) and
    // stepped by the grid stride without a division (a 64-bit division
    // branches, and the compiler then waits for all loads at the join).
    const int64_t rows16 = rows / 16;  // >= 1: the pass runs on non-empty tensors only
    const int64_t sg = stride / cg, sc = stride % cg;
    int64_t g = u / cg, c = u % cg;
    auto load_next = [&](RawRow<T> (&raw)[16]) __attribute__((always_inline)) {
      const bool past = g >= rows16;  // re-read the last tile, which is dropped
      const int64_t gg = past ? rows16 - 1 : g, cc = past ? cg - 1 : c;
      const uint16_t* p = x + gg * 16 * cols + cc * 8;
#pragma unroll
      for (int r = 0; r < 16; r++) raw[r].load(p + r * cols);
      c += sc;
      const bool carry = c >= cg;
      c = carry ? c - cg : c;
      g += sg + (carry ? 1 : 0);
    };
    // The scheduling barriers keep the loads ahead of the transform (the
    // scheduler would otherwise sink them to their use to save registers).
    RawRow<T> ta[16], tb[16];
    load_next(ta);
    for (; u < units; u += 2 * stride) {
      load_next(tb);
      __builtin_amdgcn_sched_barrier(0);
      tile_max(ta);
      if (u + stride >= units) break;
      load_next(ta);
      __builtin_amdgcn_sched_barrier(0);
      tile_max(tb);
    }
  } else {
    for (; u < units; u += stride) {
      RawRow<T> raw[16];
      load_tile(u, raw);
      tile_max(raw);
    }
  }
  block_max_to(m * 0.25f, amax, mp, kPlain ? amax_plain : nullptr, slot, gridDim.x);
}

// Zero-magnitude codes (0x0 or 0x8) among the 8 nibbles of w.
__device__ __forceinline__ uint32_t zero_nibbles(uint32_t w) {
  const uint32_t m = w & 0x77777777u;
  return 8u - (uint32_t)__builtin_popcount((m | (m >> 1) | (m >> 2)) & 0x11111111u);
}

// Zero-code counts of the dual quantizer's two encode kernels, which run
// thousands of workgroups each (6144 for an [8192 x 6144] tensor).  Every
// wave adds its count to one line of a slot with an atomic whose result it
// does not wait for; after both kernels, one small kernel
// (zero_count_finish_kernel) sums the lines, writes the totals and clears
// the lines.  Finding the last workgroup in the encode kernels instead (two
// returning atomics per workgroup, as the amax passes do) kept every
// workgroup resident until its atomics returned and cost about 7 us per
// kernel.  Slots are indexed by the amax slots' round-robin numbers
// (next_slot), so calls in flight use different ones; 32 lines of 128
// bytes per slot.
constexpr int kZGroups = 32;
struct alignas(128) ZLine {
  unsigned long long sum;
};
struct ZSlot {
  ZLine group[kZGroups];
};
__device__ ZSlot g_zslots[kSlots];

// Zero-code count z of each thread, summed over the wave and added by its
// first lane to zero-count slot `slot` (line = the wave's number in the grid
// mod kZGroups).  No barrier: a workgroup-wide sum made the waves that
// finish first wait for the others, which cost more than the atomics.
__device__ __forceinline__ void grid_zero_count(uint32_t z, int slot) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  if ((threadIdx.x & 63) == 0 && z) {
    const unsigned int w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    (void)__hip_atomic_fetch_add(&g_zslots[slot].group[w % kZGroups].sum,
                                 (unsigned long long)z, __ATOMIC_RELAXED, kAgent);
  }
}

// The totals of zero-count slots s0 and s1 into out[0] and out[1], and the
// slots' lines cleared for their next use.  One wave; it runs after the
// kernels that counted (stream order), so their atomics are complete.
__global__ __launch_bounds__(64) void zero_count_finish_kernel(int s0, int s1,
                                                               unsigned long long* out) {
  static_assert(kZGroups <= 64, "one line per lane");
  const int l = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    ZLine* lines = g_zslots[k == 0 ? s0 : s1].group;
    unsigned long long v = 0;
    if (l < kZGroups) {
      v = __hip_atomic_load(&lines[l].sum, __ATOMIC_RELAXED, kAgent);
      __hip_atomic_store(&lines[l].sum, 0ull, __ATOMIC_RELAXED, kAgent);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (l == 0) out[k] = v;
  }
}

// ---- ROW quantizer ---------------------------------------------------------------------------
// Lane chunk i (8 elements) belongs to block i >> 1; with stochastic rounding
// its Philox counter is 2 * block + (i & 1) = i.
constexpr int kRowUnroll = 4;

// kZeros: also the number of zero-magnitude codes written, added to
// zero-count slot zslot (grid_zero_count).
template <typename T, bool kSR, bool kRHT, bool kGather = false, bool kZeros = false>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(
    const T* __restrict__ x, int64_t chunks, const float* __restrict__ amax,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec,
    uint32_t mask, uint64_t seed, uint64_t offset, uint32_t rounds, RowSrc<kGather> rs = {},
    uint32_t cpr = 1, int zslot = 0) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kRowUnroll + threadIdx.x;
  uint32_t zc = 0;  // zero codes written (kZeros)
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
    if (kSR) sr_values8(y, sr_call((uint64_t)i, seed, offset, rounds));
    const uint32_t packed = pack8_rne(y);
    codes[i] = packed;
    if (!odd) scales[i >> 1] = (uint8_t)e;
    if (kZeros) zc += zero_nibbles(packed);
  }
  if constexpr (kZeros) grid_zero_count(zc, zslot);
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
    if (kSR) sr_values8(y, sr_call((uint64_t)i, seed, offset, rounds));
    const uint32_t packed = pack8_rne(y);
    codes[i] = packed;
    if (!(i & 1)) scales[i >> 1] = (uint8_t)e;
  }
}

// ---- PTQ weights: ROW blocks with MSE-calibrated scales ----------------------------------------
// One lane per 16-element block.  Each block's E4M3 scale is the code, of all
// 127 finite ones, whose encoding of the block has the smallest squared
// error: the max-based code e0 is tried first, then codes 0 .. 126 in order,
// each replacing the choice only when strictly better (so a tie keeps e0 if
// it is a minimum, else the smallest code).  A code e encodes the block as
// the ROW quantizer would with that scale (r from the reciprocal table,
// y = RN32(x r), hardware RNE), decodes it as the dequantizer does
// (v_cvt_scalef32_pk_f16_fp4, exact, then RN32(RN32(val d) g)), and sums the
// 16 terms (x - xh)^2 in fp64 in index order.  Offline work (once per
// weight), so the 127 candidates are all evaluated.

// Squared error of the block v encoded with scale code e; packed receives
// its 16 codes (element 2j in the low nibble of byte j).
__device__ __forceinline__ double mse_block(const float v[16], const double vd[16], uint32_t e,
                                            const float* rtab, float g, uint2& packed) {
  const float d = e4m3_decode(e);
  const float r = rtab[e];
  float y[16];
#pragma unroll
  for (int t = 0; t < 16; t++) y[t] = v[t] * r;
  packed.x = pack8_rne(y);
  packed.y = pack8_rne(y + 8);
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < 8; q++) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const uint32_t w = q < 4 ? packed.x : packed.y;
    f16x2 h2;
    switch (q & 3) {
      case 0: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
      case 1: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
      case 2: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
      default: h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
    }
    const float xh0 = ((float)h2[0] * d) * g, xh1 = ((float)h2[1] * d) * g;
    const double e0 = vd[2 * q] - (double)xh0, e1 = vd[2 * q + 1] - (double)xh1;
    acc = acc + e0 * e0;
    acc = acc + e1 * e1;
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_mse_row_kernel(
    const T* __restrict__ x, int64_t blocks, const float* __restrict__ amax,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t bc = b < blocks ? b : blocks - 1;
  float v[16];
  In<T>::load8(x + bc * 16, v);
  In<T>::load8(x + bc * 16 + 8, v + 8);
  build_recip_table(rtab, ts.S);
  if (b >= blocks) return;
  double vd[16];
#pragma unroll
  for (int t = 0; t < 16; t++) vd[t] = (double)v[t];
  const uint32_t e0 = block_code(fmaxf(max8(v), max8(v + 8)), ts.k);
  uint2 best_q, q;
  double best_err = mse_block(v, vd, e0, rtab, ts.g, best_q);
  uint32_t best = e0;
#pragma unroll 1
  for (uint32_t e = 0; e <= 126; e++) {
    if (e == e0) continue;
    const double err = mse_block(v, vd, e, rtab, ts.g, q);
    if (err < best_err) {
      best_err = err;
      best = e;
      best_q = q;
    }
  }
  codes[b] = best_q;
  scales[b] = (uint8_t)best;
}

// ---- COL quantizer -----------------------------------------------------------------------------
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 dword3)
constexpr uint32_t kDropOff = 0x80000000u;  // past every range: loads read 0, stores are dropped

// The raw words of one column pair in one row (the COL kernels' lane unit).
template <typename T>
struct RawPair;

template <>
struct RawPair<uint16_t> {  // 2 bf16 = 1 word
  uint32_t w;
  __device__ __forceinline__ void load_or_zero(const uint16_t* p, bool ok) {  // p readable
    const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
    w = ok ? t : 0u;
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  }
  __device__ __forceinline__ void get(float& a, float& b) const {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ __forceinline__ void flip(bool neg) { w ^= neg ? 0x80008000u : 0u; }
};

template <>
struct RawPair<float> {
  uint2 w;
  __device__ __forceinline__ void load_or_zero(const float* p, bool ok) {  // p readable
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w = ok ? t : make_uint2(0u, 0u);
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  }
  __device__ __forceinline__ void get(float& a, float& b) const {
    a = __uint_as_float(w.x);
    b = __uint_as_float(w.y);
  }
  __device__ __forceinline__ void flip(bool neg) {
    const uint32_t m = neg ? 0x80000000u : 0u;
    w = make_uint2(w.x ^ m, w.y ^ m);
  }
};

// COL encode of the column pair (c0, c0 + 1) of block row g from its 16 raw
// rows (with the transform, its sign flips are applied to raw in place:
// exact negations of whole rows): code[r] gets row r's code byte (column c0
// in the low nibble), the result the two scale bytes (c0's low).
template <typename T, bool kSR, bool kRHT>
__device__ __forceinline__ uint32_t col_pair_encode(RawPair<T> (&raw)[16], int64_t rows,
                                                    int64_t g, uint32_t c0,
                                                    const TensorScales& ts, const float* rtab,
                                                    uint32_t mask, uint64_t seed,
                                                    uint64_t offset, uint32_t rounds,
                                                    uint32_t (&code)[16]) {
  if (kRHT)
#pragma unroll
    for (int r = 0; r < 16; r++) raw[r].flip((mask >> r) & 1u);
  float col[2][16];
#pragma unroll
  for (int r = 0; r < 16; r++) raw[r].get(col[0][r], col[1][r]);
  uint32_t sc = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    if (kRHT) {
      hadamard16_unscaled(col[h]);
#pragma unroll
      for (int r = 0; r < 16; r++) col[h][r] = col[h][r] * 0.25f;
    }
    float bm = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) bm = fmaxf(bm, __builtin_fabsf(col[h][r]));
    const uint32_t e = block_code(bm, ts.k);
    const float rcp = rtab[e];
    sc |= e << (8 * h);
#pragma unroll
    for (int r = 0; r < 16; r++) col[h][r] = col[h][r] * rcp;
    if (kSR) {  // rows 0..7 take call 2 * block, rows 8..15 call 2 * block + 1
      const uint64_t blk = (uint64_t)(c0 + h) * (uint64_t)(rows / 16) + (uint64_t)g;  // COL-major
      sr_values8(col[h], sr_call(2 * blk, seed, offset, rounds));
      sr_values8(col[h] + 8, sr_call(2 * blk + 1, seed, offset, rounds));
    }
  }
  // RNE, or (after stochastic rounding) the exact conversion of grid values.
#pragma unroll
  for (int r = 0; r < 16; r++)
    code[r] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, col[0][r], col[1][r], 1.0f, 0) & 0xFFu;
  return sc;
}

// The largest |value| of the pair's 32 elements, after the transform's
// butterflies (unscaled: the caller multiplies the maximum by 1/4) when rht.
template <typename T, bool kRHT>
__device__ __forceinline__ float col_pair_max(const RawPair<T> (&raw)[16], uint32_t mask) {
  float col[2][16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    RawPair<T> t = raw[r];  // the caller's words stay as loaded
    if (kRHT) t.flip((mask >> r) & 1u);
    t.get(col[0][r], col[1][r]);
  }
  float m = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    if (kRHT) hadamard16_unscaled(col[h]);
#pragma unroll
    for (int r = 0; r < 16; r++) m = fmaxf(m, __builtin_fabsf(col[h][r]));
  }
  return m;
}

// COL quantizer kernel: one lane per column pair and block row (2 blocks
// of 16 rows), whose 16 raw rows are one word (bf16) or two (fp32) each.
// With 8 columns per lane, a rolled loop over the column pairs has to pick
// each pair's words out of the row's four (selects or rotations, about a
// quarter of the loop's instructions); with one pair per lane there is
// nothing to pick, the raw rows take 16 registers instead of 64, and
// every load and store is still coalesced (consecutive lanes read
// consecutive words of a row and write consecutive code bytes).  A
// workgroup takes 256 column pairs of one block row, so that its 16 rows
// (and their 16 code rows) sit in one buffer resource based at the block
// row: the lane's column in the vector offset, the row step in the scalar
// one, no address arithmetic per row (rows up to 2^25 bytes wide; wider
// ones, and gathered rows, are addressed by pointer).
// kZeros: also the number of zero-magnitude codes written, as in
// quant_row_kernel.
template <typename T, bool kSR, bool kRHT, bool kGather = false, bool kZeros = false>
__global__ __launch_bounds__(kThreads) void quant_col_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ amax,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec,
    uint32_t mask, uint64_t seed, uint64_t offset, uint32_t rounds, RowSrc<kGather> rs = {},
    int zslot = 0) {
  __shared__ float rtab[128];
  const TensorScales ts = tensor_scales(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gdec = ts.g;
  const uint32_t per_row = (uint32_t)((cols / 2 + kThreads - 1) / kThreads);  // workgroups per block row
  const int64_t g = blockIdx.x / per_row;                                 // wave-uniform
  const uint32_t cl = ((blockIdx.x % per_row) * kThreads + threadIdx.x) * 2;
  const bool live = cl < cols;
  const uint32_t c0 = live ? cl : (uint32_t)cols - 2;  // idle lanes re-read the last pair
  const int64_t rb = cols * (int64_t)sizeof(T);  // bytes per row
  const bool buf = !kGather && rb <= (1 << 25);
  RawPair<T> raw[16];
  if (buf) {
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(x + g * 16 * cols), 0, (int)(16 * rb), kBufFlags);
#pragma unroll
    for (int r = 0; r < 16; r++) raw[r].load_buf(xr, c0 * (uint32_t)sizeof(T), (int)(r * rb));
  } else {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t sr = rs.at(g * 16 + r);  // wave-uniform
      raw[r].load_or_zero(x + (kGather && sr < 0 ? 0 : sr) * cols + c0, !kGather || sr >= 0);
    }
  }
  build_recip_table(rtab, ts.S);
  if (!kZeros && !live) return;  // with kZeros every thread reaches the count
  uint32_t zc = 0;
  if (live) {
    uint32_t code[16];
    const uint32_t sc = col_pair_encode<T, kSR, kRHT>(raw, rows, g, c0, ts, rtab, mask, seed,
                                                      offset, rounds, code);
    uint8_t* cp0 = codes + g * 16 * (cols / 2);
    if (buf) {
      const __amdgpu_buffer_rsrc_t cr =
          __builtin_amdgcn_make_buffer_rsrc(cp0, 0, (int)(8 * cols), kBufFlags);
#pragma unroll
      for (int r = 0; r < 16; r++)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code[r], cr, c0 / 2, (int)(r * (cols / 2)),
                                             0);
    } else {
#pragma unroll
      for (int r = 0; r < 16; r++) cp0[r * (cols / 2) + c0 / 2] = (uint8_t)code[r];
    }
    *reinterpret_cast<uint16_t*>(scales + g * cols + c0) = (uint16_t)sc;
    if (kZeros)
#pragma unroll
      for (int q = 0; q < 4; q++)  // 4 rows of 2 codes per word
        zc += zero_nibbles((code[4 * q] & 0xFFu) | ((code[4 * q + 1] & 0xFFu) << 8) |
                           ((code[4 * q + 2] & 0xFFu) << 16) | ((code[4 * q + 3] & 0xFFu) << 24));
  }
  if constexpr (kZeros) grid_zero_count(zc, zslot);
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

// The same for bf16, a workgroup per 256 units of one block row: its 16 rows
// (and their 16 code rows) sit in one buffer resource based at the block
// row, the lane's column in the vector offset and the row step in the scalar
// one, so no address arithmetic runs per row; the rows stay raw words (64
// registers instead of 128 floats) until the encode converts them.  Lanes
// past the row's end read zeros and store nothing.  Rows up to 2^26 bytes
// wide (16 of them in one 31-bit range).
__global__ __launch_bounds__(kThreads) void quant_2d_bf16_kernel(
    const uint16_t* __restrict__ w, int64_t rows, int64_t cols, const float* __restrict__ amax,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gdec) {
  __shared__ float rtab[128];
  const int64_t slice = blockIdx.y;
  const TensorScales ts = tensor_scales(amax[slice]);
  if (blockIdx.x == 0 && threadIdx.x == 0) gdec[slice] = ts.g;
  const uint32_t cg = (uint32_t)(cols / 8);  // units per block row: even (pairs agree)
  const uint32_t per_row = (cg + kThreads - 1) / kThreads;
  const int64_t g = slice * (rows / 16) + blockIdx.x / per_row;  // block row (wave-uniform)
  const uint32_t cu = (blockIdx.x % per_row) * kThreads + threadIdx.x;
  const bool live = cu < cg;
  const int rb = (int)(cols * 2);  // bytes per row
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + g * 16 * cols), 0, 16 * rb, kBufFlags);
  const uint32_t voff = live ? cu * 16 : kDropOff;
  uint4 q[16];
#pragma unroll
  for (int r = 0; r < 16; r++)
    q[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, r * rb, 0));
  float bm = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) bm = fmaxf(bm, max8_bf16_bits(q[r]));
  bm = fmaxf(bm, xor1(bm));
  build_recip_table(rtab, ts.S);
  if (!live) return;
  const uint32_t e = block_code(bm, ts.k);
  const float rcp = rtab[e];
  const int cb = (int)(cols / 2);  // code bytes per row
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(codes + g * 16 * cb, 0, 16 * cb, kBufFlags);
#pragma unroll
  for (int r = 0; r < 16; r++) {
    float v[8], y[8];
    RawRow<uint16_t>{q[r]}.all(v);
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = v[k] * rcp;
    __builtin_amdgcn_raw_buffer_store_b32(pack8_rne(y), cr, cu * 4, r * cb, 0);
  }
  if ((cu & 1) == 0) scales[g * (cols / 16) + cu / 2] = (uint8_t)e;
}

// ---- single-pass quantizers (tensor amax and encode in one launch) -------------------------
// A bf16 tensor is read once as far as the registers of one workgroup per CU
// hold it: every thread loads its share and keeps it, the workgroups combine
// their maxima through a grid barrier, then every thread encodes what it
// holds, exactly as the two-pass kernels do (same block codes, reciprocal
// table, rounding and Philox calls), so the outputs are bit-identical.  What
// does not fit is read twice, once for the maximum before the barrier and
// once to be encoded after it, which still reads less than two passes.  The grid is one
// workgroup per CU, and a workgroup fills a CU's registers (kSpThreads
// threads, up to 256 VGPRs each), so on an otherwise idle device all of them
// are resident at once.  When they are not (another kernel holds CUs, e.g.
// from a concurrent stream), the barrier's wait is bounded by wait_ticks of
// the 100 MHz real-time counter: a workgroup that gives up takes the tensor
// maximum by reading the whole tensor itself, which is slow but gives the
// same value, so the results stay exact and no wait can last.
constexpr int kSpThreads = 512;
constexpr int kSpRowHold = 48;    // 16-byte chunks (8 bf16) held per thread: 192 VGPRs
constexpr int kSpRowHoldSr = 42;  // the same with stochastic rounding (its encode needs more)
constexpr int kSp2dHold = 3;      // 16 x 8 bf16 units held per thread: 192 VGPRs
constexpr int kSpColHold = 8;     // COL column-pair units (16 rows x 2 bf16) held per thread
constexpr int kSpColStream = 4;   // COL units in flight per thread in the rounds read twice
constexpr int kSpStream = 8;      // chunks in flight per thread in the rounds read twice
constexpr int64_t kSpMaxBytes = int64_t(1) << 30;  // single pass up to 1 GiB of bf16 (31-bit offsets)

// Max of |x| over n16 16-byte chunks of bf16 by the whole workgroup (the
// fallback of a workgroup that gave up waiting at a barrier).  Kept out of
// line and small: the kernels' registers stay live across the call.
__device__ __noinline__ float own_tensor_max(const uint16_t* x, int64_t n16) {
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x)
    m = fmaxf(m, max8_bf16_bits(*reinterpret_cast<const uint4*>(x + i * 8)));
  float m1 = 0.0f;
  block_max2(m, m1);
  return m;  // valid in thread 0
}

// The same fallback for COL blocks with the transform over a [rows x cols]
// bf16 tensor: the maximum the COL amax pass takes (after the butterflies,
// times 1/4).
__device__ __noinline__ float own_col_rht_max(const uint16_t* x, int64_t rows, int64_t cols,
                                              uint32_t mask) {
  float m = 0.0f;
  const int64_t cp = cols / 2, units = (rows / 16) * cp;
  for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
    const int64_t g = u / cp, c0 = (u % cp) * 2;
    float col[2][16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(x + (g * 16 + r) * cols + c0);
      w ^= ((mask >> r) & 1u) ? 0x80008000u : 0u;
      col[0][r] = __uint_as_float(w << 16);
      col[1][r] = __uint_as_float(w & 0xFFFF0000u);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      hadamard16_unscaled(col[h]);
#pragma unroll
      for (int r = 0; r < 16; r++) m = fmaxf(m, __builtin_fabsf(col[h][r]));
    }
  }
  float m1 = 0.0f;
  block_max2(m, m1);
  return m * 0.25f;  // valid in thread 0
}

// What a workgroup that gave up waiting at a barrier reads to take the
// tensor maximum itself: max |x| over n16 16-byte chunks of bf16, or (for
// kColRht) the COL-with-transform maximum of the [rows x cols] tensor x.
struct MaxSource {
  const uint16_t* x;
  int64_t n16;
  int64_t rows, cols;
  uint32_t mask;
};

// The grid barrier is a board: one 8-byte entry per workgroup, holding
// (epoch << 32) | the workgroup's maximum (fp32 bits), written with a single
// store; every workgroup then reads all the entries until each carries the
// call's epoch, and takes the largest maximum.  No read-modify-write atomics
// (same-address atomics serialize) and nothing to clear: the host gives each
// call a board (round robin over kSlots) and an epoch that no earlier use of
// that board had, so entries left by earlier calls never match.  Relaxed
// device-scope loads and stores are coherent across the XCDs on their own.
constexpr int kBoardMax = 256;  // workgroups (one per CU) a board holds
__device__ unsigned long long g_board[kSlots][kBoardMax];

// Tensor amax from the maxima m of the n workgroups sharing board[0 .. n)
// (this one is entry me; all threads call it, the result is returned to
// all).  Wave 0 polls the board, bounded by wait_ticks of the real-time
// counter and, independently of it, by a poll count (s_sleep 2 between
// polls: at least 0.05 us each).  src: what a workgroup that gives up reads
// for the maximum itself.
template <bool kColRht = false>
__device__ __forceinline__ float board_amax(float m, unsigned long long* board, unsigned int n,
                                            unsigned int me, uint32_t epoch, const MaxSource& src,
                                            uint64_t wait_ticks) {
  __shared__ float bcast;
  __shared__ int late;
  float m1 = 0.0f;
  block_max2(m, m1);
  if (threadIdx.x == 0)
    __hip_atomic_store(&board[me], ((unsigned long long)epoch << 32) | __float_as_uint(m),
                       __ATOMIC_RELAXED, kAgent);
  if (threadIdx.x < 64) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t max_polls = wait_ticks * 20 + 1;
    uint64_t polls = 0;
    unsigned int mx;
    bool ok = true;
    for (;;) {
      // All of a lane's loads in flight at once (indices past the grid
      // re-read the last entry).
      unsigned long long e[kBoardMax / 64];
#pragma unroll
      for (int j = 0; j < kBoardMax / 64; j++) {
        const unsigned int k = threadIdx.x + 64u * j;
        e[j] = __hip_atomic_load(&board[k < n ? k : n - 1], __ATOMIC_RELAXED, kAgent);
      }
      bool ready = true;
      mx = 0;
#pragma unroll
      for (int j = 0; j < kBoardMax / 64; j++) {
        ready = ready && (unsigned int)(e[j] >> 32) == epoch;
        mx = mx > (unsigned int)e[j] ? mx : (unsigned int)e[j];
      }
      if (__all(ready)) break;  // wave-uniform
      if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks || ++polls > max_polls) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned int other = (unsigned int)__shfl_xor((int)mx, o);
      mx = mx > other ? mx : other;
    }
    if (threadIdx.x == 0) {
      bcast = __uint_as_float(mx);
      late = ok ? 0 : 1;
    }
  }
  __syncthreads();
  const bool gave_up = late;  // workgroup-uniform
  float a = bcast;
  if (gave_up) {
    if constexpr (kColRht)
      a = own_col_rht_max(src.x, src.rows, src.cols, src.mask);
    else
      a = own_tensor_max(src.x, src.n16);
  }
  __syncthreads();  // every read of bcast and late is done before a later call writes them
  if (!gave_up) return a;
  if (threadIdx.x == 0) bcast = a;
  __syncthreads();
  const float r = bcast;
  __syncthreads();
  return r;
}

// The whole grid's tensor amax (one workgroup per board entry).
__device__ __forceinline__ float grid_amax(float m, int slot, uint32_t epoch, const uint16_t* x,
                                           int64_t n16, uint64_t wait_ticks) {
  return board_amax(m, g_board[slot], gridDim.x, blockIdx.x, epoch,
                    MaxSource{x, n16, 0, 0, 0u}, wait_ticks);
}

// The caller's amax and g, from workgroup 0 (every workgroup holds the same
// tensor maximum).
__device__ __forceinline__ void grid_outputs(float A, float* amax_out, float* gdec) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *amax_out = A;
    *gdec = tensor_scales(A).g;
  }
}

// ROW blocks.  Thread t of the grid (P threads) takes chunks t + j P
// (consecutive lanes: consecutive 16-byte chunks; lanes 2t and 2t+1 hold the
// two halves of a block, as in quant_row_kernel).  Loads and stores go
// through buffer resources sized to the tensor: the per-lane part of an
// offset is the thread's, the per-round part (j P) a wave-uniform scalar, so
// no per-round address stays live in vector registers; chunks past the end
// read zeros and their stores are dropped by the range check.  The tensor is
// at most kSpMaxBytes here, so the byte offsets fit 31 bits, also for the
// rounds past the end that a streamed batch reads (kSpStream rounds further
// at most).

// Thread t takes the chunks of rounds j < J = ceil(chunks / P): rounds j < H
// (kSpRowHold, or kSpRowHoldSr with stochastic rounding, whose encode needs
// more registers) are loaded once and kept; rounds H .. J-1, when there are
// more, are streamed first, before the held rounds are loaded, for their
// maximum only, and again after the barrier to be encoded.  Block maxima of
// the held rounds are taken before the barrier and kept in LDS as bf16 bits
// (a block's maximum is one of its bf16 values), two rounds per word; each
// thread reads back only its own words.  With stochastic rounding chunk i
// draws Philox call i, as in quant_row_kernel.
template <bool kSR>
__global__ __launch_bounds__(kSpThreads) void quant_row_1pass_kernel(
    const uint16_t* __restrict__ x, int64_t chunks, int slot, uint32_t epoch,
    float* __restrict__ amax_out, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ gdec, uint64_t seed, uint64_t offset, uint32_t rounds,
    uint64_t wait_ticks) {
  constexpr int H = kSR ? kSpRowHoldSr : kSpRowHold;
  static_assert(H % 2 == 0, "rounds pair up in the LDS words");
  __shared__ float rtab[128];
  __shared__ uint32_t bmax[H / 2][kSpThreads];
  const uint32_t P = gridDim.x * kSpThreads;
  const uint32_t J = (uint32_t)((chunks + P - 1) / P);  // rounds (wave-uniform)
  const uint32_t wg0 = blockIdx.x * kSpThreads;          // first chunk of the workgroup, round 0
  const uint32_t tid = threadIdx.x;
  const int odd = (int)(tid & 1);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), 0, (int)(chunks * 16), kBufFlags);
  auto load = [&](uint32_t j) {  // round j's chunk (past the end: zeros)
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         xr, tid * 16, (int)((wg0 + j * P) * 16), 0));
  };
  float m = 0.0f;
  for (uint32_t j0 = H; j0 < J; j0 += kSpStream) {  // the rounds read twice: maximum
    uint4 sq[kSpStream];
#pragma unroll
    for (int k = 0; k < kSpStream; k++) sq[k] = load(j0 + k);
#pragma unroll
    for (int k = 0; k < kSpStream; k++) m = fmaxf(m, max8_bf16_bits(sq[k]));
  }
  uint4 q[H];
#pragma unroll
  for (int j = 0; j < H; j++) q[j] = load(j);
#pragma unroll
  for (int j = 0; j < H; j += 2) {
    const float c0 = max8_bf16_bits(q[j]), c1 = max8_bf16_bits(q[j + 1]);
    const float b0 = fmaxf(c0, xor1(c0)), b1 = fmaxf(c1, xor1(c1));
    bmax[j / 2][tid] = (__float_as_uint(b0) >> 16) | (__float_as_uint(b1) & 0xFFFF0000u);
    m = fmaxf(m, fmaxf(b0, b1));
  }
  const float A = grid_amax(m, slot, epoch, x, chunks, wait_ticks);
  grid_outputs(A, amax_out, gdec);
  const TensorScales ts = tensor_scales(A);
  build_recip_table(rtab, ts.S);
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(codes, 0, (int)(chunks * 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t sr =
      __builtin_amdgcn_make_buffer_rsrc(scales, 0, (int)(chunks / 2), kBufFlags);
  const uint32_t s_off = odd ? kDropOff : tid / 2;  // even lanes store the block's scale
  // Encode round j's chunk v (8 values) with its block's maximum bm.
  auto encode = [&](uint32_t j, const uint4& qq, float bm) {
    const uint32_t base = wg0 + j * P;  // wave-uniform
    const uint32_t e = block_code(bm, ts.k);
    const float r = rtab[e];
    float v[8], y[8];
    RawRow<uint16_t>{qq}.all(v);
#pragma unroll
    for (int u = 0; u < 8; u++) y[u] = v[u] * r;
    if (kSR) sr_values8(y, sr_call((uint64_t)(base + tid), seed, offset, rounds));
    __builtin_amdgcn_raw_buffer_store_b32(pack8_rne(y), cr, tid * 4, (int)(base * 4), 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)e, sr, s_off, (int)(base / 2), 0);
  };
#pragma unroll
  for (int j = 0; j < H; j++) {
    const uint32_t bw = bmax[j / 2][tid];
    encode(j, q[j], __uint_as_float((j & 1) ? (bw & 0xFFFF0000u) : (bw << 16)));
  }
  for (uint32_t j0 = H; j0 < J; j0 += kSpStream) {  // the rounds read twice: encode
    uint4 sq[kSpStream];
#pragma unroll
    for (int k = 0; k < kSpStream; k++) sq[k] = load(j0 + k);
#pragma unroll
    for (int k = 0; k < kSpStream; k++) {
      const float c = max8_bf16_bits(sq[k]);
      encode(j0 + k, sq[k], fmaxf(c, xor1(c)));  // past the end: zeros, stores dropped
    }
  }
}

// The units of a single pass over n workgroups of kSpThreads threads.
// Whole rounds go over the grid as one stream (unit t + j P for grid thread
// t, P = n kSpThreads: concurrent loads cover one contiguous span).  The
// partial last round, when there is one, is split evenly: each workgroup
// takes `per` consecutive units of it (ceil(rem / n), rounded up to even so
// that the two lanes of a block agree), on its first `per` threads.  Handing
// the partial round out as the whole ones left it to the first workgroups
// only (a [6144 x 6144] matrix is 2.25 rounds: 64 CUs loaded 3 units per
// thread, 192 loaded 2), and a pass runs at the pace of its busiest CUs.
// Giving every workgroup one contiguous range of the whole tensor instead
// made the [8192 x 8192] pass slower (51.7 -> 58.5 us): 256 concurrent
// streams 512 KB apart.  unit() is false where the round has no unit for
// the thread (the caller then loads zeros and stores nothing).  Unit
// indices fit 32 bits: a matrix here is at most kSpMaxBytes.
struct SpShare {
  uint32_t units, P, full, tail0, per, b;
  __device__ SpShare(uint32_t units_, uint32_t n, uint32_t b_) : units(units_), b(b_) {
    P = n * kSpThreads;
    full = units_ / P;
    tail0 = full * P;
    per = ((units_ - tail0 + n - 1) / n + 1) & ~1u;
  }
  __device__ uint32_t rounds() const { return full + (tail0 < units ? 1u : 0u); }
  __device__ bool unit(uint32_t j, uint32_t t, uint32_t& u) const {
    if (j < full) {
      u = b * kSpThreads + t + j * P;
      return true;
    }
    u = tail0 + b * per + t;
    return j == full && t < per && u < units;
  }
};

// 16x16 blocks of one bf16 matrix.  Units are 16 rows x 8 columns, as in
// quant_2d_kernel (lanes 2t and 2t+1 hold the two halves of a block), handed
// out in rounds as SpShare says: rounds j < kSp2dHold are held, later ones
// (when there are more) are streamed for the maximum first and read again
// after the barrier, as in the ROW kernel.
__global__ __launch_bounds__(kSpThreads) void quant_2d_1pass_kernel(
    const uint16_t* __restrict__ w, int64_t rows, int64_t cols, int slot, uint32_t epoch,
    float* __restrict__ amax_out, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ gdec, uint64_t wait_ticks) {
  __shared__ float rtab[128];
  // At most kSpMaxBytes: unit indices and byte offsets fit 32 bits.  Loads
  // and stores go through buffer resources: the unit's first row in the
  // vector offset, the row step (wave-uniform) in the scalar one; a unit
  // past the end gets an offset past the range (loads read zeros).
  const uint32_t cols32 = (uint32_t)cols;
  const uint32_t cg = cols32 / 8;  // a multiple of 4: pairs never straddle rows
  const uint32_t units = (uint32_t)(rows / 16) * cg;
  const SpShare sh(units, gridDim.x, blockIdx.x);
  const uint32_t J = sh.rounds();  // wave-uniform
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w), 0, (int)(rows * cols * 2), kBufFlags);
  // Row block g and first column c0 of the thread's unit of round j; false
  // when the round has no unit for the thread.
  auto unit_at = [&](uint32_t j, uint32_t& g, uint32_t& c0) {
    uint32_t u;
    const bool ok = sh.unit(j, threadIdx.x, u);
    g = u / cg;
    c0 = (u - g * cg) * 8;
    return ok;
  };
  auto load_unit = [&](uint32_t j, uint4 (&qq)[16]) {  // past the end: zeros
    uint32_t g, c0;
    const bool ok = unit_at(j, g, c0);
    const uint32_t voff = ok ? (g * 16 * cols32 + c0) * 2 : kDropOff;
#pragma unroll
    for (int r = 0; r < 16; r++)
      qq[r] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, (int)(r * cols32 * 2), 0));
  };
  auto unit_max = [&](const uint4 (&qq)[16]) {  // the block's maximum (both lanes)
    float bm = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) bm = fmaxf(bm, max8_bf16_bits(qq[r]));
    return fmaxf(bm, xor1(bm));
  };
  float m = 0.0f;
  for (uint32_t j = kSp2dHold; j < J; j++) {  // the rounds read twice: maximum
    uint4 sq[16];
    load_unit(j, sq);
    m = fmaxf(m, unit_max(sq));
  }
  uint4 q[kSp2dHold][16];
#pragma unroll
  for (int j = 0; j < kSp2dHold; j++) load_unit(j, q[j]);
  // Block maxima before the barrier, kept in LDS (each thread reads back
  // only its own entries).
  __shared__ float bmax[kSp2dHold][kSpThreads];
#pragma unroll
  for (int j = 0; j < kSp2dHold; j++) {
    const float bm = unit_max(q[j]);
    bmax[j][threadIdx.x] = bm;
    m = fmaxf(m, bm);
  }
  const float A = grid_amax(m, slot, epoch, w, rows * cols / 8, wait_ticks);
  grid_outputs(A, amax_out, gdec);
  const TensorScales ts = tensor_scales(A);
  build_recip_table(rtab, ts.S);
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(codes, 0, (int)(rows * cols / 2), kBufFlags);
  auto encode = [&](uint32_t j, const uint4 (&qq)[16], float bm) {
    uint32_t g, c0;
    if (!unit_at(j, g, c0)) return;  // share and units are even: the lanes of a pair agree
    const uint32_t e = block_code(bm, ts.k);
    const float rcp = rtab[e];
    const uint32_t voff = g * 16 * (cols32 / 2) + c0 / 2;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      float v[8], y[8];
      RawRow<uint16_t>{qq[r]}.all(v);
#pragma unroll
      for (int k = 0; k < 8; k++) y[k] = v[k] * rcp;
      __builtin_amdgcn_raw_buffer_store_b32(pack8_rne(y), cr, voff, (int)(r * (cols32 / 2)), 0);
    }
    if ((c0 & 8) == 0) scales[g * (cols32 / 16) + c0 / 16] = (uint8_t)e;
  };
#pragma unroll
  for (int j = 0; j < kSp2dHold; j++) encode(j, q[j], bmax[j][threadIdx.x]);
  for (uint32_t j = kSp2dHold; j < J; j++) {  // the rounds read twice: encode
    uint4 sq[16];
    load_unit(j, sq);
    encode(j, sq, unit_max(sq));
  }
}

// 16x16 blocks of a batch of bf16 matrices (the routed experts' weights),
// each with its own amax, in one pass.  The grid (one workgroup per CU) is
// split into `groups` groups of gridDim.x / groups workgroups, each large
// enough to hold one matrix in its registers (streamed rounds as above when
// it is not); group k quantizes matrices k, k + groups, k + 2 groups, ...
// exactly as quant_2d_1pass_kernel quantizes one: load and hold, the
// matrix's maximum through the group's own barrier, encode.  Round i of a
// group (its i-th matrix) uses board i % 2 of the call and epoch epoch + i:
// a workgroup can only write round i + 2's entry after every workgroup of
// its group has written round i + 1's, i.e. after all of them have read
// round i's, so two boards suffice.  Workgroups past the groups idle.
__device__ unsigned long long g_board2[kSlots][2][kBoardMax];

__global__ __launch_bounds__(kSpThreads) void quant_2d_batch_1pass_kernel(
    const uint16_t* __restrict__ w, int64_t batch, int64_t rows, int64_t cols, uint32_t groups,
    int slot, uint32_t epoch, float* __restrict__ amax_out, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gdec, uint64_t wait_ticks) {
  __shared__ float rtab[128];
  __shared__ float bmax[kSp2dHold][kSpThreads];
  const uint32_t gsz = gridDim.x / groups;  // workgroups per group
  const uint32_t grp = blockIdx.x / gsz;
  if (grp >= groups) return;  // workgroup-uniform
  const uint32_t me = blockIdx.x - grp * gsz;
  // Per matrix at most kSpMaxBytes: unit indices and byte offsets fit 32
  // bits; each matrix gets buffer resources based at its first element.
  const uint32_t cols32 = (uint32_t)cols;
  const uint32_t cg = cols32 / 8;  // a multiple of 4: pairs never straddle rows
  const uint32_t units = (uint32_t)(rows / 16) * cg;
  const SpShare sh(units, gsz, me);  // the group's workgroups share a matrix
  const uint32_t J = sh.rounds();      // rounds per matrix (wave-uniform)
  const int64_t mat = rows * cols;
  auto unit_at = [&](uint32_t j, uint32_t& g, uint32_t& c0) {
    uint32_t u;
    const bool ok = sh.unit(j, threadIdx.x, u);
    g = u / cg;
    c0 = (u - g * cg) * 8;
    return ok;
  };
  auto unit_max = [&](const uint4 (&qq)[16]) {  // the block's maximum (both lanes)
    float bm = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) bm = fmaxf(bm, max8_bf16_bits(qq[r]));
    return fmaxf(bm, xor1(bm));
  };
  uint32_t round = 0;
  for (int64_t b = grp; b < batch; b += groups, round++) {
    const uint16_t* wb = w + b * mat;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wb), 0, (int)(mat * 2), kBufFlags);
    auto load_unit = [&](uint32_t j, uint4 (&qq)[16]) {  // past the end: zeros
      uint32_t g, c0;
      const bool ok = unit_at(j, g, c0);
      const uint32_t voff = ok ? (g * 16 * cols32 + c0) * 2 : kDropOff;
#pragma unroll
      for (int r = 0; r < 16; r++)
        qq[r] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, (int)(r * cols32 * 2), 0));
    };
    float m = 0.0f;
    for (uint32_t j = kSp2dHold; j < J; j++) {  // the rounds read twice: maximum
      uint4 sq[16];
      load_unit(j, sq);
      m = fmaxf(m, unit_max(sq));
    }
    uint4 q[kSp2dHold][16];
#pragma unroll
    for (int j = 0; j < kSp2dHold; j++) load_unit(j, q[j]);
#pragma unroll
    for (int j = 0; j < kSp2dHold; j++) {
      const float bm = unit_max(q[j]);
      bmax[j][threadIdx.x] = bm;
      m = fmaxf(m, bm);
    }
    const float A = board_amax(m, g_board2[slot][round & 1] + grp * gsz, gsz, me, epoch + round,
                               MaxSource{wb, mat / 8, 0, 0, 0u}, wait_ticks);
    if (me == 0 && threadIdx.x == 0) {
      amax_out[b] = A;
      gdec[b] = tensor_scales(A).g;
    }
    const TensorScales ts = tensor_scales(A);
    build_recip_table(rtab, ts.S);
    uint8_t* cb = codes + b * (mat / 2);
    uint8_t* sb = scales + b * (mat / 256);
    const __amdgpu_buffer_rsrc_t cr =
        __builtin_amdgcn_make_buffer_rsrc(cb, 0, (int)(mat / 2), kBufFlags);
    auto encode = [&](uint32_t j, const uint4 (&qq)[16], float bm) {
      uint32_t g, c0;
      if (!unit_at(j, g, c0)) return;  // share and units are even: the lanes of a pair agree
      const uint32_t e = block_code(bm, ts.k);
      const float rcp = rtab[e];
      const uint32_t voff = g * 16 * (cols32 / 2) + c0 / 2;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float v[8], y[8];
        RawRow<uint16_t>{qq[r]}.all(v);
#pragma unroll
        for (int k = 0; k < 8; k++) y[k] = v[k] * rcp;
        __builtin_amdgcn_raw_buffer_store_b32(pack8_rne(y), cr, voff, (int)(r * (cols32 / 2)), 0);
      }
      if ((c0 & 8) == 0) sb[g * (cols32 / 16) + c0 / 16] = (uint8_t)e;
    };
#pragma unroll
    for (int j = 0; j < kSp2dHold; j++) encode(j, q[j], bmax[j][threadIdx.x]);
    for (uint32_t j = kSp2dHold; j < J; j++) {  // the rounds read twice: encode
      uint4 sq[16];
      load_unit(j, sq);
      encode(j, sq, unit_max(sq));
    }
  }
}

// COL blocks (16 x 1, with or without the transform, RNE) of one bf16 matrix.
// Column-pair units (16 rows x 2 columns, as in quant_col_kernel) are handed
// out in rounds as SpShare says: rounds j < kSpColHold are held, later ones are
// streamed (kSpColStream units in flight) for the maximum first and read
// again after the barrier.  The maximum is
// taken after the transform's butterflies (times 1/4 at the end, as the COL
// amax pass does); a workgroup that gives up at the barrier takes it the
// same way from the whole tensor.  Then every held unit is encoded exactly
// as quant_col_kernel encodes it (the transform computed again).
template <bool kRHT>
__global__ __launch_bounds__(kSpThreads) void quant_col_1pass_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint32_t mask, int slot,
    uint32_t epoch, float* __restrict__ amax_out, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gdec, uint64_t wait_ticks) {
  constexpr int H = kSpColHold;
  __shared__ float rtab[128];
  // At most kSpMaxBytes: unit indices and byte offsets fit 32 bits.  Loads
  // and stores go through buffer resources: the unit's first row in the
  // vector offset, the row step (wave-uniform) in the scalar one; a unit
  // past the end gets an offset past the range (loads read zeros, stores
  // are dropped).
  const uint32_t cols32 = (uint32_t)cols;
  const uint32_t cp = cols32 / 2;
  const uint32_t units = (uint32_t)(rows / 16) * cp;
  const SpShare sh(units, gridDim.x, blockIdx.x);
  const uint32_t J = sh.rounds();  // wave-uniform
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), 0, (int)(rows * cols * 2), kBufFlags);
  auto unit_at = [&](uint32_t j, uint32_t& g, uint32_t& c0) {
    uint32_t u;
    const bool ok = sh.unit(j, threadIdx.x, u);
    g = u / cp;
    c0 = (u - g * cp) * 2;
    return ok;
  };
  auto load_unit = [&](uint32_t j, RawPair<uint16_t> (&raw)[16])
                       __attribute__((always_inline)) {  // past the end: zeros
    uint32_t g, c0;
    const bool ok = unit_at(j, g, c0);
    const uint32_t voff = ok ? (g * 16 * cols32 + c0) * 2 : kDropOff;
#pragma unroll
    for (int r = 0; r < 16; r++) raw[r].load_buf(xr, voff, (int)(r * cols32 * 2));
  };
  float m = 0.0f;
  for (uint32_t j0 = H; j0 < J; j0 += kSpColStream) {  // the rounds read twice: maximum
    RawPair<uint16_t> sq[kSpColStream][16];
#pragma unroll
    for (int k = 0; k < kSpColStream; k++) load_unit(j0 + k, sq[k]);  // past the end: zeros
#pragma unroll
    for (int k = 0; k < kSpColStream; k++) m = fmaxf(m, col_pair_max<uint16_t, kRHT>(sq[k], mask));
  }
  RawPair<uint16_t> q[H][16];
#pragma unroll
  for (int j = 0; j < H; j++) load_unit(j, q[j]);
  // (One unit at a time: the scheduler would otherwise interleave the units'
  // transforms and run out of registers.)
#pragma unroll
  for (int j = 0; j < H; j++) {
    m = fmaxf(m, col_pair_max<uint16_t, kRHT>(q[j], mask));
    __builtin_amdgcn_sched_barrier(0);
  }
  const float A =
      board_amax<kRHT>(kRHT ? m * 0.25f : m, g_board[slot], gridDim.x, blockIdx.x, epoch,
                       MaxSource{x, rows * cols / 8, rows, cols, mask}, wait_ticks);
  grid_outputs(A, amax_out, gdec);
  const TensorScales ts = tensor_scales(A);
  build_recip_table(rtab, ts.S);
  // The encode computes the transform again from the held words.  Kept
  // opaque to the compiler, which would otherwise keep the maximum pass's
  // transformed values (fp32: twice the registers of the words) across the
  // barrier and spill them.
#pragma unroll
  for (int j = 0; j < H; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) __asm__ volatile("" : "+v"(q[j][r].w));
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(codes, 0, (int)(rows * cols / 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t sr =
      __builtin_amdgcn_make_buffer_rsrc(scales, 0, (int)(rows / 16 * cols), kBufFlags);
  auto encode = [&](uint32_t j, RawPair<uint16_t> (&raw)[16]) __attribute__((always_inline)) {
    uint32_t g, c0;
    const bool ok = unit_at(j, g, c0);
    uint32_t code[16];
    const uint32_t sc =
        col_pair_encode<uint16_t, false, kRHT>(raw, rows, g, c0, ts, rtab, mask, 0, 0, 0, code);
    const uint32_t voff = ok ? g * 16 * cp + c0 / 2 : kDropOff;
#pragma unroll
    for (int r = 0; r < 16; r++)
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code[r], cr, voff, (int)(r * cp), 0);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sc, sr, ok ? g * cols32 + c0 : kDropOff, 0,
                                          0);
  };
#pragma unroll
  for (int j = 0; j < H; j++) {
    encode(j, q[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (uint32_t j = H; j < J; j++) {  // the rounds read twice: encode
    RawPair<uint16_t> sq[16];
    load_unit(j, sq);
    encode(j, sq);
  }
}

// ---- debug check: non-finite inputs -----------------------------------------------------------
// One flag per call slot, set when any element of the tensor is an infinity
// or a NaN (exponent bits all ones).  The host reads the flag after the
// kernel and clears it again; only the entry points' debug mode runs this.
__device__ unsigned int g_nonfinite[kSlots];

template <typename T>
__global__ __launch_bounds__(kThreads) void nonfinite_kernel(const uint4* __restrict__ x,
                                                             int64_t chunks,
                                                             unsigned int* __restrict__ flag) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks; i += stride) {
    const uint4 q = x[i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      if (std::is_same<T, float>::value) {
        bad = bad || (w[k] & 0x7F800000u) == 0x7F800000u;
      } else {
        bad = bad || (w[k] & 0x7F80u) == 0x7F80u || (w[k] & 0x7F800000u) == 0x7F800000u;
      }
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
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

// The next scratch slot (round robin over kSlots).
// How long a single-pass kernel's workgroups wait at the grid barrier before
// each takes the tensor maximum on its own, in microseconds; negative: the
// single-pass kernels are not used.
std::atomic<int> g_single_pass_wait_us{2000};

int next_slot() {
  static std::atomic<unsigned int> counter{0};
  return (int)(counter.fetch_add(1u, std::memory_order_relaxed) % kSlots);
}

// The next board of the single-pass kernels (round robin over kSlots) and
// its epoch: 1 + the number of earlier uses of that board, so never 0 (the
// value of an unused entry) and never a value an earlier call left there.
struct Board {
  int slot;
  uint32_t epoch;
};
Board next_board() {
  static std::atomic<unsigned long long> counter{0};
  const unsigned long long c = counter.fetch_add(1u, std::memory_order_relaxed);
  return Board{(int)(c % kSlots), (uint32_t)((c / kSlots) % 0xFFFFFFFFull) + 1u};
}

// The next board pair of the batched single-pass kernel (round robin over
// kSlots) and the first of its `rounds` epochs.  Epochs come from one
// counter for all slots, so no call's epochs repeat an earlier call's (until
// the counter wraps after ~4e9 rounds); never 0, the value of an unused
// entry.  rounds < 2^20.
Board next_batch_board(uint32_t rounds) {
  static std::atomic<unsigned int> calls{0};
  static std::atomic<unsigned long long> epochs{0};
  const int slot = (int)(calls.fetch_add(1u, std::memory_order_relaxed) % kSlots);
  const unsigned long long e = epochs.fetch_add(rounds, std::memory_order_relaxed);
  return Board{slot, (uint32_t)(e % 0xFFF00000ull) + 1u};
}

// Compute units of the current device (the single-pass grid: one workgroup
// per CU), cached per device.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of the COL amax pass with the transform: one per kThreads
// tiles, at most two per CU (the kernel's occupancy), so that every lane
// takes the same number of tiles, give or take one.
unsigned col_amax_grid(int64_t units) {
  const int64_t cus = device_cu_count();
  const int64_t cap = cus > 0 ? 2 * cus : 512;
  const int64_t g = cdiv(units, kThreads);
  return (unsigned)(g < cap ? (g > 0 ? g : 1) : cap);
}

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
  if constexpr (!G && !std::is_same<T, float>::value) {
    // Single pass (the tensor held in the grid's registers as far as they
    // go, the rest read twice): ROW without the transform, and COL with
    // RNE.  (COL with stochastic rounding is ALU-bound: one workgroup per CU
    // hides less of it than the two-pass encode's eight waves per SIMD, and
    // the single pass measured 5% slower.)
    const int64_t chunks = a.rows * a.cols / 8;
    const int cus = device_cu_count();
    const int wait_us = g_single_pass_wait_us.load(std::memory_order_relaxed);
    if (a.axis == kBlockCol && !a.sr && !a.amax_is_input && cus > 0 && cus <= kBoardMax &&
        wait_us >= 0 && chunks * 16 <= kSpMaxBytes) {
      const Board b = next_board();
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
      const uint64_t ticks = (uint64_t)wait_us * 100u;
      if (a.rht)
        quant_col_1pass_kernel<true><<<cus, kSpThreads, 0, st>>>(
            xb, a.rows, a.cols, a.mask, b.slot, b.epoch, a.amax, a.codes, a.scales, a.gdec, ticks);
      else
        quant_col_1pass_kernel<false><<<cus, kSpThreads, 0, st>>>(
            xb, a.rows, a.cols, a.mask, b.slot, b.epoch, a.amax, a.codes, a.scales, a.gdec, ticks);
      return hipGetLastError();
    }
    if (a.axis == kBlockRow && !a.rht && !a.amax_is_input && cus > 0 && cus <= kBoardMax &&
        wait_us >= 0 && chunks * 16 <= kSpMaxBytes) {
      const Board b = next_board();
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
      uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes);
      const uint64_t ticks = (uint64_t)wait_us * 100u;
      if (a.sr)
        quant_row_1pass_kernel<true><<<cus, kSpThreads, 0, st>>>(
            xb, chunks, b.slot, b.epoch, a.amax, cd, a.scales, a.gdec, a.seed, a.offset, a.rounds,
            ticks);
      else
        quant_row_1pass_kernel<false><<<cus, kSpThreads, 0, st>>>(
            xb, chunks, b.slot, b.epoch, a.amax, cd, a.scales, a.gdec, 0, 0, 0, ticks);
      return hipGetLastError();
    }
  }
  if (!a.amax_is_input) {
    const int slot = next_slot();
    if (a.axis == kBlockCol && a.rht) {
      int64_t units = (a.rows / 16) * (a.cols / 8);
      amax_col_rht_kernel<T, false, G>
          <<<col_amax_grid(units), kThreads, 0, st>>>(
              x, a.rows, a.cols, a.mask, a.amax, nullptr, slot, rs);
    } else {
      int64_t chunks = a.rows * a.cols / 8;
      // ROW with the transform needs the pair exchange; COL amax without the
      // transform is the plain max.
      const int u = (!a.x_fp32 && !(a.rht && a.axis == kBlockRow)) ? kAmaxUnroll : 2;
      if (a.rht && a.axis == kBlockRow)
        amax_flat_kernel<T, true, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
            x, chunks, a.mask, a.amax, nullptr, slot, rs, cpr);
      else
        amax_flat_kernel<T, false, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
            x, chunks, 0, a.amax, nullptr, slot, rs, cpr);
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
    int64_t grid64 = (a.rows / 16) * cdiv(a.cols / 2, (int64_t)kThreads);
    if (grid64 > 0x7FFFFFFF) return hipErrorInvalidValue;
    int grid = (int)grid64;
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
  if constexpr (!std::is_same<T, float>::value) {
    // Single pass when one matrix fits in the grid's registers.
    const int64_t units = (a.rows / 16) * (a.cols / 8);
    const int cus = device_cu_count();
    const int wait_us = g_single_pass_wait_us.load(std::memory_order_relaxed);
    if (a.batch == 1 && !a.amax_is_input && cus > 0 && cus <= kBoardMax && wait_us >= 0 &&
        units * 256 <= kSpMaxBytes) {
      const Board b = next_board();
      quant_2d_1pass_kernel<<<cus, kSpThreads, 0, st>>>(
          reinterpret_cast<const uint16_t*>(w), a.rows, a.cols, b.slot, b.epoch, a.amax, a.codes,
          a.scales, a.gdec, (uint64_t)wait_us * 100u);
      return hipGetLastError();
    }
    // A batch: groups of workgroups that each hold one matrix (one group
    // streaming when a matrix needs more than the whole grid).
    if (a.batch > 1 && !a.amax_is_input && cus > 0 && cus <= kBoardMax && wait_us >= 0 &&
        units * 256 <= kSpMaxBytes) {
      const int64_t need = cdiv(units, (int64_t)kSpThreads * kSp2dHold);  // workgroups per matrix
      int64_t groups = need <= cus ? cus / need : 1;
      if (groups > a.batch) groups = a.batch;
      const int64_t rounds = cdiv(a.batch, groups);
      if (rounds < (int64_t(1) << 20)) {
        const Board b = next_batch_board((uint32_t)rounds);
        quant_2d_batch_1pass_kernel<<<cus, kSpThreads, 0, st>>>(
            reinterpret_cast<const uint16_t*>(w), a.batch, a.rows, a.cols, (uint32_t)groups,
            b.slot, b.epoch, a.amax, a.codes, a.scales, a.gdec, (uint64_t)wait_us * 100u);
        return hipGetLastError();
      }
    }
  }
  if (!a.amax_is_input) {
    int64_t chunks = a.rows * a.cols / 8;
    const int u = a.w_fp32 ? 2 : kAmaxUnroll;
    if (a.batch == 1) {
      amax_flat_kernel<T, false><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
          w, chunks, 0, a.amax, nullptr, next_slot());
    } else {  // one maximum per slice: straight into the cleared outputs
      fill_zero_kernel<<<(unsigned)cdiv(a.batch, 256), 256, 0, st>>>(a.amax, a.batch);
      // about 512 workgroups in all, at least one per slice
      const int64_t per = a.batch >= 512 ? 1 : 512 / a.batch;
      dim3 grid((unsigned)amax_grid(chunks, u, per), (unsigned)a.batch);
      amax_flat_kernel<T, false><<<grid, kAmaxThreads, 0, st>>>(w, chunks, 0, a.amax, nullptr, -1);
    }
  }
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (a.cols < (int64_t(1) << 25)) {  // 16 rows of bf16 in a 31-bit range
      const int64_t blocks = (a.rows / 16) * cdiv(a.cols / 8, kThreads);
      if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
      quant_2d_bf16_kernel<<<dim3((unsigned)blocks, (unsigned)a.batch), kThreads, 0, st>>>(
          w, a.rows, a.cols, a.amax, a.codes, a.scales, a.gdec);
      return hipGetLastError();
    }
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
  const int slot = next_slot();
  if (!a.amax_is_input) {
    if (a.rht) {  // transform max for COL, plain max for ROW, one read
      amax_col_rht_kernel<T, true, G>
          <<<col_amax_grid(units), kThreads, 0, st>>>(
              x, a.rows, a.cols, a.mask, a.amax + 1, a.amax, slot, rs);
    } else {  // the same plain max for both
      const int64_t chunks = a.rows * a.cols / 8;
      const int u = a.x_fp32 ? 2 : kAmaxUnroll;
      amax_flat_kernel<T, false, G><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
          x, chunks, 0, a.amax, a.amax + 1, slot, rs, (uint32_t)(a.cols / 8));
    }
  }
  // The two encodes, each as its own 1D quantizer does it (bit-identical to
  // the separate calls), with the maxima of the pass above.  Both are
  // ALU-bound (stochastic rounding, the transform), so a single encode
  // reading x once for both was slower than the two: the saved read is not
  // what bounds them.
  const int64_t chunks = a.rows * a.cols / 8;
  const int grid_r = (int)cdiv(chunks, (int64_t)kThreads * kRowUnroll);
  const int64_t grid_c = (a.rows / 16) * cdiv(a.cols / 2, (int64_t)kThreads);
  if (grid_c > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool z = a.zeros != nullptr;
  const int slot_r = z ? next_slot() : 0, slot_c = z ? next_slot() : 0;
  uint32_t* rc = reinterpret_cast<uint32_t*>(a.row_codes);
  const uint32_t cpr = (uint32_t)(a.cols / 8);
#define NVFP4_DUAL_ROW(Z)                                                                        \
  quant_row_kernel<T, true, false, G, Z><<<grid_r, kThreads, 0, st>>>(                           \
      x, chunks, a.amax, rc, a.row_scales, a.row_gdec, 0, a.seed_r, a.offset_r, a.rounds_r, rs, \
      cpr, slot_r)
#define NVFP4_DUAL_COL(RHT, Z)                                                                  \
  quant_col_kernel<T, true, RHT, G, Z><<<(int)grid_c, kThreads, 0, st>>>(                       \
      x, a.rows, a.cols, a.amax + 1, a.col_codes, a.col_scales, a.col_gdec, a.mask, a.seed_c,   \
      a.offset_c, a.rounds_c, rs, slot_c)
  if (z) {
    NVFP4_DUAL_ROW(true);
    if (a.rht) NVFP4_DUAL_COL(true, true);
    else NVFP4_DUAL_COL(false, true);
  } else {
    NVFP4_DUAL_ROW(false);
    if (a.rht) NVFP4_DUAL_COL(true, false);
    else NVFP4_DUAL_COL(false, false);
  }
#undef NVFP4_DUAL_ROW
#undef NVFP4_DUAL_COL
  if (z) zero_count_finish_kernel<<<1, 64, 0, st>>>(slot_r, slot_c, a.zeros);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_mse_t(const void* xv, int64_t rows, int64_t cols, bool x_fp32,
                                 float* amax, bool amax_is_input, uint8_t* codes,
                                 uint8_t* scales, float* gdec, hipStream_t st) {
  const T* x = static_cast<const T*>(xv);
  const int64_t chunks = rows * cols / 8;
  if (!amax_is_input) {
    const int u = x_fp32 ? 2 : kAmaxUnroll;
    amax_flat_kernel<T, false><<<dim3(amax_grid(chunks, u), 1), kAmaxThreads, 0, st>>>(
        x, chunks, 0, amax, nullptr, next_slot());
  }
  const int64_t blocks = rows * cols / 16;
  const int grid = (int)cdiv(blocks, (int64_t)kThreads);
  quant_mse_row_kernel<T><<<grid, kThreads, 0, st>>>(x, blocks, amax,
                                                     reinterpret_cast<uint2*>(codes), scales,
                                                     gdec);
  return hipGetLastError();
}

}  // namespace

int set_single_pass_wait_us(int us) {
  return g_single_pass_wait_us.exchange(us < 0 ? -1 : us, std::memory_order_relaxed);
}

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

hipError_t check_finite(const void* x, bool x_fp32, int64_t n, hipStream_t st, bool* finite) {
  *finite = true;
  if (n <= 0) return hipSuccess;
  unsigned int* flags = nullptr;  // this device's copy of the flags
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&flags), HIP_SYMBOL(g_nonfinite));
  if (e != hipSuccess) return e;
  unsigned int* flag = flags + next_slot();
  const int64_t chunks = n * (x_fp32 ? 4 : 2) / 16;  // n is a multiple of 32
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(chunks, kThreads), 4096);
  const uint4* xv = static_cast<const uint4*>(x);
  if (x_fp32)
    nonfinite_kernel<float><<<grid, kThreads, 0, st>>>(xv, chunks, flag);
  else
    nonfinite_kernel<uint16_t><<<grid, kThreads, 0, st>>>(xv, chunks, flag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned int v = 0;
  e = hipMemcpyAsync(&v, flag, sizeof v, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess || v == 0) return e;
  *finite = false;
  const unsigned int zero = 0;
  e = hipMemcpyAsync(flag, &zero, sizeof zero, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e;
}

}  // namespace nvfp4
