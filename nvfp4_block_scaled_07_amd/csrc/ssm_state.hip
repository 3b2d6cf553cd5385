// ssm_state.hip -- fp32 -> fp16 stochastic rounding of an SSM-state cache on
// gfx950 (bandwidth-bound).
//
// The Super report summary, section 4.3 (Mamba state quantization): decoding
// is bound by reading the SSM cache from DRAM; an fp16 cache written with
// round-to-nearest-even drifts (its bias accumulates through the recurrence),
// and the recipe is fp16 with stochastic rounding from Philox<5>, with no
// block scales.  Rounding rule: with lo the largest fp16 <= |x| and hi the
// next, the magnitude rounds up iff u < 65536 (|x| - lo) / (hi - lo), u the
// element's 16-bit random slot (slot i % 8 of Philox call i / 8, as in the
// block quantizers); |x| >= 65504 saturates, NaN stays NaN, the sign is kept.
//
// Work mapping: a lane takes 8 consecutive elements (two 16-byte loads, one
// 16-byte store, one Philox call), kUnroll chunks per thread with all loads
// issued first; a partial last chunk is done element by element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// fp16 bits of x rounded stochastically with u16, on the fp32 bits F of |x|:
//  * fp16 normals (|x| >= 2^-14): drop the 13 low mantissa bits and rebias the
//    exponent ((F >> 13) - 112 * 2^10); the fraction toward the next fp16 is
//    those 13 bits over 2^13, so "u < 65536 * fraction" is u < 8 * bits.
//    Above 65504 the count passes 0x7BFF and is clamped there (also for inf);
//  * fp16 subnormals (step 2^-24): t = |x| * 2^24 (exact), k = floor(t) is the
//    lower code and t - k (exact) the fraction; k + 1 = 1024 is 2^-14.
// Checked equal to the table-based definition on 685M (value, u) pairs on
// the CPU, every u at the range boundaries included.
__device__ __forceinline__ uint32_t sr_fp16_bits(float x, uint32_t u16) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t F = bits & 0x7FFFFFFFu, sign = (bits >> 16) & 0x8000u;
  const uint32_t hn = __builtin_elementwise_min(
      (F >> 13) - (112u << 10) + (u16 < ((F & 0x1FFFu) << 3) ? 1u : 0u), 0x7BFFu);
  const float t = __uint_as_float(F) * 16777216.0f;
  const float k = __builtin_floorf(t);
  const uint32_t hs = (uint32_t)k + ((float)u16 < (t - k) * 65536.0f ? 1u : 0u);
  const uint32_t h = F > 0x7F800000u ? 0x7E00u : (F >= 0x38800000u ? hn : hs);
  return sign | h;
}

__global__ __launch_bounds__(kThreads) void sr_fp16_kernel(const float* __restrict__ x, int64_t n,
                                                           uint16_t* __restrict__ y, uint64_t seed,
                                                           uint64_t offset, uint32_t rounds) {
  const int64_t full = n / 8, chunks = (n + 7) / 8;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  float v[kUnroll][8];
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + (int64_t)u * kThreads;
    if (c < full) {
      const float4 a = reinterpret_cast<const float4*>(x + 8 * c)[0];
      const float4 b = reinterpret_cast<const float4*>(x + 8 * c)[1];
      v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
      v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) v[u][t] = c < chunks && 8 * c + t < n ? x[8 * c + t] : 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + (int64_t)u * kThreads;
    if (c >= chunks) continue;
    const Philox4 p = sr_call((uint64_t)c, seed, offset, rounds);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
      w[q] = sr_fp16_bits(v[u][2 * q], sr_slot(p, 2 * q)) |
             (sr_fp16_bits(v[u][2 * q + 1], sr_slot(p, 2 * q + 1)) << 16);
    if (c < full) {
      reinterpret_cast<uint4*>(y)[c] = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++)
        if (8 * c + t < n) y[8 * c + t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
    }
  }
}

}  // namespace

hipError_t launch_sr_fp16(const float* x, int64_t n, uint64_t seed, uint64_t offset,
                          uint32_t rounds, uint16_t* y, hipStream_t st) {
  const int64_t chunks = (n + 7) / 8;
  const int64_t per = (int64_t)kThreads * kUnroll;
  const int64_t grid = (chunks + per - 1) / per;
  sr_fp16_kernel<<<(unsigned)grid, kThreads, 0, st>>>(x, n, y, seed, offset, rounds);
  return hipGetLastError();
}

}  // namespace nvfp4
