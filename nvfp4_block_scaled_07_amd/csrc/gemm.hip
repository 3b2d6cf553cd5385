// gemm.hip -- NVFP4 GEMMs (dense NT/NN/TN and grouped) for gfx950.
//
// Design (the operation: Super summary, Infra table; Ultra report 2.2):
//  * CDNA4's FP4 matrix instructions take power-of-two scales per 32
//    elements, which cannot carry an E4M3 scale per 16 elements.  Instead
//    every element is decoded to fp16 -- exact: val(code) has 2 significant
//    bits, an E4M3 scale 4, so their product has at most 6 and lies in
//    [2^-10, 2688] -- and fed to v_mfma_f32_32x32x16_f16 with fp32
//    accumulation.
//  * Codes and scales (0.5625 B per element) are staged global -> VGPR ->
//    LDS in a canonical K-major layout: 32 code bytes (64 k) per row per stage
//    and the scales pre-expanded to packed fp16 pairs (d, d).  MN-major
//    operands (the TN/NN layouts) are transposed on the way in with an 8x8
//    nibble transpose in registers.
//  * Each wave decodes only the fragments it multiplies: lane l reads 16 code
//    bytes of row l%32 (k = 32*(l/32) .. +32 of the stage) and the two scale
//    pairs, and for each of the four 16-k MFMA steps converts 8 nibbles with
//    v_cvt_scalef32_pk_f16_fp4 (scale 1) and v_pk_mul_f16 by (d, d).  The k
//    order inside an MFMA is a permutation shared by A and B, so the sum is
//    unchanged.
//  * Epilogue: C = RN32(acc * RN32(gA * gB)), stored as bf16 (RNE) or fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs

constexpr int BK = 64;  // k per LDS stage

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM / 32;  // 32x32 MFMA tiles per wave along M
  static constexpr int TN = BN / WN / 32;
  static constexpr int kACodes = BM * 32, kAScales = BM * 16;
  static constexpr int kBCodes = BN * 32, kBScales = BN * 16;
  static constexpr int kStage = kACodes + kAScales + kBCodes + kBScales;
};

// Operand view for one tile: base pointers and the strides of its stored
// layout.  K-major: stored [MN][K]; MN-major: stored [K][MN] (mn_total wide).
struct OpView {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t mn_total;  // stored width of an MN-major operand
  int block;
};

__device__ __forceinline__ uint32_t bits_of(half2 h) { return __builtin_bit_cast(uint32_t, h); }

// Every E4M3 byte -> its packed fp16 pair (d, d), for the 256-entry table each
// workgroup keeps in LDS (exact: every E4M3 value is an fp16 value).
__device__ __forceinline__ uint32_t e4m3_pair_f16(uint32_t e) {
  _Float16 h = (_Float16)e4m3_decode(e & 0x7Fu);
  half2 p = {h, h};
  return bits_of(p);
}

__device__ __forceinline__ void build_scale_table(uint32_t* table, int tid, int nt) {
  for (int i = tid; i < 256; i += nt) table[i] = e4m3_pair_f16((uint32_t)i);
}

// 4 E4M3 scale bytes -> 4 packed fp16 pairs, through the LDS table.
__device__ __forceinline__ uint4 expand_scales(uint32_t s4, const uint32_t* table) {
  return make_uint4(table[s4 & 0xFFu], table[(s4 >> 8) & 0xFFu], table[(s4 >> 16) & 0xFFu],
                    table[s4 >> 24]);
}

// Swizzled LDS addresses (bytes within one operand's region).
__device__ __forceinline__ int code_addr(int row, int half) {
  return row * 32 + 16 * (half ^ ((row >> 2) & 1));
}
__device__ __forceinline__ int scale_addr(int row, int half) {
  return row * 16 + 8 * (half ^ ((row >> 3) & 1));
}

// In-register transpose of an 8x8 matrix of nibbles: d[i] nibble j -> d[j]
// nibble i (three rounds of block swaps: 4x4, 2x2, 1x1).
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t d[8]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t t = ((d[i] >> 16) ^ d[i + 4]) & 0x0000FFFFu;
    d[i + 4] ^= t;
    d[i] ^= t << 16;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if (i & 2) continue;
    uint32_t t = ((d[i] >> 8) ^ d[i + 2]) & 0x00FF00FFu;
    d[i + 2] ^= t;
    d[i] ^= t << 8;
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    uint32_t t = ((d[i] >> 4) ^ d[i + 1]) & 0x0F0F0F0Fu;
    d[i + 1] ^= t;
    d[i] ^= t << 4;
  }
}

// ---- staging: global -> registers -> LDS ---------------------------------------------------
// Loads are branch-free and unmasked: a row past the operand's edge re-reads
// the last valid row (always in bounds).  Row i of A only reaches row i of C
// and row j of B only column j, so such rows only feed outputs that are never
// stored.  The main loop stays one basic block the scheduler can interleave,
// and the prefetched values are not consumed until the stage is written out.

// K-major operand, ROWS rows of the tile, NT threads.
template <int ROWS, int NT>
struct StageK {
  static_assert((ROWS * 2) % NT == 0 && ROWS % NT == 0, "tile rows must divide evenly");
  static constexpr int CN = ROWS * 2 / NT;  // uint4 of codes per thread
  static constexpr int SN = ROWS / NT;      // scale dwords per thread
  u32x4 c[CN];
  uint32_t s[SN];

  __device__ __forceinline__ void load(const OpView& op, int64_t mn0, int64_t mn_lim,
                                       int64_t k0, int64_t K, int tid) {
#pragma unroll
    for (int j = 0; j < CN; j++) {
      int idx = tid + j * NT;
      int64_t mn = mn0 + (idx >> 1);
      int64_t mc = mn < mn_lim ? mn : mn_lim - 1;
      c[j] = *reinterpret_cast<const u32x4*>(op.codes + mc * (K / 2) + k0 / 2 + 16 * (idx & 1));
    }
#pragma unroll
    for (int j = 0; j < SN; j++) {
      int64_t mn = mn0 + tid + j * NT;
      int64_t mc = mn < mn_lim ? mn : mn_lim - 1;
      int64_t off = op.block == kBlock2d ? (mc / 16) * (K / 16) : mc * (K / 16);
      s[j] = *reinterpret_cast<const uint32_t*>(op.scales + off + k0 / 16);
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes, uint8_t* lds_scales, int tid,
                                        const uint32_t* table) const {
    store_codes(lds_codes, tid);
    store_scales(lds_scales, tid, table);
  }

  __device__ __forceinline__ void store_codes(uint8_t* lds_codes, int tid) const {
#pragma unroll
    for (int j = 0; j < CN; j++) {
      int idx = tid + j * NT;
      *reinterpret_cast<u32x4*>(lds_codes + code_addr(idx >> 1, idx & 1)) = c[j];
    }
  }

  __device__ __forceinline__ void store_scales(uint8_t* lds_scales, int tid,
                                               const uint32_t* table) const {
#pragma unroll
    for (int j = 0; j < SN; j++) {
      int idx = tid + j * NT;
      uint4 e = expand_scales(s[j], table);
      *reinterpret_cast<uint2*>(lds_scales + scale_addr(idx, 0)) = make_uint2(e.x, e.y);
      *reinterpret_cast<uint2*>(lds_scales + scale_addr(idx, 1)) = make_uint2(e.z, e.w);
    }
  }
};

// MN-major operand: the stage is BK rows (k) x ROWS columns (mn).  A unit is
// 8 k x 8 mn (8 dwords, one per k row), transposed to 8 dwords along k.
template <int ROWS, int NT>
struct StageMN {
  static constexpr int UNITS = (BK / 8) * (ROWS / 8);
  static_assert(UNITS % NT == 0 && ROWS % NT == 0, "tile must divide evenly");
  static constexpr int UN = UNITS / NT;
  static constexpr int SN = ROWS / NT;
  uint32_t c[UN][8];
  uint32_t s[SN];

  __device__ __forceinline__ void load(const OpView& op, int64_t mn0, int64_t mn_lim,
                                       int64_t k0, int64_t K, int tid) {
    (void)K;
    const int64_t W = op.mn_total;
#pragma unroll
    for (int j = 0; j < UN; j++) {
      int u = tid + j * NT;
      int kg = u / (ROWS / 8), md = u % (ROWS / 8);
      int64_t mn = mn0 + 8 * md;
      int64_t mc = mn < mn_lim ? mn : mn_lim - 8;  // mn_lim is a multiple of 8
#pragma unroll
      for (int r = 0; r < 8; r++)
        c[j][r] = *reinterpret_cast<const uint32_t*>(op.codes + (k0 + 8 * kg + r) * (W / 2) +
                                                      mc / 2);
    }
#pragma unroll
    for (int j = 0; j < SN; j++) {
      int64_t mn = mn0 + tid + j * NT;
      int64_t mc = mn < mn_lim ? mn : mn_lim - 1;
      uint32_t v = 0;
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        int64_t row = k0 / 16 + kb;
        int64_t off = op.block == kBlock2d ? row * (W / 16) + mc / 16 : row * W + mc;
        v |= (uint32_t)op.scales[off] << (8 * kb);
      }
      s[j] = v;
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes, uint8_t* lds_scales, int tid,
                                        const uint32_t* table) {
    store_codes(lds_codes, tid);
    store_scales(lds_scales, tid, table);
  }

  __device__ __forceinline__ void store_codes(uint8_t* lds_codes, int tid) {
#pragma unroll
    for (int j = 0; j < UN; j++) {
      int u = tid + j * NT;
      int kg = u / (ROWS / 8), md = u % (ROWS / 8);
      transpose8x8_nibbles(c[j]);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        int row = 8 * md + i;
        *reinterpret_cast<uint32_t*>(lds_codes + code_addr(row, kg >> 2) + 4 * (kg & 3)) =
            c[j][i];
      }
    }
  }

  __device__ __forceinline__ void store_scales(uint8_t* lds_scales, int tid,
                                               const uint32_t* table) const {
#pragma unroll
    for (int j = 0; j < SN; j++) {
      int idx = tid + j * NT;
      uint4 e = expand_scales(s[j], table);
      *reinterpret_cast<uint2*>(lds_scales + scale_addr(idx, 0)) = make_uint2(e.x, e.y);
      *reinterpret_cast<uint2*>(lds_scales + scale_addr(idx, 1)) = make_uint2(e.z, e.w);
    }
  }
};

template <bool KMAJOR, int ROWS, int NT>
using Stage = typename std::conditional<KMAJOR, StageK<ROWS, NT>, StageMN<ROWS, NT>>::type;

// Decode 8 nibbles (one dword) scaled by the packed pair sc = (d, d).  The
// conversion's own scale operand only applies a power of two, so it stays 1
// and the E4M3 scale is a separate exact fp16 multiply.
__device__ __forceinline__ half8 decode8(uint32_t q, uint32_t sc) {
  half2 d = __builtin_bit_cast(half2, sc);
  half2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * d;
  half2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * d;
  half2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * d;
  half2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * d;
  half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// One output tile: C[m0 : m0+BM) x [n0 : n0+BN) restricted to rows < m_lim,
// cols < N.  lds holds 2 stages and then the 256-entry scale table, which
// the caller has built (and synchronized) before the first tile.
//
// Per 64-k stage each wave: loads the next stage from global memory (held in
// registers), reads its fragments' codes and scales from LDS, decodes the
// first 16-k step, then runs the four steps' MFMAs while decoding the next
// step between them, and writes the next stage to the other LDS buffer
// during the last step.
template <class C, bool AK, bool BKM>
__device__ __forceinline__ void gemm_tile(const OpView& A, const OpView& B, int64_t m0,
                                          int64_t m_lim, int64_t n0, int64_t N, int64_t K,
                                          float gscale, void* Cout, bool c_bf16, int64_t ldc,
                                          uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lrow = lane & 31, lhalf = lane >> 5;

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; i++)
#pragma unroll
    for (int j = 0; j < C::TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  Stage<AK, C::BM, C::NT> sa;
  Stage<BKM, C::BN, C::NT> sb;
  const int64_t KT = K / BK;
  const uint32_t* table = reinterpret_cast<const uint32_t*>(lds + 2 * C::kStage);

  // Fragment rows of one wave step by 32, which keeps both swizzles (they
  // depend on row bits 2 and 3), so each operand needs one base address.
  const int a_row0 = wm * (C::BM / C::WM) + lrow, b_row0 = wn * (C::BN / C::WN) + lrow;
  const int a_code0 = code_addr(a_row0, lhalf);
  const int a_sc0 = C::kACodes + scale_addr(a_row0, lhalf);
  const int b_code0 = C::kACodes + C::kAScales + code_addr(b_row0, lhalf);
  const int b_sc0 = C::kACodes + C::kAScales + C::kBCodes + scale_addr(b_row0, lhalf);

  sa.load(A, m0, m_lim, 0, K, tid);
  sb.load(B, n0, N, 0, K, tid);
  sa.store(lds, lds + C::kACodes, tid, table);
  sb.store(lds + C::kACodes + C::kAScales, lds + C::kACodes + C::kAScales + C::kBCodes, tid,
           table);
  __syncthreads();

  for (int64_t kt = 0; kt < KT; kt++) {
    const int buf = (int)(kt & 1);
    // Next stage (the last iteration reloads the final stage into the idle
    // buffer, which keeps the loop free of branches).
    const int64_t kn = (kt + 1 < KT ? kt + 1 : kt) * BK;
    sa.load(A, m0, m_lim, kn, K, tid);
    sb.load(B, n0, N, kn, K, tid);

    const uint8_t* st = lds + buf * C::kStage;
    uint4 aq[C::TM], bq[C::TN];
    uint2 as[C::TM], bs[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++) {
      aq[i] = *reinterpret_cast<const uint4*>(st + a_code0 + i * 32 * 32);
      as[i] = *reinterpret_cast<const uint2*>(st + a_sc0 + i * 32 * 16);
    }
#pragma unroll
    for (int j = 0; j < C::TN; j++) {
      bq[j] = *reinterpret_cast<const uint4*>(st + b_code0 + j * 32 * 32);
      bs[j] = *reinterpret_cast<const uint2*>(st + b_sc0 + j * 32 * 16);
    }

    // A fragments are single-buffered: fragment i of the next step is decoded
    // once row i's MFMAs of this step have issued.  B fragments, used by every
    // row, are double-buffered.
    half8 af[C::TM], bf[2][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++) af[i] = decode8(aq[i].x, as[i].x);
#pragma unroll
    for (int j = 0; j < C::TN; j++) bf[0][j] = decode8(bq[j].x, bs[j].x);

    // Steps 0..3 of the stage.  The order is fixed in the source and fenced
    // with sched_barrier: after every second MFMA one fragment of the next
    // step is decoded (8 VALU ops that issue while the MFMAs run) -- first the
    // B fragments, then A fragment f once row f is done; during the last step
    // the next stage is written to the other LDS buffer instead.
    uint8_t* sn = lds + (buf ^ 1) * C::kStage;
    static_assert(C::TM == 4 && C::TN == 4, "interleave expects 4x4 MFMA tiles per wave");
#pragma unroll
    for (int s = 0; s < 3; s++) {
      const int cur = s & 1, nxt = cur ^ 1;
#pragma unroll
      for (int i = 0; i < C::TM; i++) {
#pragma unroll
        for (int j = 0; j < C::TN; j++) {
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[cur][j], acc[i][j], 0, 0, 0);
          const int t = i * C::TN + j;
          if (t & 1) {
            const int f = t >> 1;  // 0..3: B fragment f; 4..7: A fragment f-4
            if (f < C::TN)
              bf[nxt][f] = decode8(pick(bq[f], s + 1), s + 1 < 2 ? bs[f].x : bs[f].y);
            else
              af[f - C::TN] = decode8(pick(aq[f - C::TN], s + 1),
                                      s + 1 < 2 ? as[f - C::TN].x : as[f - C::TN].y);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    // Step 3 (uses bf[1]): one row of MFMAs, then a quarter of the next
    // stage's LDS writes.
#pragma unroll
    for (int j = 0; j < C::TN; j++)
      acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0], bf[1][j], acc[0][j], 0, 0, 0);
    sa.store_codes(sn, tid);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < C::TN; j++)
      acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[1], bf[1][j], acc[1][j], 0, 0, 0);
    sa.store_scales(sn + C::kACodes, tid, table);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < C::TN; j++)
      acc[2][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[2], bf[1][j], acc[2][j], 0, 0, 0);
    sb.store_codes(sn + C::kACodes + C::kAScales, tid);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < C::TN; j++)
      acc[3][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[3], bf[1][j], acc[3][j], 0, 0, 0);
    sb.store_scales(sn + C::kACodes + C::kAScales + C::kBCodes, tid, table);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane l holds column l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < C::TM; i++) {
#pragma unroll
    for (int j = 0; j < C::TN; j++) {
      const int64_t col = n0 + wn * (C::BN / C::WN) + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = m0 + wm * (C::BM / C::WM) + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (row < m_lim && col < N) {
          float v = acc[i][j][r] * gscale;
          if (c_bf16)
            static_cast<uint16_t*>(Cout)[row * ldc + col] = (uint16_t)bf16_rne_bits(v);
          else
            static_cast<float*>(Cout)[row * ldc + col] = v;
        }
      }
    }
  }
}

// Tile order: groups of 8 M-tiles sweep N, so a wave of workgroups shares
// both operands' panels in L2.
__device__ __forceinline__ void tile_coords(int64_t t, int64_t ntm, int64_t ntn, int64_t& tm,
                                            int64_t& tn) {
  const int64_t G = 8;
  int64_t per_group = G * ntn;
  int64_t grp = t / per_group;
  int64_t first = grp * G;
  int64_t gsize = ntm - first < G ? ntm - first : G;
  int64_t r = t % per_group;
  tm = first + r % gsize;
  tn = r / gsize;
}

template <class C, bool AK, bool BKM>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  int64_t tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  OpView A{a.A.codes, a.A.scales, a.M, a.A.block};
  OpView B{a.B.codes, a.B.scales, a.N, a.B.block};
  const float gs = *a.A.gdec * *a.B.gdec;
  build_scale_table(reinterpret_cast<uint32_t*>(lds + 2 * C::kStage), threadIdx.x, C::NT);
  __syncthreads();
  gemm_tile<C, AK, BKM>(A, B, tm * C::BM, a.M, tn * C::BN, a.N, a.K, gs, a.C, a.c_bf16, a.N, lds);
}

// Persistent grouped kernel: every workgroup builds the prefix of per-group
// tile counts in LDS, then walks tiles blockIdx.x, +gridDim.x, ...
template <class C>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(GroupedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  build_scale_table(reinterpret_cast<uint32_t*>(lds + 2 * C::kStage), threadIdx.x, C::NT);
  int32_t* prefix = reinterpret_cast<int32_t*>(lds + 2 * C::kStage + 1024);  // [groups + 1]
  __shared__ int32_t part[C::NT];
  const int tid = threadIdx.x;
  const int64_t G = a.groups;
  const int64_t ntn = (a.N + C::BN - 1) / C::BN;
  const int64_t per = (G + C::NT - 1) / C::NT;
  int32_t local = 0;
  for (int64_t e = tid * per; e < (tid + 1) * per && e < G; e++) {
    int64_t rows = a.offsets[e + 1] - a.offsets[e];
    local += (int32_t)(((rows + C::BM - 1) / C::BM) * ntn);
  }
  part[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int i = 0; i < C::NT; i++) {
      int32_t v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  {
    int32_t run = part[tid];
    for (int64_t e = tid * per; e < (tid + 1) * per && e < G; e++) {
      prefix[e] = run;
      int64_t rows = a.offsets[e + 1] - a.offsets[e];
      run += (int32_t)(((rows + C::BM - 1) / C::BM) * ntn);
    }
    if (tid == C::NT - 1) prefix[G] = run;  // last thread's run covers all groups
  }
  __syncthreads();
  const int32_t total = prefix[G];
  const float ga = *a.A.gdec;
  const int64_t b_codes_stride = a.N * a.K / 2;
  const int64_t b_scales_stride =
      a.B.block == kBlock2d ? (a.N / 16) * (a.K / 16) : a.N * (a.K / 16);
  for (int32_t t = blockIdx.x; t < total; t += gridDim.x) {
    // largest e with prefix[e] <= t (empty groups share a prefix value)
    int64_t lo = 0, hi = G;  // prefix[lo] <= t < prefix[hi]
    while (hi - lo > 1) {
      int64_t mid = (lo + hi) >> 1;
      if (prefix[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t e = lo;
    const int32_t lt = t - prefix[e];
    const int64_t mt = lt / ntn, nt = lt % ntn;
    const int64_t r0 = a.offsets[e], r1 = a.offsets[e + 1];
    OpView A{a.A.codes + r0 * (a.K / 2), a.A.scales + r0 * (a.K / 16), 0, kBlockRow};
    OpView B{a.B.codes + e * b_codes_stride, a.B.scales + e * b_scales_stride, 0, a.B.block};
    const float gs = ga * a.B.gdec[e];
    gemm_tile<C, true, true>(A, B, mt * C::BM, r1 - r0, nt * C::BN, a.N, a.K, gs,
                             a.c_bf16 ? (void*)(static_cast<uint16_t*>(a.C) + r0 * a.N)
                                      : (void*)(static_cast<float*>(a.C) + r0 * a.N),
                             a.c_bf16, a.N, lds);
    __syncthreads();
  }
}

using Dense = Cfg<256, 256, 2, 2>;
using Grouped = Cfg<256, 256, 2, 2>;

template <class C, bool AK, bool BKM>
hipError_t launch_dense(const GemmArgs& a, hipStream_t st) {
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  const size_t smem = 2 * C::kStage + 1024;
  auto kern = gemm_kernel<C, AK, BKM>;
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  kern<<<(unsigned)(ntm * ntn), C::NT, smem, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.a_kmajor && a.b_kmajor) return launch_dense<Dense, true, true>(a, st);
  if (a.a_kmajor && !a.b_kmajor) return launch_dense<Dense, true, false>(a, st);
  return launch_dense<Dense, false, false>(a, st);
}

hipError_t launch_grouped_gemm(const GroupedArgs& a, hipStream_t st) {
  if (a.total_rows == 0 || a.N == 0 || a.groups == 0) return hipSuccess;
  using C = Grouped;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t ntn = (a.N + C::BN - 1) / C::BN;
  const int64_t max_tiles = ((a.total_rows + C::BM - 1) / C::BM + a.groups) * ntn;
  int64_t grid = cus > 0 ? cus : 256;
  if (grid > max_tiles) grid = max_tiles;
  const size_t smem = 2 * C::kStage + 1024 + sizeof(int32_t) * (size_t)(a.groups + 1);
  auto kern = grouped_gemm_kernel<C>;
  if (smem > 65536) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
    if (e != hipSuccess) return e;
  }
  kern<<<(unsigned)grid, C::NT, smem, st>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
