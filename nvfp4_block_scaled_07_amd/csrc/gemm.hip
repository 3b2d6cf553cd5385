// gemm.hip -- NVFP4 GEMMs (dense NT/NN/TN and grouped) for gfx950.
//
// Design (the operation: Super summary, Infra table; Ultra report 2.2):
//  * CDNA4's FP4 matrix instructions take power-of-two scales per 32
//    elements, which cannot carry an E4M3 scale per 16 elements.  Instead
//    every element is decoded to fp16 -- exact: val(code) has 2 significant
//    bits, an E4M3 scale 4, so their product has at most 6 and lies in
//    [2^-10, 2688] -- and fed to v_mfma_f32_32x32x16_f16 with fp32
//    accumulation.
//  * Codes and scale bytes (0.5625 B per element) are staged in LDS in a
//    canonical K-major layout per 64-k stage: 32 code bytes per row (two
//    16-byte halves, swapped on rows with bit 2 set to spread LDS banks) and
//    4 raw scale bytes per row.  K-major operands go global -> LDS directly
//    (4-byte LDS DMA, no registers); MN-major operands (the TN/NN layouts)
//    go through registers and an 8x8 nibble transpose.
//  * Each wave decodes only the fragments it multiplies: lane l reads 16 code
//    bytes of row l%32 (k = 32*(l/32) .. +32 of the stage) and the row's two
//    scale bytes for those k, converts the scales to an fp16 pair with
//    v_cvt_scalef32_pk_f16_fp8 and, for each 16-k MFMA step, 8 nibbles with
//    v_cvt_scalef32_pk_f16_fp4 (both with scale 1: their scale operand only
//    applies a power of two) and v_pk_mul_f16.  The k order inside an MFMA
//    is a permutation shared by A and B, so the sum is unchanged.
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

constexpr int BK = 64;       // k per LDS stage
constexpr int kStages = 4;   // LDS ring depth

template <int BM_, int BN_, int WM_, int WN_, bool FENCE_ = true>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool kFence = FENCE_;  // fence the MFMA/decode order with sched_barrier
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM / 32;  // 32x32 MFMA tiles per wave along M
  static constexpr int TN = BN / WN / 32;
  static constexpr int kACodes = BM * 32, kAScales = BM * 4;
  static constexpr int kBCodes = BN * 32, kBScales = BN * 4;
  static constexpr int kStage = kACodes + kAScales + kBCodes + kBScales;
  static constexpr int kLds = kStages * kStage;
};

// Operand view for one tile: base pointers and the strides of its stored
// layout.  K-major: stored [MN][K]; MN-major: stored [K][MN] (mn_total wide).
struct OpView {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t mn_total;  // stored width of an MN-major operand
  int block;
};

// Makes v look redefined here, so arithmetic on a prefetched value cannot be
// hoisted up to its load (which would wait for the load right away).
template <typename T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (expcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Swizzled byte address of half `half` (16 bytes) of code row `row`.
__device__ __forceinline__ int code_addr(int row, int half) {
  return row * 32 + 16 * (half ^ ((row >> 2) & 1));
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

// ---- staging: K-major operands by LDS DMA ----------------------------------------------------
// buffer_load_dword{,x4} ... lds moves 4 or 16 bytes per lane into LDS at
// (wave-uniform base + size * lane); the lane's source offset is chosen so
// that the LDS image is the swizzled canonical layout.  A row past the
// operand's edge re-reads the last valid row (always in bounds): row i of A
// only reaches row i of C, row j of B only column j, so such rows only feed
// outputs that are never stored.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 dword3)

template <int ROWS, int NW, int SW0, int SWN>
struct DmaK {
  // Code chunks (1 KiB = 32 rows, 16 bytes per lane) spread over all NW
  // waves; scale chunks (256 B = 64 rows, 4 bytes per lane) over waves
  // [SW0, SW0 + SWN), one each.
  static constexpr int kCodeChunks = ROWS * 32 / 1024;
  static_assert(kCodeChunks % NW == 0, "code chunks must split over waves");
  static_assert(ROWS * 4 / 256 == SWN, "one scale chunk per scale wave");
  static constexpr int CPW = kCodeChunks / NW;
  uint32_t coff[CPW];  // lane byte offsets from the tile's first code row
  uint32_t soff;       // lane byte offset from the tile's first scale row
  __amdgpu_buffer_rsrc_t crsrc, srsrc;
  int wave;

  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int lane, int wv) {
    wave = wv;
    const int64_t kc = K / 2, ks = K / 16;
#pragma unroll
    for (int q = 0; q < CPW; q++) {
      const int c = wave * CPW + q;
      const int row = 32 * c + (lane >> 1);
      const int h = (lane & 1) ^ ((row >> 2) & 1);
      const int64_t mn = mn0 + row < mn_lim ? mn0 + row : mn_lim - 1;
      coff[q] = (uint32_t)((mn - mn0) * kc + 16 * h);
    }
    const bool two_d = op.block == kBlock2d;
    const int srow = (wave - SW0) * 64 + lane;  // meaningful on scale waves only
    const int64_t smn = mn0 + srow < mn_lim ? mn0 + srow : mn_lim - 1;
    const int64_t sbase = two_d ? (mn0 / 16) * ks : mn0 * ks;
    const int64_t slim = two_d ? ((mn_lim + 15) / 16) * ks : mn_lim * ks;
    soff = (uint32_t)((two_d ? (smn / 16) * ks : smn * ks) - sbase);
    crsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.codes + mn0 * kc), 0,
                                              (int)((mn_lim - mn0) * kc), kBufferFlags);
    srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.scales + sbase), 0,
                                              (int)(slim - sbase), kBufferFlags);
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds_codes, uint8_t* lds_scales) const {
#pragma unroll
    for (int q = 0; q < CPW; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, lds_codes + (wave * CPW + q) * 1024, 16,
                                               coff[q], (int)(k0 / 2), 0, 0);
    if (wave >= SW0 && wave < SW0 + SWN)  // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, lds_scales + (wave - SW0) * 256, 4, soff,
                                               (int)(k0 / 16), 0, 0);
  }
};

// ---- staging: MN-major operands through registers ------------------------------------------
// The stage is BK rows (k) x ROWS columns (mn).  A unit is 8 k x 8 mn (8
// dwords, one per k row), transposed to 8 dwords along k.
// Threads [T0, T0 + NT) take part (a wave-uniform predicate).
template <int ROWS, int T0, int NT>
struct StageMN {
  static constexpr int UNITS = (BK / 8) * (ROWS / 8);
  static_assert(UNITS % NT == 0 && ROWS % NT == 0, "tile must divide evenly");
  static constexpr int UN = UNITS / NT;
  static constexpr int SN = ROWS / NT;
  uint32_t c[UN][8];
  uint32_t s[SN][4];  // the four k-block scale bytes of each row, assembled at store time

  __device__ __forceinline__ void load(const OpView& op, int64_t mn0, int64_t mn_lim,
                                       int64_t k0, int tid_all) {
    const int tid = tid_all - T0;
    if (tid < 0 || tid >= NT) return;
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
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        int64_t row = k0 / 16 + kb;
        int64_t off = op.block == kBlock2d ? row * (W / 16) + mc / 16 : row * W + mc;
        s[j][kb] = op.scales[off];
      }
    }
  }

  __device__ __forceinline__ void store_codes(uint8_t* lds_codes, int tid_all) {
    const int tid = tid_all - T0;
    if (tid < 0 || tid >= NT) return;
#pragma unroll
    for (int j = 0; j < UN; j++) {
      int u = tid + j * NT;
      int kg = u / (ROWS / 8), md = u % (ROWS / 8);
#pragma unroll
      for (int r = 0; r < 8; r++) pin(c[j][r]);
      transpose8x8_nibbles(c[j]);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        int row = 8 * md + i;
        *reinterpret_cast<uint32_t*>(lds_codes + code_addr(row, kg >> 2) + 4 * (kg & 3)) =
            c[j][i];
      }
    }
  }

  __device__ __forceinline__ void store_scales(uint8_t* lds_scales, int tid_all) {
    const int tid = tid_all - T0;
    if (tid < 0 || tid >= NT) return;
#pragma unroll
    for (int j = 0; j < SN; j++) {
#pragma unroll
      for (int kb = 0; kb < 4; kb++) pin(s[j][kb]);
      *reinterpret_cast<uint32_t*>(lds_scales + 4 * (tid + j * NT)) =
          s[j][0] | (s[j][1] << 8) | (s[j][2] << 16) | (s[j][3] << 24);
    }
  }
};

// Decode 8 nibbles (one dword) scaled by the packed pair d = (d, d).
__device__ __forceinline__ half8 decode8(uint32_t q, half2 d) {
  half2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * d;
  half2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * d;
  half2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * d;
  half2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * d;
  half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// Two E4M3 scale bytes (low 16 bits) -> fp16 pair, exact.
__device__ __forceinline__ half2 scale_pair(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ half2 splat(half2 d, int hi) {
  return hi ? half2{d[1], d[1]} : half2{d[0], d[0]};
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Decode schedule within a 16-k step of TM x TN MFMAs (t = i*TN + j): B
// fragment j (double-buffered) is decoded after MFMA `b_slot`, A fragment i
// (single-buffered) once row i's MFMAs have issued.  In the last step the
// fragments come from LDS reads issued at the step's start, so decodes wait
// for two MFMAs first.
template <int TM, int TN>
__device__ __forceinline__ constexpr int b_slot(int s, int j) {
  return s < 3 ? j : (2 + j < TM * TN ? 2 + j : TM * TN - 1);
}
template <int TM, int TN>
__device__ __forceinline__ constexpr int a_slot(int s, int i) {
  return s < 3 || i * TN + TN - 1 >= 2 ? i * TN + TN - 1 : 2;
}

// Per-operand staging: DMA for K-major, registers for MN-major.  OPB
// selects operand B's share of waves/threads (A uses the first half of the
// scale waves and MN threads, B the second).
template <bool KMAJOR, int ROWS, class C, int OPB>
struct Staging;

template <int ROWS, class C, int OPB>
struct Staging<true, ROWS, C, OPB> {
  static constexpr int kSW = ROWS * 4 / 256;  // scale waves
  static_assert(kSW <= C::NW, "one scale chunk per wave at most");
  // Both operands' scale chunks on disjoint waves when there are enough
  // waves, else on the same ones.
  static constexpr int kSW0 = (2 * kSW <= C::NW) ? OPB * kSW : 0;
  DmaK<ROWS, C::NW, kSW0, kSW> d;
  static constexpr int kCodeDma = DmaK<ROWS, C::NW, kSW0, kSW>::CPW;
  __device__ __forceinline__ int scale_dma(int wave) const {
    return wave >= kSW0 && wave < kSW0 + kSW ? 1 : 0;
  }
  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int tid) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
  }
  __device__ __forceinline__ void load_regs(const OpView&, int64_t, int64_t, int64_t, int) {}
  __device__ __forceinline__ void load_dma(int64_t k0, uint8_t* codes, uint8_t* scales) {
    d.issue(k0, codes, scales);
  }
  __device__ __forceinline__ void store_codes(uint8_t*, int) {}
  __device__ __forceinline__ void store_scales(uint8_t*, int) {}
};

template <int ROWS, class C, int OPB>
struct Staging<false, ROWS, C, OPB> {
  static constexpr int kThreads = C::NT >= 2 * ROWS ? ROWS : C::NT;
  static constexpr int kT0 = C::NT >= 2 * ROWS ? OPB * ROWS : 0;
  StageMN<ROWS, kT0, kThreads> r;
  static constexpr int kCodeDma = 0;
  __device__ __forceinline__ int scale_dma(int) const { return 0; }
  __device__ __forceinline__ void init(const OpView&, int64_t, int64_t, int64_t, int) {}
  __device__ __forceinline__ void load_regs(const OpView& op, int64_t mn0, int64_t mn_lim,
                                            int64_t k0, int tid) {
    r.load(op, mn0, mn_lim, k0, tid);
  }
  __device__ __forceinline__ void load_dma(int64_t, uint8_t*, uint8_t*) {}
  __device__ __forceinline__ void store_codes(uint8_t* codes, int tid) { r.store_codes(codes, tid); }
  __device__ __forceinline__ void store_scales(uint8_t* scales, int tid) {
    r.store_scales(scales, tid);
  }
};

// One output tile: C[m0 : m0+BM) x [n0 : n0+BN) restricted to rows < m_lim,
// cols < N, using lds (kLds bytes).
//
// Software pipeline over 64-k stages (stage s lives in LDS buffer s % 4):
//  * iteration kt starts stage kt+3's transfer: register loads for MN-major
//    operands at its start (written to LDS during steps 2 and 3), DMA for
//    K-major ones during its last step;
//  * its four 16-k steps run TM x TN MFMAs each; between MFMAs it decodes
//    the fragments of the following step -- for the last step, those of step
//    0 of stage kt+1, read from LDS at that step's start;
//  * it ends with one barrier, after waiting for this wave's transfers of
//    stage kt+2 (issued an iteration ago): stage kt+2 is read in the next
//    iteration, and the buffer stage kt+3 overwrites (stage kt-1's) was last
//    read two iterations ago.
// Decoded fragments: B double-buffered (every row uses them), A single-
// buffered, fragment i of the next step decoded once row i's MFMAs issued.
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

  Staging<AK, C::BM, C, 0> sa;
  Staging<BKM, C::BN, C, 1> sb;
  sa.init(A, m0, m_lim, K, tid);
  sb.init(B, n0, N, K, tid);
  // DMA instructions this wave issues per stage (wave-uniform): the code
  // chunks plus one scale chunk per operand whose scales this wave moves.
  constexpr int kCodeDma = Staging<AK, C::BM, C, 0>::kCodeDma + Staging<BKM, C::BN, C, 1>::kCodeDma;
  const int n_scale_dma = sa.scale_dma(wave) + sb.scale_dma(wave);
  const int64_t KT = K / BK;

  constexpr int oAS = C::kACodes, oBC = C::kACodes + C::kAScales,
                oBS = C::kACodes + C::kAScales + C::kBCodes;
  // Fragment rows of one wave step by 32, which keeps the code swizzle (it
  // depends on row bit 2), so each operand needs one base address.
  const int a_row0 = wm * (C::BM / C::WM) + lrow, b_row0 = wn * (C::BN / C::WN) + lrow;
  const int a_code0 = code_addr(a_row0, lhalf), b_code0 = oBC + code_addr(b_row0, lhalf);
  const int a_sc0 = oAS + 4 * a_row0 + 2 * lhalf, b_sc0 = oBS + 4 * b_row0 + 2 * lhalf;

  auto buffer = [&](int idx) { return lds + idx * C::kStage; };
  auto load_regs = [&](int64_t k0) {
    sa.load_regs(A, m0, m_lim, k0, tid);
    sb.load_regs(B, n0, N, k0, tid);
  };
  auto load_dma = [&](int64_t k0, uint8_t* dst) {
    sa.load_dma(k0, dst, dst + oAS);
    sb.load_dma(k0, dst + oBC, dst + oBS);
  };

  uint4 aq[C::TM], bq[C::TN];
  half2 as[C::TM], bs[C::TN];
  auto read_frags = [&](const uint8_t* st) {
    uint32_t ar[C::TM], br[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++) {
      aq[i] = *reinterpret_cast<const uint4*>(st + a_code0 + i * 32 * 32);
      ar[i] = *reinterpret_cast<const uint16_t*>(st + a_sc0 + i * 32 * 4);
    }
#pragma unroll
    for (int j = 0; j < C::TN; j++) {
      bq[j] = *reinterpret_cast<const uint4*>(st + b_code0 + j * 32 * 32);
      br[j] = *reinterpret_cast<const uint16_t*>(st + b_sc0 + j * 32 * 4);
    }
#pragma unroll
    for (int i = 0; i < C::TM; i++) as[i] = scale_pair(ar[i]);
#pragma unroll
    for (int j = 0; j < C::TN; j++) bs[j] = scale_pair(br[j]);
  };

  // Prologue: stages 0, 1 and 2 in LDS, step 0 of stage 0 decoded.
  auto stage_k = [&](int64_t st) { return (st < KT ? st : KT - 1) * BK; };
#pragma unroll
  for (int st = 0; st < kStages - 1; st++) {
    load_regs(stage_k(st));
    load_dma(stage_k(st), buffer(st));
    sa.store_codes(buffer(st), tid);
    sa.store_scales(buffer(st) + oAS, tid);
    sb.store_codes(buffer(st) + oBC, tid);
    sb.store_scales(buffer(st) + oBS, tid);
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  read_frags(buffer(0));
  half8 af[C::TM], bf[2][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; i++) af[i] = decode8(aq[i].x, splat(as[i], 0));
#pragma unroll
  for (int j = 0; j < C::TN; j++) bf[0][j] = decode8(bq[j].x, splat(bs[j], 0));
  int b_next = 1, b_load = kStages - 1;  // buffers of stages kt+1 and kt+3

  for (int64_t kt = 0; kt < KT; kt++) {
    // Stage kt+3 (clamped: near the end the last stage is reloaded into an
    // idle buffer, which keeps the loop free of branches).
    const int64_t kl = stage_k(kt + kStages - 1);
    uint8_t* dst = buffer(b_load);
    load_regs(kl);

#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int cur = s & 1, nxt = cur ^ 1;
      // Step s+1 of this stage, or step 0 of the next stage (read now).
      const int ns = s < 3 ? s + 1 : 0;
      if (s == 3) {
        // The compiler may make these LDS reads wait for every outstanding
        // LDS DMA; issuing stage kt+3's DMA only after them keeps that wait
        // to transfers issued an iteration ago or earlier.
        read_frags(buffer(b_next));
        load_dma(kl, dst);
        if (C::kFence) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < C::TM; i++) {
#pragma unroll
        for (int j = 0; j < C::TN; j++) {
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[cur][j], acc[i][j], 0, 0, 0);
          const int t = i * C::TN + j;
          bool any = false;
#pragma unroll
          for (int jj = 0; jj < C::TN; jj++)
            if (b_slot<C::TM, C::TN>(s, jj) == t) {
              bf[nxt][jj] = decode8(pick(bq[jj], ns), splat(bs[jj], ns >= 2));
              any = true;
            }
#pragma unroll
          for (int ii = 0; ii < C::TM; ii++)
            if (a_slot<C::TM, C::TN>(s, ii) == t) {
              af[ii] = decode8(pick(aq[ii], ns), splat(as[ii], ns >= 2));
              any = true;
            }
          // MN-major operands write stage kt+2 to LDS during steps 2 and 3.
          constexpr int kLast = C::TM * C::TN - 1;
          const bool st = (s == 2 && (t == kLast / 2 || t == kLast)) ||
                          (s == 3 && (t == kLast / 4 || t == (3 * kLast) / 4));
          if (s == 2 && t == kLast / 2) sa.store_codes(dst, tid);
          if (s == 2 && t == kLast) sa.store_scales(dst + oAS, tid);
          if (s == 3 && t == kLast / 4) sb.store_codes(dst + oBC, tid);
          if (s == 3 && t == (3 * kLast) / 4) sb.store_scales(dst + oBS, tid);
          if (C::kFence && (any || (st && (!AK || !BKM)))) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    b_next = b_next == kStages - 1 ? 0 : b_next + 1;
    b_load = b_load == kStages - 1 ? 0 : b_load + 1;
    // Stage kt+2, read in the next iteration, complete: this wave's DMA for
    // it was issued an iteration ago, so only this iteration's transfers may
    // still be in flight; then every wave's (barrier).
    if (n_scale_dma == 0)
      wait_vm_lgkm0<kCodeDma>();
    else if (n_scale_dma == 1)
      wait_vm_lgkm0<kCodeDma + 1>();
    else
      wait_vm_lgkm0<kCodeDma + 2>();
    __builtin_amdgcn_s_barrier();
  }
  // No transfer may still target this workgroup's LDS when it is reused.
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();

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
  gemm_tile<C, AK, BKM>(A, B, tm * C::BM, a.M, tn * C::BN, a.N, a.K, gs, a.C, a.c_bf16, a.N, lds);
}

// Persistent grouped kernel: every workgroup builds the prefix of per-group
// tile counts in LDS, then walks tiles blockIdx.x, +gridDim.x, ...
template <class C>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(GroupedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int32_t* prefix = reinterpret_cast<int32_t*>(lds + C::kLds);  // [groups + 1]
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

using Dense = Cfg<256, 256, 2, 4, false>;
using Grouped = Cfg<256, 256, 2, 4, false>;

template <class C, bool AK, bool BKM>
hipError_t launch_dense(const GemmArgs& a, hipStream_t st) {
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  const size_t smem = C::kLds;
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
  const size_t smem = C::kLds + sizeof(int32_t) * (size_t)(a.groups + 1);
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
