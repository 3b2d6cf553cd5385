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
//    by LDS DMA.  MN-major operands (the TN/NN layouts) also go by LDS DMA,
//    as stored rows of k, and are transposed by the LDS read itself
//    (ds_read_b64_tr_b4), which hands each lane 16 consecutive k of one
//    column.
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

// ---- staging: MN-major operands by LDS DMA, transposed when read ----------------------------
// The stage of an operand stored [K][W] is 64 stored rows (k) of the tile's
// 256 columns (mn): 64 x 128 code bytes.  16-byte unit c (32 columns) of
// stage row k lands in LDS unit 8k + (c ^ ((k >> 1) & 7)): the 16 rows that
// one transposing read gathers (below) then sit in 16 different 16-byte
// slots of a 256-byte span.  Columns past the operand's edge re-read its last
// valid unit (W is a multiple of 32), which only feeds unstored outputs.
// Scales of stage row kb (k-block k0/16 + kb) go to LDS bytes 256*kb: COL
// blocks as the tile's 256 bytes of that row; 2D blocks as the 4-byte words
// holding the row's (up to) 16 bytes for the tile, read from the aligned word
// at or below their start, so a reader adds that start's offset (0 or 2).
template <int ROWS, int NW, int SW0, int SWN>
struct DmaMN {
  static_assert(ROWS == 256, "a stage row of codes is 128 bytes, a scale row 256");
  static constexpr int kCodeChunks = BK * ROWS / 2 / 1024;
  static_assert(kCodeChunks % NW == 0, "code chunks must split over waves");
  static_assert(SWN == BK / 16, "one scale row per scale wave");
  static constexpr int CPW = kCodeChunks / NW;
  uint32_t coff[CPW];
  uint32_t soff;
  uint32_t crow, srow;  // bytes per stored code row, per scale row
  __amdgpu_buffer_rsrc_t crsrc, srsrc;
  int wave;

  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int lane, int wv) {
    wave = wv;
    const int64_t W = op.mn_total;
    const int64_t last_unit = W / 32 - 1;
    crow = (uint32_t)(W / 2);
#pragma unroll
    for (int q = 0; q < CPW; q++) {
      const int unit = 64 * (wave * CPW + q) + lane;  // LDS 16-byte unit of the stage
      const int k = unit >> 3;
      const int c = (unit & 7) ^ ((k >> 1) & 7);
      int64_t cg = mn0 / 32 + c;
      cg = cg < last_unit ? cg : last_unit;
      coff[q] = (uint32_t)(k * (W / 2) + 16 * cg);
    }
    const int kb = wave - SW0;  // meaningful on scale waves only
    if (op.block == kBlock2d) {
      const int64_t w16 = W / 16;
      const int64_t rel = kb * w16 + mn0 / 16;
      const int64_t rel4 = rel & ~(int64_t)3;
      const int64_t need = w16 - mn0 / 16 < 16 ? w16 - mn0 / 16 : 16;
      const int nd = (int)((rel - rel4 + need + 3) / 4);
      const int d = (lane & 7) < nd - 1 ? (lane & 7) : nd - 1;
      soff = (uint32_t)(rel4 + 4 * d);
      srow = (uint32_t)w16;
    } else {
      int64_t col = mn0 + 4 * lane;
      col = col < W - 4 ? col : W - 4;
      soff = (uint32_t)(kb * W + col);
      srow = (uint32_t)W;
    }
    (void)mn_lim;
    crsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.codes), 0,
                                              (int)(K * (W / 2)), kBufferFlags);
    srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.scales), 0,
                                              (int)((K / 16) * srow), kBufferFlags);
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds_codes, uint8_t* lds_scales) const {
#pragma unroll
    for (int q = 0; q < CPW; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, lds_codes + (wave * CPW + q) * 1024, 16,
                                               coff[q], (int)(k0 * crow), 0, 0);
    if (wave >= SW0 && wave < SW0 + SWN)  // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, lds_scales + (wave - SW0) * 256, 4, soff,
                                               (int)((k0 / 16) * srow), 0, 0);
  }
};

typedef int v2i32 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b4: in each group of 16 lanes, lane i receives nibble i of
// the 8-byte rows addressed by lanes 0..15 of its group, in lane order.
__device__ __forceinline__ v2i32 lds_read_tr4(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) v2i32*)(p));
}

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

// Per-operand staging, both layouts by LDS DMA.  OPB selects operand B's
// share of the scale waves (A uses the first half, B the second).  A
// fragment is what one lane multiplies in one 64-k stage: 32 nibbles of its
// row (row l%32 of the fragment, k = 32*(l/32) .. +32 of the stage; dword s
// holds the k of 16-k step s) and the two scale bytes of those k.
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
  int code0, sc0;  // this lane's LDS offsets for fragment 0
  __device__ __forceinline__ int scale_dma(int wave) const {
    return wave >= kSW0 && wave < kSW0 + kSW ? 1 : 0;
  }
  // row0: first row (of the tile) of this wave's fragments; fragment i
  // starts 32*i rows further.
  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int tid, int row0) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
    const int lane = tid & 63;
    code0 = code_addr(row0 + (lane & 31), lane >> 5);  // rows step by 32: same swizzle
    sc0 = 4 * (row0 + (lane & 31)) + 2 * (lane >> 5);
  }
  __device__ __forceinline__ void load_dma(int64_t k0, uint8_t* codes, uint8_t* scales) {
    d.issue(k0, codes, scales);
  }
  __device__ __forceinline__ void frag(const uint8_t* codes, const uint8_t* scales, int i,
                                       uint4& q, uint32_t& sc) const {
    q = *reinterpret_cast<const uint4*>(codes + code0 + i * 32 * 32);
    sc = *reinterpret_cast<const uint16_t*>(scales + sc0 + i * 32 * 4);
  }
};

template <int ROWS, class C, int OPB>
struct Staging<false, ROWS, C, OPB> {
  static constexpr int kSW = BK / 16;  // scale waves: one per k-block row
  static_assert(kSW <= C::NW, "one scale row per wave at most");
  static constexpr int kSW0 = (2 * kSW <= C::NW) ? OPB * kSW : 0;
  DmaMN<ROWS, C::NW, kSW0, kSW> d;
  static constexpr int kCodeDma = DmaMN<ROWS, C::NW, kSW0, kSW>::CPW;
  // Lane l (group g = l/16, j = l%16, half h = l/32) addresses, for read
  // r = 0, 1, stage row k = 32h + 16r + j at the 8 bytes of columns
  // [row0 + 32i + 16(g&1), +16): it receives the 16 k of its own column.
  uint32_t tr_base[2];
  int tr_c[2];
  int sc_off[2], sc_step;
  __device__ __forceinline__ int scale_dma(int wave) const {
    return wave >= kSW0 && wave < kSW0 + kSW ? 1 : 0;
  }
  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int tid, int row0) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
    const int lane = tid & 63;
    const int g = lane >> 4, j = lane & 15, h = lane >> 5;
    const int c0 = row0 / 32;  // a multiple of the fragment count: c0 + i == c0 ^ i
    const bool two_d = op.block == kBlock2d;
    const int64_t w16 = op.mn_total / 16;
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const int k = 32 * h + 16 * r + j;
      tr_base[r] = 128 * k + 8 * (g & 1);
      tr_c[r] = c0 ^ ((k >> 1) & 7);
      const int kb = 2 * h + r;
      sc_off[r] = two_d ? 256 * kb + (int)((kb * w16 + mn0 / 16) & 3) + (row0 + (lane & 31)) / 16
                        : 256 * kb + row0 + (lane & 31);
    }
    sc_step = two_d ? 2 : 32;
  }
  __device__ __forceinline__ void load_dma(int64_t k0, uint8_t* codes, uint8_t* scales) {
    d.issue(k0, codes, scales);
  }
  __device__ __forceinline__ void frag(const uint8_t* codes, const uint8_t* scales, int i,
                                       uint4& q, uint32_t& sc) const {
    const v2i32 lo = lds_read_tr4(codes + tr_base[0] + 16 * (tr_c[0] ^ i));
    const v2i32 hi = lds_read_tr4(codes + tr_base[1] + 16 * (tr_c[1] ^ i));
    q = uint4{(uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)hi.x, (uint32_t)hi.y};
    sc = (uint32_t)scales[sc_off[0] + i * sc_step] |
         ((uint32_t)scales[sc_off[1] + i * sc_step] << 8);
  }
};

// One output tile: C[m0 : m0+BM) x [n0 : n0+BN) restricted to rows < m_lim,
// cols < N, using lds (kLds bytes).
//
// Software pipeline over 64-k stages (stage s lives in LDS buffer s % 4):
//  * iteration kt issues stage kt+3's LDS DMA during its last step;
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
  sa.init(A, m0, m_lim, K, tid, wm * (C::BM / C::WM));
  sb.init(B, n0, N, K, tid, wn * (C::BN / C::WN));
  // DMA instructions this wave issues per stage (wave-uniform): the code
  // chunks plus one scale chunk per operand whose scales this wave moves.
  constexpr int kCodeDma = Staging<AK, C::BM, C, 0>::kCodeDma + Staging<BKM, C::BN, C, 1>::kCodeDma;
  const int n_scale_dma = sa.scale_dma(wave) + sb.scale_dma(wave);
  const int64_t KT = K / BK;

  constexpr int oAS = C::kACodes, oBC = C::kACodes + C::kAScales,
                oBS = C::kACodes + C::kAScales + C::kBCodes;

  auto buffer = [&](int idx) { return lds + idx * C::kStage; };
  auto load_dma = [&](int64_t k0, uint8_t* dst) {
    sa.load_dma(k0, dst, dst + oAS);
    sb.load_dma(k0, dst + oBC, dst + oBS);
  };

  uint4 aq[C::TM], bq[C::TN];
  half2 as[C::TM], bs[C::TN];
  auto read_frags = [&](const uint8_t* st) {
    uint32_t ar[C::TM], br[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++) sa.frag(st, st + oAS, i, aq[i], ar[i]);
#pragma unroll
    for (int j = 0; j < C::TN; j++) sb.frag(st + oBC, st + oBS, j, bq[j], br[j]);
#pragma unroll
    for (int i = 0; i < C::TM; i++) as[i] = scale_pair(ar[i]);
#pragma unroll
    for (int j = 0; j < C::TN; j++) bs[j] = scale_pair(br[j]);
  };

  // Prologue: stages 0, 1 and 2 in LDS, step 0 of stage 0 decoded.
  auto stage_k = [&](int64_t st) { return (st < KT ? st : KT - 1) * BK; };
#pragma unroll
  for (int st = 0; st < kStages - 1; st++) load_dma(stage_k(st), buffer(st));
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
          if (C::kFence && any) __builtin_amdgcn_sched_barrier(0);
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

// Tile order: groups of 8 M-tiles sweep N, so tiles that run together share
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

// Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b % 8) and
// every XCD has its own L2: give each XCD a contiguous run of the tile order,
// so the tiles running together on one XCD share panels in its L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t total) {
  constexpr int64_t kXcds = 8;
  const int64_t per = total / kXcds;
  return b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
}

template <class C, bool AK, bool BKM>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  int64_t tm, tn;
  tile_coords(xcd_tile(blockIdx.x, ntm * ntn), ntm, ntn, tm, tn);
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
