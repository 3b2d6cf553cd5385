// gemm.hip -- NVFP4 GEMMs (dense NT/NN/TN and grouped) for gfx950.
//
// Design (the operation: Super summary, Infra table; Ultra report 2.2):
//  * CDNA4's FP4 matrix instructions take power-of-two scales per 32
//    elements, which cannot carry an E4M3 scale per 16 elements.  Instead
//    every element is decoded to fp16 -- exact: val(code) has 2 significant
//    bits, an E4M3 scale 4, so their product has at most 6 and lies in
//    [2^-10, 2688] -- and fed to v_mfma_f32_32x32x16_f16 with fp32
//    accumulation.
//  * Codes and scale bytes (0.5625 B per element) reach LDS by LDS DMA
//    (buffer loads that write LDS directly), one stage of BK = 128 (or 64)
//    k at a time, in a ring of three stage buffers.  K-major operands keep
//    their rows: BK/2 code bytes per row in 16-byte units whose order is
//    swizzled per row, and BK/16 scale bytes per row.  MN-major operands
//    (the TN/NN layouts) are staged as stored, rows of k, and transposed by
//    the LDS read itself (ds_read_b64_tr_b4), which hands each lane 16
//    consecutive k of one column.
//  * Each wave decodes only the fragments it multiplies.  Lane l owns row
//    l%32 of a 32-row fragment and, in each 64-k half of a stage, the 32 k
//    at 32*(l/32); per 16-k MFMA step it decodes 8 nibbles with
//    v_cvt_scalef32_pk_f16_fp4 and scales them by the fp16 value of their
//    E4M3 scale byte (v_cvt_scalef32_pk_f16_fp8, then v_pk_mul_f16; both
//    converts with scale 1, since their scale operand only applies a power
//    of two).  The k order inside an MFMA is a permutation shared by A and
//    B, so every output is the same sum whatever the tile shape or depth.
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
typedef int v2i32 __attribute__((ext_vector_type(2)));

template <int BM_, int BN_, int WM_, int WN_, int BK_, int PK_ = 64>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, PK = PK_;
  static_assert(BM % 64 == 0 && BN % 64 == 0 && BM <= 256 && BN <= 256, "tile sizes");
  static_assert(BK == 64 || BK == 128, "stage depth");
  static_assert((PK == 64 || PK == 128) && BK % PK == 0, "phase depth");
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM / 32;  // 32x32 MFMA tiles per wave along M
  static constexpr int TN = BN / WN / 32;
  static constexpr int H = BK / 64;        // 64-k halves per stage
  static constexpr int NPH = BK / PK;      // phases (barrier intervals) per stage
  static constexpr int PH = PK / 16;       // MFMA steps per phase
  static constexpr int STEPS = BK / 16;    // MFMA steps per stage
  static constexpr int RB = BK / 2;        // code bytes per row per stage
  static constexpr int SB = BK / 16;       // scale bytes per row (k-blocks) per stage
  // Scales: SB bytes per row (K-major) or SB rows of 256 bytes (MN-major).
  static constexpr int kACodes = BM * RB, kAScales = BM * SB > SB * 256 ? BM * SB : SB * 256;
  static constexpr int kBCodes = BN * RB, kBScales = BN * SB > SB * 256 ? BN * SB : SB * 256;
  static constexpr int kStage = kACodes + kAScales + kBCodes + kBScales;  // one raw stage
  static constexpr int kA16 = BM * PK * 2;  // A of one phase, decoded to fp16
};

// Operand view for one tile: base pointers and the strides of its stored
// layout.  K-major: stored [MN][K]; MN-major: stored [K][MN] (mn_total wide).
struct OpView {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t mn_total;  // stored width of an MN-major operand
  int block;
};

// s_waitcnt with vmcnt <= N and lgkmcnt == 0 (expcnt not waited on); N = 63
// does not wait for vector memory.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// ---- K-major stage layout --------------------------------------------------------------------
// Row r of a stage holds RB code bytes as UR = RB/16 units of 16 bytes; unit
// u (k = 32u .. 32u+31 of the stage) sits in slot u ^ kmaj_swz(r).  A 16-byte
// LDS read is served 16 lanes at a time over a 256-byte bank window, and the
// 16 lanes of a fragment read take 16 consecutive rows and the same unit:
// the swizzle spreads them over 16 distinct 16-byte slots of the window.
template <int RB>
__device__ __forceinline__ int kmaj_swz(int row) {
  static_assert(RB == 32 || RB == 64, "row bytes");
  return RB == 32 ? (row >> 3) & 1 : (row >> 2) & 3;
}

template <int RB>
__device__ __forceinline__ int kmaj_code_addr(int row, int unit) {
  return row * RB + 16 * (unit ^ kmaj_swz<RB>(row));
}

// ---- staging plans -----------------------------------------------------------------------------
// buffer_load_dword{,x4} ... lds moves 4 or 16 bytes per lane into LDS at
// (wave-uniform base + size * lane).  Code chunks (1 KiB: 64 lanes x 16
// bytes) go to wave c % NW; scale chunks (256 bytes: 64 lanes x 4 bytes) to
// wave (W0 + j) % NW.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 dword3)

template <int NW, int CHUNKS, int SCHUNKS, int W0>
struct DmaPlan {
  static constexpr int CPW = (CHUNKS + NW - 1) / NW;   // most code chunks on one wave
  static constexpr int SPW = (SCHUNKS + NW - 1) / NW;  // most scale chunks on one wave
  __device__ __forceinline__ static bool code_on(int wave, int q) {
    return wave + q * NW < CHUNKS;
  }
  __device__ __forceinline__ static int scale_chunk(int wave, int q) {
    return ((wave - W0) % NW + NW) % NW + q * NW;  // valid if < SCHUNKS
  }
  __device__ __forceinline__ static int count(int wave) {
    int n = 0;
#pragma unroll
    for (int q = 0; q < CPW; q++) n += code_on(wave, q) ? 1 : 0;
#pragma unroll
    for (int q = 0; q < SPW; q++) n += scale_chunk(wave, q) < SCHUNKS ? 1 : 0;
    return n;
  }
};

// ---- staging: K-major operands ----------------------------------------------------------------
// The lane's source offset is chosen so that the LDS image is the swizzled
// layout above.  A row past the operand's edge re-reads the last valid row
// (always in bounds): row i of A only reaches row i of C, row j of B only
// column j, so such rows only feed outputs that are never stored.
template <class C, int ROWS, int W0>
struct DmaK {
  static constexpr int RB = C::RB, SB = C::SB, UR = RB / 16;
  static constexpr int kCodeChunks = ROWS * RB / 1024;
  static constexpr int kScaleChunks = ROWS * SB / 256;
  using Plan = DmaPlan<C::NW, kCodeChunks, kScaleChunks, W0>;
  uint32_t coff[Plan::CPW];
  uint32_t soff[Plan::SPW];
  __amdgpu_buffer_rsrc_t crsrc, srsrc;
  int wave;

  __device__ __forceinline__ int count(int w) const { return Plan::count(w); }

  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int lane, int wv) {
    wave = wv;
    const int64_t kc = K / 2, ks = K / 16;
#pragma unroll
    for (int q = 0; q < Plan::CPW; q++) {
      const int row = (1024 / RB) * (wave + q * C::NW) + lane / UR;
      const int unit = (lane % UR) ^ kmaj_swz<RB>(row);
      const int64_t mn = mn0 + row < mn_lim ? mn0 + row : mn_lim - 1;
      coff[q] = (uint32_t)((mn - mn0) * kc + 16 * unit);
    }
    // The buffer ranges cover the tile's own rows (at most ROWS of them), so
    // they fit 31 bits whatever the operand's size (K < 2^24).
    const int64_t rows_t = mn_lim - mn0 < ROWS ? mn_lim - mn0 : ROWS;
    const bool two_d = op.block == kBlock2d;
    const int64_t sbase = two_d ? (mn0 / 16) * ks : mn0 * ks;
    const int64_t slim = two_d ? ((mn0 + rows_t + 15) / 16) * ks : (mn0 + rows_t) * ks;
#pragma unroll
    for (int q = 0; q < Plan::SPW; q++) {
      // Row SB bytes = SB/4 lanes of 4 bytes (the stage's k-blocks).
      const int j = Plan::scale_chunk(wave, q);
      const int row = (256 / SB) * j + lane / (SB / 4);
      const int part = lane % (SB / 4);
      const int64_t mn = mn0 + row < mn_lim ? mn0 + row : mn_lim - 1;
      soff[q] = (uint32_t)((two_d ? (mn / 16) * ks : mn * ks) - sbase + 4 * part);
    }
    crsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.codes + mn0 * kc), 0,
                                              (int)(rows_t * kc), kBufferFlags);
    srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.scales + sbase), 0,
                                              (int)(slim - sbase), kBufferFlags);
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds_codes, uint8_t* lds_scales) const {
#pragma unroll
    for (int q = 0; q < Plan::CPW; q++)
      if (Plan::code_on(wave, q))  // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, lds_codes + (wave + q * C::NW) * 1024, 16,
                                                 coff[q], (int)(k0 / 2), 0, 0);
#pragma unroll
    for (int q = 0; q < Plan::SPW; q++) {
      const int j = Plan::scale_chunk(wave, q);
      if (j < kScaleChunks)  // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, lds_scales + j * 256, 4, soff[q],
                                                 (int)(k0 / 16), 0, 0);
    }
  }
};

// ---- staging: MN-major operands, transposed when read ------------------------------------------
// The stage of an operand stored [K][W] is BK stored rows (k) of the tile's
// ROWS columns (mn): rows of U = ROWS/32 16-byte units.  Unit c of stage row
// k lands in LDS unit U*k + mn_swz(c, k).  A transposing read (below)
// gathers the same unit of 16 consecutive rows; the swizzle puts them in 16
// different 16-byte slots of a 256-byte span (U = 8: XOR with bits 1..3 of
// k; U = 6: 6k already spreads 8 rows, XOR with bit 3 of k separates the
// two octets).  Columns past the operand's edge re-read its last valid unit
// (W is a multiple of 32), which only feeds unstored outputs.
// Scales of stage row kb (k-block k0/16 + kb) go to LDS bytes 256*kb: COL
// blocks as the tile's ROWS bytes of that row; 2D blocks as the 4-byte words
// holding the row's (up to) ROWS/16 bytes for the tile, read from the aligned
// word at or below their start, so a reader adds that start's offset (0 or
// 2).
template <int U>
__device__ __forceinline__ int mn_swz(int c, int k) {
  static_assert(U == 8 || U == 6, "units per stage row");
  return U == 8 ? c ^ ((k >> 1) & 7) : c ^ ((k >> 3) & 1);
}

template <class C, int ROWS, int W0>
struct DmaMN {
  static constexpr int U = ROWS / 32;  // 16-byte units per stage row
  static constexpr int kCodeChunks = C::BK * U / 64;
  static constexpr int kScaleChunks = C::SB;  // one per k-block row
  static_assert(ROWS <= 256, "a scale row holds at most 256 bytes");
  using Plan = DmaPlan<C::NW, kCodeChunks, kScaleChunks, W0>;
  uint32_t coff[Plan::CPW];
  uint32_t soff[Plan::SPW];
  uint32_t crow, srow;  // bytes per stored code row, per scale row
  __amdgpu_buffer_rsrc_t crsrc, srsrc;
  int wave;

  __device__ __forceinline__ int count(int w) const { return Plan::count(w); }

  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t, int64_t K,
                                       int lane, int wv) {
    wave = wv;
    const int64_t W = op.mn_total;
    const int64_t last_unit = W / 32 - 1;
    crow = (uint32_t)(W / 2);
#pragma unroll
    for (int q = 0; q < Plan::CPW; q++) {
      const int unit = 64 * (wave + q * C::NW) + lane;  // LDS 16-byte unit of the stage
      const int k = unit / U;
      const int c = mn_swz<U>(unit % U, k);
      int64_t cg = mn0 / 32 + c;
      cg = cg < last_unit ? cg : last_unit;
      coff[q] = (uint32_t)(k * (W / 2) + 16 * cg);
    }
    const bool two_d = op.block == kBlock2d;
    srow = (uint32_t)(two_d ? W / 16 : W);
#pragma unroll
    for (int q = 0; q < Plan::SPW; q++) {
      const int kb = Plan::scale_chunk(wave, q);  // meaningful if < kScaleChunks
      if (two_d) {
        const int64_t w16 = W / 16;
        const int64_t rel = kb * w16 + mn0 / 16;
        const int64_t rel4 = rel & ~(int64_t)3;
        const int64_t need = w16 - mn0 / 16 < ROWS / 16 ? w16 - mn0 / 16 : ROWS / 16;
        const int nd = (int)((rel - rel4 + need + 3) / 4);
        const int d = (lane & 7) < nd - 1 ? (lane & 7) : nd - 1;
        soff[q] = (uint32_t)(rel4 + 4 * d);
      } else {
        int64_t col = mn0 + 4 * lane;
        col = col < W - 4 ? col : W - 4;
        soff[q] = (uint32_t)(kb * W + col);
      }
    }
    crsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.codes), 0,
                                              (int)(K * (W / 2)), kBufferFlags);
    srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.scales), 0,
                                              (int)((K / 16) * srow), kBufferFlags);
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds_codes, uint8_t* lds_scales) const {
#pragma unroll
    for (int q = 0; q < Plan::CPW; q++)
      if (Plan::code_on(wave, q))  // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, lds_codes + (wave + q * C::NW) * 1024, 16,
                                                 coff[q], (int)(k0 * crow), 0, 0);
#pragma unroll
    for (int q = 0; q < Plan::SPW; q++) {
      const int kb = Plan::scale_chunk(wave, q);
      if (kb < kScaleChunks)  // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, lds_scales + kb * 256, 4, soff[q],
                                                 (int)((k0 / 16) * srow), 0, 0);
    }
  }
};

// ds_read_b64_tr_b4: in each group of 16 lanes, lane i receives nibble i of
// the 8-byte rows addressed by lanes 0..15 of its group, in lane order.
__device__ __forceinline__ v2i32 lds_read_tr4(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) v2i32*)(p));
}

// ---- decode -----------------------------------------------------------------------------------
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

// Two bf16 (round to nearest even: v_cvt_pk_bf16_f32) packed low | high << 16.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(__bf16 lo, __bf16 hi) {
  const bf16x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Value of the partner lane (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float xor1_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// ---- per-operand staging ------------------------------------------------------------------------
// A fragment half is what one lane multiplies in one 64-k half of a stage:
// 32 nibbles of its row (row l%32 of the fragment, k = 32*(l/32) .. +32 of
// the half; dword s holds the k of 16-k step s) and the two scale bytes of
// those k.  W0 places the operand's scale chunks on the waves (B after A's).
template <bool KMAJOR, int ROWS, class C, int W0, int NF>
struct Staging;

template <int ROWS, class C, int W0, int NF>
struct Staging<true, ROWS, C, W0, NF> {
  using Dma = DmaK<C, ROWS, W0>;
  static constexpr int kScaleChunks = Dma::kScaleChunks;
  Dma d;
  int code0[C::H];  // this lane's LDS code offsets for fragment 0, per half
  int sc0;          // this lane's LDS scale offset for fragment 0, half 0
  __device__ __forceinline__ int dma_count(int wave) const { return d.count(wave); }
  // row0: first row (of the tile) of this wave's fragments; fragment i
  // starts 32*i rows further (which keeps the row swizzle).
  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int tid, int row0) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
    const int lane = tid & 63;
    const int row = row0 + (lane & 31);
#pragma unroll
    for (int hs = 0; hs < C::H; hs++)
      code0[hs] = kmaj_code_addr<C::RB>(row, 2 * hs + (lane >> 5));
    sc0 = C::SB * row + 2 * (lane >> 5);
  }
  // Point the transfers at another tile (the LDS offsets do not change).
  __device__ __forceinline__ void retarget(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                           int tid) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
  }
  __device__ __forceinline__ void load_dma(int64_t k0, uint8_t* codes, uint8_t* scales) {
    d.issue(k0, codes, scales);
  }
  __device__ __forceinline__ void frag(const uint8_t* codes, const uint8_t* scales, int i, int hs,
                                       uint4& q, uint32_t& sc) const {
    q = *reinterpret_cast<const uint4*>(codes + code0[hs] + i * 32 * C::RB);
    sc = *reinterpret_cast<const uint16_t*>(scales + sc0 + 4 * hs + i * 32 * C::SB);
  }
  // Fragment 0 of half hs given at run time (wave-uniform).
  __device__ __forceinline__ void frag_h(const uint8_t* codes, const uint8_t* scales, int hs,
                                         uint4& q, uint32_t& sc) const {
    int off = code0[0];
#pragma unroll
    for (int x = 1; x < C::H; x++)
      if (hs == x) off = code0[x];
    q = *reinterpret_cast<const uint4*>(codes + off);
    sc = *reinterpret_cast<const uint16_t*>(scales + sc0 + 4 * hs);
  }
};

template <int ROWS, class C, int W0, int NF>
struct Staging<false, ROWS, C, W0, NF> {
  using Dma = DmaMN<C, ROWS, W0>;
  static constexpr int kScaleChunks = Dma::kScaleChunks;
  static constexpr int U = ROWS / 32;
  Dma d;
  // Lane l (group g = l/16, half h = l/32) addresses, for stage half hs and
  // read r = 0, 1, stage row k = 64hs + 32h + 16r + l%16 at the 8 bytes of
  // columns [row0 + 32i + 16(g&1), +16) of fragment i: it receives the 16 k
  // of its own column.  The row swizzle only depends on k mod 16, so hs and
  // r only add constants.  The lane's scale bytes are those of k-blocks
  // kb = 4hs + 2h + r of its column.
  int col[NF];   // LDS offset of the tr-read row for hs = 0, r = 0
  int scb;       // LDS offset of the scale byte for fragment 0, hs = 0, r = 0
  int scb1;      // the same for r = 1
  int sc_step;   // from fragment i to i + 1 (wave-uniform)
  __device__ __forceinline__ int dma_count(int wave) const { return d.count(wave); }
  __device__ __forceinline__ void init(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                       int tid, int row0) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
    const int lane = tid & 63;
    const int g = lane >> 4, h = lane >> 5;
    const int krow0 = 32 * h + (lane & 15);
    const int sw = mn_swz<U>(0, krow0);
    const bool two_d = op.block == kBlock2d;
    const int64_t w16 = op.mn_total / 16;
    // 2D scale rows start 2 bytes past a 4-byte word on odd k-block rows when
    // w16 = 2 mod 4 (every other start offset is 0; see the DMA).
    const int m1 = two_d && (w16 & 3) == 2 ? 2 : 0;
    sc_step = two_d ? 2 : 32;
    scb = 256 * 2 * h + (two_d ? (row0 + (lane & 31)) / 16 : row0 + (lane & 31));
    scb1 = scb + 256 + m1;
#pragma unroll
    for (int i = 0; i < NF; i++) col[i] = 16 * (U * krow0 + ((row0 / 32 + i) ^ sw)) + 8 * (g & 1);
  }
  __device__ __forceinline__ void retarget(const OpView& op, int64_t mn0, int64_t mn_lim, int64_t K,
                                           int tid) {
    d.init(op, mn0, mn_lim, K, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6));
  }
  __device__ __forceinline__ void load_dma(int64_t k0, uint8_t* codes, uint8_t* scales) {
    d.issue(k0, codes, scales);
  }
  __device__ __forceinline__ void frag(const uint8_t* codes, const uint8_t* scales, int i, int hs,
                                       uint4& q, uint32_t& sc) const {
    const uint8_t* p = codes + col[i];
    const v2i32 lo = lds_read_tr4(p + 16 * U * 64 * hs);
    const v2i32 hi = lds_read_tr4(p + 16 * U * (64 * hs + 16));
    q = uint4{(uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)hi.x, (uint32_t)hi.y};
    // Two plain per-lane offsets (not one plus a distance between them):
    // then the compiler can tell these reads from a transfer into the other
    // stage buffer, and does not wait for it.
    const int d = i * sc_step + 1024 * hs;
    sc = (uint32_t)scales[scb + d] | ((uint32_t)scales[scb1 + d] << 8);
  }
};

// LDS buffers of one workgroup: two raw stages (codes and scale bytes as
// staged by LDS DMA) and two fp16 images of A, each one 64-k half.  They are
// separate variables so that the compiler can tell a read of one buffer from
// an LDS DMA into another.
struct TileLds {
  uint8_t* raw[2];
  uint8_t* a16[2];
};

// fp16 image of A for one phase of PK k: row r holds PK halves as PK/8 units
// of 16 bytes (unit v = k 8v .. 8v+7); unit v sits in a swizzled slot.  A
// fragment read or write touches one unit of consecutive rows: 16-byte reads
// are served 16 lanes (rows) at a time over a 256-byte bank window, 16-byte
// writes 8 lanes at a time over 128 bytes.  PK = 64 (128-byte rows): slot
// v ^ (r & 7) ^ ((r >> 3) & 1) puts any 8 aligned rows in distinct slots and
// any 16 in distinct (row parity, slot) pairs; PK = 128 (256-byte rows):
// slot v ^ (r & 15) puts any 16 aligned rows in distinct slots.
template <int PK>
__device__ __forceinline__ int a16_addr(int row, int unit) {
  return PK == 64 ? row * 128 + 16 * (unit ^ (row & 7) ^ ((row >> 3) & 1))
                  : row * 256 + 16 * (unit ^ (row & 15));
}

// One output tile: C[m0 : m0+BM) x [n0 : n0+BN) restricted to rows < m_lim
// (and columns < N); C points at row 0 of the tile's row coordinates.
struct TileDesc {
  OpView A, B;
  int64_t m0, m_lim, n0;
  float gscale;
  void* C;
};

// The output tiles of a workgroup, one after another, as one pipeline of
// stages (stage g = stage g % KT of tile g / KT), so that the next tile's
// first stages are fetched and decoded while the current one finishes.
//
// Work is split in phases of 64 k (H = BK/64 phases per stage).  In phase p:
//  * every wave multiplies its share of the tile in 4 steps of 16 k: A
//    fragments come ready-made from the fp16 image a16[p%2] (read one step
//    ahead); B fragments are decoded by the wave itself from registers, one
//    step ahead;
//  * every wave also decodes its 32 rows of A for phase p+1 (one fragment
//    half: 32 nibbles and 2 scale bytes per lane, read from the raw stage)
//    into a16[(p+1)%2], one 8-k dword per half step from the end of the
//    first step on -- so each A element is decoded once per workgroup
//    instead of once per wave that multiplies it;
//  * the last phase of a stage reads the next stage's B fragments (both
//    halves) into registers;
//  * a barrier precedes the last step: a16[(p+1)%2] is then complete and
//    every read of a16[p%2] done (the last step's A is already in
//    registers), so the last step reads the first fragments of phase p+1.
// Raw stage g is used during phases H*g - 1 .. H*g + H - 2 (its A decoded
// for phases H*g .. H*g+H-1; its B read in the last step of phase H*g - 1),
// so its buffer is refilled with stage g+2 at the start of phase H*g + H - 1,
// and the barrier of phase H*(g+1) + H - 2 waits for that transfer.  After a
// tile's last stage its accumulators are stored and cleared.
//
// Src: count() tiles, get(j) -> TileDesc of the j-th (wave-uniform); kSingle
// when there is always exactly one (its store then follows the loop).
template <class C, bool AK, bool BKM, class Src>
__device__ __forceinline__ void gemm_tiles(const Src& src, int64_t N, int64_t K, bool c_bf16,
                                           bool c_acc, int64_t ldc, const TileLds& L) {
  constexpr int H = C::H, TM = C::TM, TN = C::TN;
  const int64_t NJ = src.count();
  if (NJ <= 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // The A image of a phase is RBLK row blocks of 32 rows, each PQ 64-k halves
  // of 4 dwords (8 k) per lane.  With at least as many row blocks as waves,
  // wave w decodes row block w whole (and none when w >= RBLK).  With fewer
  // row blocks than waves, and the waves a multiple of them, wave w decodes
  // AD consecutive dwords (within one half) of row block w % RBLK: every wave
  // then takes part, which keeps the step code free of a branch on it.
  constexpr int RBLK = C::BM / 32;
  constexpr int PQ = C::PK / 64;  // 64-k halves per phase
  constexpr int SPLIT = RBLK < C::NW && C::NW % RBLK == 0 ? C::NW / RBLK : 1;
  constexpr bool kSplitA = SPLIT > 1 && SPLIT >= PQ && (4 * PQ) % SPLIT == 0;
  constexpr int AD = kSplitA ? 4 * PQ / SPLIT : 4 * PQ;  // dwords per wave per phase
  const bool decodes_a = kSplitA || RBLK >= C::NW || wave < RBLK;
  const int a_rb = kSplitA ? wave % RBLK : wave;      // row block this wave decodes
  const int a_i0 = kSplitA ? (wave / RBLK) * AD : 0;  // its first dword (4 * half + dword)
  // Stages per tile.  K need not be a multiple of BK: the operands' buffer
  // ranges end at K, so the rows of a last, partial stage past K read as
  // zeros and add nothing (K itself is a multiple of 16, whole blocks).
  const int64_t KT = (K + C::BK - 1) / C::BK;
  const int64_t GT = NJ * KT;

  f32x16 acc[TM][TN];
  auto clear_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  };
  clear_acc();

  // Tiles j0 and j0+1: the current one and the next, which transfers reach
  // when KT >= 2 (the caller's precondition when NJ > 1).  Separate
  // variables, not an array, so that they stay in registers.
  int64_t j0 = 0;
  TileDesc d0 = src.get(0);
  TileDesc d1 = src.get(1 < NJ ? 1 : NJ - 1);

  using SA = Staging<AK, C::BM, C, 0, 1>;
  constexpr int kBW0 = SA::kScaleChunks % C::NW;  // B's scale chunks after A's
  using SB = Staging<BKM, C::BN, C, kBW0, TN>;
  SA sa;
  SB sb;
  sa.init(d0.A, d0.m0, d0.m_lim, K, tid, 32 * a_rb);  // rows this wave decodes
  sb.init(d0.B, d0.n0, N, K, tid, wn * (C::BN / C::WN));

  constexpr int oAS = C::kACodes, oBC = C::kACodes + C::kAScales,
                oBS = C::kACodes + C::kAScales + C::kBCodes;

  // A16 offsets: fragment reads (row wm*BM/WM + 32i + lrow, unit 8q + 4*lhalf
  // + nd for 64-k half q of the phase and step nd of it) and this wave's
  // decode writes (row 32*a_rb + lrow, same units, dword c of its share); the
  // slot swizzle only depends on lrow.
  const int a_row0 = wm * (C::BM / C::WM);
  int a16_rd[PQ][4];
#pragma unroll
  for (int q = 0; q < PQ; q++)
#pragma unroll
    for (int nd = 0; nd < 4; nd++)
      a16_rd[q][nd] = a16_addr<C::PK>(a_row0 + lrow, 8 * q + 4 * lhalf + nd);
  const int a16_wr_delta = 2 * C::PK * (32 * a_rb - a_row0);  // wave-uniform
  int a16_wr[AD];
#pragma unroll
  for (int c = 0; c < AD; c++) {
    int v = a16_rd[0][0];
#pragma unroll
    for (int it = 0; it < 4 * PQ; it++)
      if (it == a_i0 + c) v = a16_rd[it / 4][it % 4];  // a_i0 == 0 unless split
    a16_wr[c] = v + a16_wr_delta;
  }

  // Transfer the next global stage into dst.  Transfers run two stages ahead
  // of the multiply, in order, so they move to the next tile (d1, as KT >= 2)
  // at its first stage.  dma_kt: k-stage of the next transfer within its
  // tile (a running count, not a division per stage).
  int64_t dma_kt = 0;
  auto load_dma = [&](uint8_t* dst) {
    if (!Src::kSingle && dma_kt == KT) {
      sa.retarget(d1.A, d1.m0, d1.m_lim, K, tid);
      sb.retarget(d1.B, d1.n0, N, K, tid);
      dma_kt = 0;
    }
    const int64_t k0 = dma_kt * C::BK;
    sa.load_dma(k0, dst, dst + oAS);
    sb.load_dma(k0, dst + oBC, dst + oBS);
    dma_kt++;
  };

  // This wave's raw B for one stage: per 64-k half and fragment, 32 nibbles
  // and two scale bytes (converted where they are used).
  uint4 bq[H][TN];
  uint32_t bsr[H][TN];
  auto read_b = [&](const uint8_t* st) {
#pragma unroll
    for (int hs = 0; hs < H; hs++)
#pragma unroll
      for (int j = 0; j < TN; j++) sb.frag(st + oBC, st + oBS, j, hs, bq[hs][j], bsr[hs][j]);
  };
  auto decode_b = [&](int hs, int j, int nd) {
    return decode8(pick(bq[hs][j], nd), splat(scale_pair(bsr[hs][j]), nd >= 2));
  };

  // This wave's raw A for one phase: per 64-k half, 32 nibbles and the two
  // scale bytes (stage halves h0 .. h0+PQ-1; split: only the half of its
  // share).  The bytes are converted where they are used, so that no
  // conversion waits for the read right after it.
  constexpr int NQ = kSplitA ? 1 : PQ;
  const int a_q = a_i0 / 4, a_nd0 = AD % 4 == 0 ? 0 : a_i0 % 4;
  uint4 dq[NQ];
  uint32_t dsr[NQ];
  auto read_a = [&](const uint8_t* st, int h0) {
    if constexpr (kSplitA) {
      sa.frag_h(st, st + oAS, h0 + a_q, dq[0], dsr[0]);
    } else {
#pragma unroll
      for (int q = 0; q < PQ; q++) sa.frag(st, st + oAS, 0, h0 + q, dq[q], dsr[q]);
    }
  };
  auto decode_a = [&](uint8_t* a16, int c) {  // dword c of this wave's share
    const int q = kSplitA ? 0 : c / 4, nd = kSplitA ? a_nd0 + c : c % 4;
    const half8 v = decode8(pick(dq[q], nd), splat(scale_pair(dsr[q]), nd >= 2));
    *reinterpret_cast<half8*>(a16 + a16_wr[c]) = v;
  };

  half8 af[2][TM], bf[2][TN];
  auto read_af = [&](const uint8_t* a16, int s, int buf) {
#pragma unroll
    for (int i = 0; i < TM; i++)
      af[buf][i] = *reinterpret_cast<const half8*>(a16 + a16_rd[s / 4][s % 4] +
                                                   i * 32 * 2 * C::PK);
  };

  // Epilogue of tile d0.  32x32 accumulator layout: lane l holds column
  // l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  bf16: lanes l and
  // l^1 hold neighbouring columns of the same rows; they swap one value per
  // row pair so that the even lane stores rows r (r even) and the odd lane
  // rows r+1, two columns (4 bytes) at a time.  Stores go through a buffer
  // resource based at the tile's first row, with the lane's offset in the
  // vector operand and the row step of element r (wave-uniform) in the
  // scalar one; a lane whose element lies past the last row or column gets
  // a vector offset beyond the resource's range, and the hardware drops that
  // store -- no branches, full tile or not.  The offsets fit 31 bits as
  // N < 2^21 (checked by the caller) and a tile has at most 256 rows.
  const int esz = c_bf16 ? 2 : 4;
  const int ldc32 = (int)ldc;
  auto store_tile = [&]() {
    // Kept apart from the surrounding pipeline code by the scheduler, which
    // would otherwise interleave the two and run out of registers.
    __builtin_amdgcn_sched_barrier(0);
    const TileDesc& t = d0;
    const bool odd = lane & 1;
    const int64_t left = t.m_lim - t.m0;  // rows of the tile that exist (32-bit compare below)
    const int rows_left = left < C::BM ? (int)left : C::BM;
    char* base = static_cast<char*>(t.C) + t.m0 * ldc * esz;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, kBufferFlags);
    constexpr uint32_t kDrop = 0x80000000u;  // past the range: not stored
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const int col = (int)t.n0 + wn * (C::BN / C::WN) + j * 32 + lrow;
        const int rl0 = a_row0 + i * 32 + 4 * lhalf;  // row within the tile, r = 0
        if (c_bf16) {
          const int lr = rl0 + (odd ? 1 : 0);
          const int c2 = odd ? col - 1 : col;  // c2 + 1 < N when c2 < N (N % 8 == 0)
          const uint32_t loff = (uint32_t)(lr * ldc32 + c2) * 2u;
          const bool cok = c2 < N;
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float v0 = acc[i][j][r] * t.gscale, v1 = acc[i][j][r + 1] * t.gscale;
            const float other = xor1_f(odd ? v0 : v1);
            const __bf16 lo = (__bf16)(odd ? other : v0), hi = (__bf16)(odd ? v1 : other);
            const int dr = 8 * (r >> 2) + (r & 3);
            const bool ok = cok && lr + dr < rows_left;
            __builtin_amdgcn_raw_buffer_store_b32(bf16_pair(lo, hi), rs, ok ? loff : kDrop,
                                                  dr * ldc32 * 2, 0);
          }
        } else {
          const uint32_t loff = (uint32_t)(rl0 * ldc32 + col) * 4u;
          const bool cok = col < N;
          // Accumulating output: C = RN32(C + RN32(acc * g)).  The loads take
          // the stores' offsets (past the range: 0, never stored), all issued
          // before the first add.
          float prev[16];
          if (c_acc) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int dr = 8 * (r >> 2) + (r & 3);
              const bool ok = cok && rl0 + dr < rows_left;
              prev[r] = __uint_as_float(
                  __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? loff : kDrop, dr * ldc32 * 4, 0));
            }
          }
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int dr = 8 * (r >> 2) + (r & 3);
            const bool ok = cok && rl0 + dr < rows_left;
            const float v = acc[i][j][r] * t.gscale;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c_acc ? prev[r] + v : v), rs,
                                                  ok ? loff : kDrop, dr * ldc32 * 4, 0);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: stages 0 and 1 in LDS, phase 0's A image, stage 0's B.
  load_dma(L.raw[0]);
  if (GT > 1) load_dma(L.raw[1]);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  if (decodes_a) {
    read_a(L.raw[0], 0);
#pragma unroll
    for (int c = 0; c < AD; c++) decode_a(L.a16[0], c);
  }
  read_b(L.raw[0]);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  read_af(L.a16[0], 0, 0);
#pragma unroll
  for (int j = 0; j < TN; j++) bf[0][j] = decode_b(0, j, 0);

  // One global stage g whose raw buffer is raw[PAR] (the next one's is
  // raw[1-PAR]); mul_kt is its k-stage within its tile.
  int64_t mul_kt = 0;
  auto stage = [&](int64_t g, auto par) {
    constexpr int PAR = decltype(par)::value;
    constexpr int NPH = C::NPH, PH = C::PH;
    static_assert(PH >= 4, "the A image is written by the middle of step PH/2 <= PH-2");
    uint8_t* raw_cur = L.raw[PAR];
    uint8_t* raw_nxt = L.raw[1 - PAR];
#pragma unroll
    for (int h = 0; h < NPH; h++) {
      // Phase p = NPH*g + h uses a16[p%2] and fills a16[(p+1)%2].
      const int ab = NPH == 2 ? h : PAR;  // (NPH*g + h) % 2 with g % 2 == PAR
      uint8_t* a16_cur = L.a16[ab];
      uint8_t* a16_nxt = L.a16[1 - ab];
      if (h == NPH - 1 && g + 2 < GT) load_dma(raw_cur);  // stage g+2; raw[PAR] is free
      // A of phase p+1: the next phase of this stage, or the first of the next.
      if (decodes_a) read_a(h + 1 < NPH ? raw_cur : raw_nxt, h + 1 < NPH ? (h + 1) * PQ : 0);
#pragma unroll
      for (int s = 0; s < PH; s++) {
        const int cur = s & 1, nxt = cur ^ 1;
        const bool last_step = s == PH - 1;
        const bool stage_end = last_step && h == NPH - 1;  // next step is the next stage's
        if (stage_end) read_b(raw_nxt);
        // B fragment of the next step: step sg + 1 of this stage (64-k half
        // (sg+1)/4, dword (sg+1)%4), or step 0 of the next (just read).
        const int sg = h * PH + s;
        const int nh = stage_end ? 0 : (sg + 1) / 4;
        const int nd = stage_end ? 0 : (sg + 1) % 4;
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
          for (int j = 0; j < TN; j++) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], bf[cur][j],
                                                               acc[i][j], 0, 0, 0);
            const int t = i * TN + j;
            // Raised wave priority while the first half of the step's MFMAs
            // issue: with both waves of a SIMD ready, the one feeding the
            // matrix core goes first (measured +1-3%).
            if (t == 0) __builtin_amdgcn_s_setprio(1);
            if (t == TM * TN / 2) __builtin_amdgcn_s_setprio(0);
            // A fragments of the next step: from this phase's image, or
            // (last step, after the barrier) step 0 of the next phase's.
            if (t == 0) {
              if (!last_step) read_af(a16_cur, s + 1, nxt);
              else read_af(a16_nxt, 0, nxt);
            }
            // B decodes after MFMAs j (2 + j when the raw registers were
            // just reloaded, to leave the LDS reads time to land).
#pragma unroll
            for (int jj = 0; jj < TN; jj++) {
              const int slot = stage_end ? (2 + jj < TM * TN ? 2 + jj : TM * TN - 1) : jj;
              if (slot == t) bf[nxt][jj] = decode_b(nh, jj, nd);
            }
            // The next phase's A image, dword c after half-step c + 1 (the
            // middle or the end of step (c+1)/2): the last write goes out
            // half a step or more before the barrier's wait.
            if (decodes_a && (t == TM * TN / 2 - 1 || t == TM * TN - 1)) {
              const int c = 2 * s + (t == TM * TN - 1 ? 1 : 0) - 1;
              if (c >= 0 && c < AD) decode_a(a16_nxt, c);
            }
          }
        }
        // The barrier sits before the phase's last step, whose operands are
        // already in registers: once past it, every wave has written its part
        // of the next image and read the last fragments of this one (so
        // a16_cur is free for the phase after), and the first reads of the
        // next image then land behind the last step's MFMAs instead of
        // stalling every wave after the barrier.  The next phase reads raw
        // stage g+1 (NPH = 2: from its start; NPH = 1: it is the stage
        // after), whose transfer is this wave's only one in flight here.
        if (s == PH - 2) {
          if ((h + 2) % NPH == 0)
            wait_vm_lgkm0<0>();
          else
            wait_vm_lgkm0<63>();
          __builtin_amdgcn_s_barrier();
        }
      }
    }
    if (!Src::kSingle && ++mul_kt == KT) {  // the tile's last stage: store, move on
      mul_kt = 0;
      store_tile();
      clear_acc();
      j0++;
      d0 = d1;
      d1 = src.get(j0 + 1 < NJ ? j0 + 1 : NJ - 1);
    }
  };

  int64_t g = 0;
  for (; g + 1 < GT; g += 2) {
    stage(g, std::integral_constant<int, 0>{});
    stage(g + 1, std::integral_constant<int, 1>{});
  }
  if (g < GT) stage(g, std::integral_constant<int, 0>{});
  if (Src::kSingle) store_tile();
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

// The workgroup's LDS buffers (static, so that each is its own variable).
#define NVFP4_TILE_LDS(C)                                            \
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw0[C::kStage]; \
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw1[C::kStage]; \
  __shared__ __attribute__((aligned(16))) uint8_t lds_a16a[C::kA16];   \
  __shared__ __attribute__((aligned(16))) uint8_t lds_a16b[C::kA16];   \
  const TileLds lds{{lds_raw0, lds_raw1}, {lds_a16a, lds_a16b}}

// One tile per workgroup.
struct DenseTile {
  static constexpr bool kSingle = true;
  TileDesc t;
  __device__ __forceinline__ int64_t count() const { return 1; }
  __device__ __forceinline__ TileDesc get(int64_t) const { return t; }
};

template <class C, bool AK, bool BKM>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs a) {
  NVFP4_TILE_LDS(C);
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  int64_t tm, tn;
  tile_coords(xcd_tile(blockIdx.x, ntm * ntn), ntm, ntn, tm, tn);
  DenseTile src;
  src.t.A = OpView{a.A.codes, a.A.scales, a.M, a.A.block};
  src.t.B = OpView{a.B.codes, a.B.scales, a.N, a.B.block};
  src.t.m0 = tm * C::BM;
  src.t.m_lim = a.M;
  src.t.n0 = tn * C::BN;
  src.t.gscale = *a.A.gdec * *a.B.gdec;
  src.t.C = a.C;
  gemm_tiles<C, AK, BKM>(src, a.N, a.K, a.c_bf16, a.c_acc, a.N, lds);
}

constexpr int kMaxGroups = 4096;  // the ABI's limit on groups
static_assert(kMaxGroups == 64 * 64, "the group search reads prefix[0 .. 4095]: 64 blocks of 64");

// Load of a value the kernel never writes, at a wave-uniform address, as a
// scalar load: it then counts on the scalar counter, so waiting for it does
// not also wait for the LDS transfers in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// The workgroup's tiles of the per-group tile list (group e owns tiles
// prefix[e] .. prefix[e+1]-1, column tile major, row tiles minor, so that
// neighbouring tiles share the group's B panel).  Round j runs tiles
// j*G .. j*G+G-1 (G = grid size) and hands neighbours to the same XCD:
// workgroup b (on XCD b % 8) takes slot (b % 8) * (G/8) + b / 8.
template <class C>
struct GroupedTiles {
  static constexpr bool kSingle = false;
  const GroupedArgs* a;
  const int32_t* prefix;  // LDS, [groups + 1]
  int64_t ntn;
  int32_t total;
  __device__ __forceinline__ int64_t slot() const {
    const int64_t G = gridDim.x, b = blockIdx.x;
    return G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
  }
  // The largest e with prefix[e] <= t (empty groups share a prefix value;
  // prefix[0] = 0 <= t), by the whole wave at once: prefix is nondecreasing,
  // so the entries <= t are a leading run, and two ballots over 64 entries
  // each (the first of every block of 64 groups, then the entries of one
  // block) count it.  The reads stay inside the LDS array (kMaxGroups + 1
  // entries); entries past the groups are left out of the counts.
  __device__ __forceinline__ int find_group(int32_t t) const {
    const int lane = threadIdx.x & 63;
    const int G = (int)a->groups;
    const int32_t v1 = prefix[lane << 6];
    const int c1 = __popcll(__ballot(lane < ((G + 63) >> 6) && v1 <= t)) - 1;
    const int i2 = (c1 << 6) + lane;
    const int32_t v2 = prefix[i2];
    return (c1 << 6) + __popcll(__ballot(i2 < G && v2 <= t)) - 1;
  }
  __device__ __forceinline__ int64_t count() const {
    const int64_t s = slot();
    return s < total ? (total - 1 - s) / gridDim.x + 1 : 0;
  }
  __device__ __forceinline__ TileDesc get(int64_t j) const {
    const int32_t t = (int32_t)(slot() + j * gridDim.x);
    const int64_t e = __builtin_amdgcn_readfirstlane(find_group(t));
    const int32_t lt = __builtin_amdgcn_readfirstlane(t - prefix[e]);
    const int64_t r0 = load_uniform(a->offsets + e), r1 = load_uniform(a->offsets + e + 1);
    const int64_t mtiles = (r1 - r0 + C::BM - 1) / C::BM;
    const int64_t nt = lt / mtiles, mt = lt % mtiles;
    const int64_t K = a->K, N = a->N;
    const int64_t b_scales_stride =
        a->B.block == kBlock2d ? (N / 16) * (K / 16) : N * (K / 16);
    TileDesc d;
    d.A = OpView{a->A.codes + r0 * (K / 2), a->A.scales + r0 * (K / 16), 0, kBlockRow};
    // B slice e: stored [N x K] (K-major) or [K x N] (MN-major, width N).
    d.B = OpView{a->B.codes + e * (N * K / 2), a->B.scales + e * b_scales_stride,
                 a->b_kmajor ? 0 : N, a->B.block};
    d.m0 = mt * C::BM;
    d.m_lim = r1 - r0;
    d.n0 = nt * C::BN;
    d.gscale = load_uniform(a->A.gdec) * load_uniform(a->B.gdec + e);
    d.C = a->c_bf16 ? (void*)(static_cast<uint16_t*>(a->C) + r0 * N)
                    : (void*)(static_cast<float*>(a->C) + r0 * N);
    return d;
  }
};

// Persistent grouped kernel: every workgroup builds the prefix of per-group
// tile counts in LDS, then walks tiles blockIdx.x, +gridDim.x, ...
template <class C, bool BKM>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(GroupedArgs a) {
  NVFP4_TILE_LDS(C);
  __shared__ int32_t prefix[kMaxGroups + 1];
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
  GroupedTiles<C> src{&a, prefix, ntn, total};
  if (a.K >= 2 * C::BK) {
    gemm_tiles<C, true, BKM>(src, a.N, a.K, a.c_bf16, a.c_acc, a.N, lds);
  } else {  // one stage per tile: no pipeline across tiles
    for (int64_t j = 0; j < src.count(); j++) {
      DenseTile one{src.get(j)};
      gemm_tiles<C, true, BKM>(one, a.N, a.K, a.c_bf16, a.c_acc, a.N, lds);
      __syncthreads();
    }
  }
}

// Grouped wgrad: for every group e, C_e [M x N] (fp32) = A_e^T B_e with A_e
// = A rows k_e .. k_{e+1}-1 (stored [tokens x M], COL blocks) and B_e the
// same rows of B ([tokens x N], COL blocks): the contraction runs over the
// group's own tokens, so K differs per group (a multiple of 16; zero gives
// C_e = 0).  Tiles (e, tm, tn) are spread over a persistent grid, XCD-aware
// (workgroup b on XCD b % 8 takes a contiguous run of the tile list), each
// a pipeline of its own (its stage count is its group's).  The operand views
// start at the group's first row, with buffer ranges that end at its last.
template <class C>
__global__ __launch_bounds__(C::NT) void grouped_wgrad_kernel(WgradArgs a) {
  NVFP4_TILE_LDS(C);
  const int64_t M = a.M, N = a.N;
  const int64_t mt = (M + C::BM - 1) / C::BM, nt = (N + C::BN - 1) / C::BN;
  const int64_t per = mt * nt, total = a.groups * per;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t slot = G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
  const float gscale = load_uniform(a.A.gdec) * load_uniform(a.B.gdec);
  // Tiles are visited in the order t = t0 * P mod total (a bijection when P
  // is coprime with total), so that workgroups running at the same time hold
  // different groups' tiles, of different depths: their output stores (256 KB
  // of fp32 per tile) then spread over time instead of arriving together.
  // 3% faster at the Super routed-expert shapes; the tiles are unchanged.
  const int64_t P = total % 7919 != 0 ? 7919 : 1;  // 7919 is prime
  for (int64_t t0 = slot; t0 < total; t0 += G) {
    const int64_t t = (t0 * P) % total;
    const int64_t e = t / per, r = t % per;
    const int64_t k0 = load_uniform(a.k_offsets + e), k1 = load_uniform(a.k_offsets + e + 1);
    DenseTile one;
    one.t.A = OpView{a.A.codes + k0 * (M / 2), a.A.scales + (k0 / 16) * M, M, a.A.block};
    one.t.B = OpView{a.B.codes + k0 * (N / 2), a.B.scales + (k0 / 16) * N, N, a.B.block};
    one.t.m0 = (r % mt) * C::BM;
    one.t.m_lim = M;
    one.t.n0 = (r / mt) * C::BN;
    one.t.gscale = gscale;
    one.t.C = a.C + e * M * N;
    gemm_tiles<C, false, false>(one, N, k1 - k0, false, a.c_acc, N, lds);
    __syncthreads();  // the next tile reuses the LDS buffers
  }
}

// ---- small M (decode-like shapes): NT with M <= 64 per row block ----------------------------------
// With a few rows of activations the weight codes dominate the traffic and a
// 256-row tile would leave most of the chip idle (N / 256 workgroups).  A
// workgroup here takes 32 columns of C (all M <= 64 rows of A) with NWV
// waves; wave w takes the w-th share of the K range in chunks of 256 k.  A
// chunk is loaded with whole 128-byte row segments per group of 8 lanes (B:
// 32 rows of W; A: the 8 * NA8 rows of A rounded up from M), so each load
// instruction touches 8 cache lines, with NB chunks in flight in registers;
// the wave then writes the chunk into its own LDS slot and reads back the
// fragments of the tiled kernel -- lane l: row l%32 and, per 64-k group, the
// 32 k at 32 * (l/32) with their two scale bytes -- decodes them the same
// way and multiplies with the same MFMA, into two accumulator sets (even and
// odd 16-k steps) so that consecutive MFMAs do not wait on each other.
// Partial sums are added in a fixed order (odd set onto even, then waves in
// order through LDS), so results are deterministic; they round like 2 * NWV
// partial sums, not like the tiled kernel's one sequential sum, within the
// same error bound.
//
// Slot layout (bytes): B codes [32 rows][128], B scales [32 rows][16],
// A scales [64 rows][16] (only the first 8 * NA8 rows are read), then A
// codes [8 * NA8 rows][128] or, for M <= 16, A decoded to fp16 (below).  In
// a code row, 16-byte unit u (k = 32u .. 32u+31 of the chunk) sits at
// position u ^ ((row >> 1) & 7): the 16 lanes of one 16-byte LDS access (16
// consecutive rows and one unit on reads, 2 rows and 8 units on writes) fall
// in 16 distinct slots of a 256-byte bank window.
constexpr int kSkChunkK = 256;          // k per chunk (4 groups of 64)
constexpr int kSkOob = INT32_MIN;       // buffer offset past every range: loads return 0

__device__ __forceinline__ int sk_swz(int row) { return (row >> 1) & 7; }

template <int NA8>
struct SkLayout {
  // A16: with at most 16 rows, A is decoded once per chunk into an fp16
  // image [8 * NA8 rows][256 k] (8-k unit U of row r at U ^ (r & 15)), so
  // its decode scales with M instead of the 32 fragment rows.
  static constexpr bool A16 = NA8 <= 2;
  static constexpr int kBC = 0, kBS = 4096, kAS = 4608, kAC = kAS + 64 * 16;
  static constexpr int kSlot = kAC + NA8 * (A16 ? 4096 : 1024);
  static constexpr int MT = NA8 > 4 ? 2 : 1;
};

template <int NA8>
struct SkChunk {
  uint4 bc[4];  // B codes: rows 8i + l/8, unit l%8
  uint2 bs;     // B scales: row l/2, bytes 8 (l%2) .. +8
  uint4 ac[NA8];
  uint4 as;     // A scales: row l (lanes from 8 NA8 on are never read)
};

// Per-lane sources of one wave's chunks (offsets from the buffer bases).
// Rows past an operand's edge re-read its last valid row (in bounds); they
// only reach outputs that are not stored.  Past the end of a row, a chunk's
// loads read the next row or, past the operand, zeros; those k are never
// multiplied.
template <int NA8>
struct SkSrc {
  __amdgpu_buffer_rsrc_t bcr, bsr, acr, asr;
  uint32_t boff[4], bsoff, aoff[NA8], asoff;

  __device__ __forceinline__ void load(SkChunk<NA8>& d, int64_t c, bool valid) const {
    const int cb = valid ? (int)(c * (kSkChunkK / 2)) : kSkOob;
    const int sb = valid ? (int)(c * (kSkChunkK / 16)) : kSkOob;
#pragma unroll
    for (int i = 0; i < 4; i++)
      d.bc[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bcr, boff[i], cb, 0));
    d.bs = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(bsr, bsoff, sb, 0));
#pragma unroll
    for (int i = 0; i < NA8; i++)
      d.ac[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(acr, aoff[i], cb, 0));
    d.as = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(asr, asoff, sb, 0));
  }
};

template <int NA8>
__device__ __forceinline__ void sk_put(uint8_t* lds, const SkChunk<NA8>& d, int lane) {
  using L = SkLayout<NA8>;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int row = 8 * i + lane / 8;
    *reinterpret_cast<uint4*>(lds + L::kBC + 128 * row + 16 * ((lane % 8) ^ sk_swz(row))) = d.bc[i];
  }
  *reinterpret_cast<uint2*>(lds + L::kBS + 8 * lane) = d.bs;
  *reinterpret_cast<uint4*>(lds + L::kAS + 16 * lane) = d.as;
  if constexpr (L::A16) {
    // Lane l holds unit l%8 (k = 32 (l%8) .. +32) of A row 8i + l/8: decode
    // it with that row's two scale bytes (just written above) into the image.
#pragma unroll
    for (int i = 0; i < NA8; i++) {
      const int row = 8 * i + lane / 8, u = lane % 8;
      const half2 sc = scale_pair(*reinterpret_cast<const uint16_t*>(lds + L::kAS + 16 * row + 2 * u));
#pragma unroll
      for (int j = 0; j < 4; j++)
        *reinterpret_cast<half8*>(lds + L::kAC + 512 * row + 16 * ((4 * u + j) ^ (row & 15))) =
            decode8(pick(d.ac[i], j), splat(sc, j >= 2));
    }
  } else {
#pragma unroll
    for (int i = 0; i < NA8; i++) {
      const int row = 8 * i + lane / 8;
      *reinterpret_cast<uint4*>(lds + L::kAC + 128 * row + 16 * ((lane % 8) ^ sk_swz(row))) = d.ac[i];
    }
  }
}

template <int NA8, int NWV, int NB>
__global__ __launch_bounds__(NWV * 64) void gemm_skinny_kernel(GemmArgs a) {
  using L = SkLayout<NA8>;
  constexpr int MT = L::MT, SLOT = L::kSlot;
  static_assert(NB >= 1 && NB <= 4, "chunks in flight");
  static_assert(SLOT >= MT * 4096, "the reduction reuses the slots");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NWV * SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  // Row block blockIdx.y: rows m0 .. m0 + 63 of A and C (all row blocks of
  // a column tile read the same weight columns, which the caches share).
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int64_t M = a.M - m0 < 64 ? a.M - m0 : 64, N = a.N, K = a.K, kc = K / 2, ks = K / 16;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t G = K / 64, CN = (K + kSkChunkK - 1) / kSkChunkK;
  const int64_t c0 = wave * CN / NWV, c1 = (wave + 1) * CN / NWV;
  uint8_t* const slot = lds + wave * SLOT;

  const bool b2d = a.B.block == kBlock2d, a2d = a.A.block == kBlock2d;
  const int64_t nlim = N - n0 < 32 ? N - n0 : 32;
  SkSrc<NA8> src;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = 8 * i + lane / 8;
    src.boff[i] = (uint32_t)((row < nlim ? row : nlim - 1) * kc + 16 * (lane % 8));
  }
  const int64_t bsbase = b2d ? (n0 / 16) * ks : n0 * ks;
  {
    const int64_t row = lane / 2;
    const int64_t r = n0 + (row < nlim ? row : nlim - 1);
    src.bsoff = (uint32_t)((b2d ? (r / 16) * ks : r * ks) - bsbase + 8 * (lane % 2));
  }
#pragma unroll
  for (int i = 0; i < NA8; i++) {
    const int64_t row = 8 * i + lane / 8;
    src.aoff[i] = (uint32_t)((row < M ? row : M - 1) * kc + 16 * (lane % 8));
  }
  {
    const int64_t r = lane < M ? lane : M - 1;
    src.asoff = lane < 8 * NA8 ? (uint32_t)(a2d ? (r / 16) * ks : r * ks) : (uint32_t)kSkOob;
  }
  const int64_t b_end = b2d ? ((n0 + nlim + 15) / 16) * ks : (n0 + nlim) * ks;
  src.bcr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.B.codes + n0 * kc), 0,
                                              (int)(nlim * kc), kBufferFlags);
  src.bsr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.B.scales + bsbase), 0,
                                              (int)(b_end - bsbase), kBufferFlags);
  src.acr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.A.codes + m0 * kc), 0,
                                              (int)(M * kc), kBufferFlags);
  src.asr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.A.scales + (a2d ? m0 / 16 : m0) * ks), 0,
      (int)(a2d ? ((M + 15) / 16) * ks : M * ks),
      kBufferFlags);

  // LDS rows this lane reads: B row lrow, A row min(32 s + lrow, M - 1).
  int arow[MT];
#pragma unroll
  for (int s = 0; s < MT; s++) arow[s] = 32 * s + lrow < M ? 32 * s + lrow : (int)M - 1;

  f32x16 acc[2][MT];
#pragma unroll
  for (int p = 0; p < 2; p++)
#pragma unroll
    for (int s = 0; s < MT; s++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[p][s][r] = 0.0f;

  // One chunk from the wave's slot.  All of the chunk's fragments are read
  // up front, so the LDS latency is paid once per chunk rather than once per
  // group.
  auto compute = [&](int64_t c) {
    const uint4 bsv = *reinterpret_cast<const uint4*>(slot + L::kBS + 16 * lrow);
    uint4 bq[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
      bq[u] = *reinterpret_cast<const uint4*>(slot + L::kBC + 128 * lrow +
                                              16 * ((2 * u + lhalf) ^ sk_swz(lrow)));
    // A group past K (the last chunk of a K that is not a multiple of 256)
    // is multiplied with zero scales: its finite codes then add exact zeros.
    const int64_t gleft = G - 4 * c;
    if constexpr (L::A16) {
      // 8-k unit 8u + 4h + st of A row arow: the k of B's dword st.
      const int ra = arow[0];
      half8 af[4][4];
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int st = 0; st < 4; st++)
          af[u][st] = *reinterpret_cast<const half8*>(
              slot + L::kAC + 512 * ra + 16 * ((8 * u + 4 * lhalf + st) ^ (ra & 15)));
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint32_t live = u < gleft ? 0xFFFFFFFFu : 0u;
        const half2 bsc = scale_pair((pick(bsv, u) & live) >> (16 * lhalf));
#pragma unroll
        for (int st = 0; st < 4; st++)
          acc[st & 1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              af[u][st], decode8(pick(bq[u], st), splat(bsc, st >= 2)), acc[st & 1][0], 0, 0, 0);
      }
    } else {
      uint4 asv[MT], aq[4][MT];
#pragma unroll
      for (int s = 0; s < MT; s++)
        asv[s] = *reinterpret_cast<const uint4*>(slot + L::kAS + 16 * arow[s]);
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int s = 0; s < MT; s++)
          aq[u][s] = *reinterpret_cast<const uint4*>(slot + L::kAC + 128 * arow[s] +
                                                     16 * ((2 * u + lhalf) ^ sk_swz(arow[s])));
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint32_t live = u < gleft ? 0xFFFFFFFFu : 0u;
        const half2 bsc = scale_pair((pick(bsv, u) & live) >> (16 * lhalf));
        half2 asc[MT];
#pragma unroll
        for (int s = 0; s < MT; s++) asc[s] = scale_pair(pick(asv[s], u) >> (16 * lhalf));
#pragma unroll
        for (int st = 0; st < 4; st++) {
          const half8 bf = decode8(pick(bq[u], st), splat(bsc, st >= 2));
#pragma unroll
          for (int s = 0; s < MT; s++)
            acc[st & 1][s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                decode8(pick(aq[u][s], st), splat(asc[s], st >= 2)), bf, acc[st & 1][s], 0, 0, 0);
        }
      }
    }
  };

  // Chunk c + j sits in buf[j % NB].  Every step issues its refill (out of
  // range, so without traffic, past the wave's share) and the scheduling
  // fences keep each chunk's loads together and in order: all paths then
  // carry the same load sequence, and the wait before a chunk's LDS write
  // leaves the NB - 1 later chunks in flight.
  SkChunk<NA8> buf[NB];
#pragma unroll
  for (int j = 0; j < NB; j++) {
    src.load(buf[j], c0 + j, c0 + j < c1);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t c = c0; c < c1; c += NB) {
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const bool live = c + j < c1;  // wave-uniform
      if (live) sk_put<NA8>(slot, buf[j], lane);
      __builtin_amdgcn_sched_barrier(0);
      src.load(buf[j], c + j + NB, c + j + NB < c1);
      __builtin_amdgcn_sched_barrier(0);
      if (live) compute(c + j);
    }
  }

  // Reduction through the (now idle) slots.
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [NWV][MT][16][64]
#pragma unroll
  for (int s = 0; s < MT; s++)
#pragma unroll
    for (int r = 0; r < 16; r++)
      red[((wave * MT + s) * 16 + r) * 64 + lane] = acc[0][s][r] + acc[1][s][r];
  __syncthreads();
  // Wave w adds and stores accumulator entries r with r % NWV == w (per sub-tile).
  const float gscale = *a.A.gdec * *a.B.gdec;
  const int64_t col = n0 + lrow;
#pragma unroll
  for (int s = 0; s < MT; s++) {
    for (int r = wave; r < 16; r += NWV) {
      float v = red[(s * 16 + r) * 64 + lane];
      for (int w = 1; w < NWV; w++) v = v + red[((w * MT + s) * 16 + r) * 64 + lane];
      const int64_t row = 32 * s + 8 * (r >> 2) + 4 * lhalf + (r & 3);
      if (row < M && col < N) {
        const float o = v * gscale;
        if (a.c_bf16) {
          const __bf16 b = (__bf16)o;
          static_cast<uint16_t*>(a.C)[(m0 + row) * N + col] = __builtin_bit_cast(uint16_t, b);
        } else {
          float* c = static_cast<float*>(a.C) + (m0 + row) * N + col;
          *c = a.c_acc ? *c + o : o;
        }
      }
    }
  }
}

template <int NA8, int NWV, int NB>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  const int64_t grid = (a.N + 31) / 32;
  const dim3 g3((unsigned)grid, (unsigned)((a.M + 63) / 64));  // column tiles x 64-row blocks
  gemm_skinny_kernel<NA8, NWV, NB><<<g3, NWV * 64, 0, st>>>(a);
  return hipGetLastError();
}

// Rows beyond 64 run as row blocks of 64 (blockIdx.y).
hipError_t launch_small_m(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 8) return launch_skinny<1, 8, 2>(a, st);
  if (a.M <= 16) return launch_skinny<2, 8, 2>(a, st);
  if (a.M <= 32) return launch_skinny<4, 8, 2>(a, st);
  return launch_skinny<8, 8, 2>(a, st);
}

template <class C, bool AK, bool BKM>
hipError_t launch_dense(const GemmArgs& a, hipStream_t st) {
  const int64_t ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
  gemm_kernel<C, AK, BKM><<<(unsigned)(ntm * ntn), C::NT, 0, st>>>(a);
  return hipGetLastError();
}

// Compute units of the current device (one workgroup of these tiles runs
// per CU).
hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && *cus <= 0) *cus = 256;
  return e;
}

template <class C>
hipError_t launch_layout(const GemmArgs& a, hipStream_t st) {
  if (a.a_kmajor && a.b_kmajor) return launch_dense<C, true, true>(a, st);
  if (a.a_kmajor && !a.b_kmajor) return launch_dense<C, true, false>(a, st);
  return launch_dense<C, false, false>(a, st);
}

template <int BK>
hipError_t launch_depth(const GemmArgs& a, int cus, hipStream_t st) {
  auto cost = [&](int64_t bm, int64_t bn) {
    const int64_t tiles = ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    return ((tiles + cus - 1) / cus) * bm * bn;
  };
  const int64_t c256 = cost(256, 256), c192 = cost(192, 256);
  if (a.a_kmajor && cost(128, 256) * 5 < (c192 < c256 ? c192 : c256) * 4) {
    if (a.b_kmajor) return launch_dense<Cfg<128, 256, 1, 8, BK>, true, true>(a, st);
    return launch_dense<Cfg<128, 256, 1, 8, BK>, true, false>(a, st);
  }
  if (c192 < c256) return launch_layout<Cfg<192, 256, 1, 8, BK, BK>>(a, st);
  return launch_layout<Cfg<256, 256, 2, 4, BK>>(a, st);
}

template <class C>
hipError_t launch_grouped(const GroupedArgs& a, int cus, hipStream_t st) {
  if (a.groups > kMaxGroups) return hipErrorInvalidValue;
  const int64_t ntn = (a.N + C::BN - 1) / C::BN;
  const int64_t max_tiles = ((a.total_rows + C::BM - 1) / C::BM + a.groups) * ntn;
  int64_t grid = cus;
  if (grid > max_tiles) grid = max_tiles;
  if (a.b_kmajor)
    grouped_gemm_kernel<C, true><<<(unsigned)grid, C::NT, 0, st>>>(a);
  else
    grouped_gemm_kernel<C, false><<<(unsigned)grid, C::NT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

// Stage depth: 128 k when K allows (longer row segments per transfer and
// half the barriers), else 64.  The 192-row tile also takes its phases at
// the stage depth: with 128 k its two raw stages (32 KB each) and two fp16
// A images (48 KB each) fill the 160 KB of LDS exactly, and a barrier then
// comes every 48 MFMAs of a wave instead of 24 (6144 x 6144 x 8192: TN
// 0.531 -> 0.513 ms, NN 0.518 -> 0.503 ms, NT unchanged).  The 256-row
// tile's 128-k images would not fit beside its stages.  Its eight waves sit
// side by side (192 x 32 each: 6 MFMAs and one B decode per step, where
// 2 x 4 waves of 96 x 64 decoded each B fragment twice, two per 6 MFMAs):
// TN 0.529 -> 0.497 ms, NN 0.509 -> 0.492 ms, NT unchanged.  Tile: the 256- and 192-row shapes run at
// about the same rate per output, so take the one whose last round of
// workgroups leaves the fewest CUs idle (cost = rounds of tiles times tile
// area).  With A K-major (NT, NN) a 128-row tile also competes, at a 5/4
// cost for its lower rate per output: it wins where bigger tiles leave CUs
// idle (N = K = 6144: 81 us instead of 108 us at M = 640 .. 1024) and ties
// from M = 1536 on.  Every output is the same sum in the same order whatever
// the choice.
//
// NT with few rows takes the small-M kernel: always up to 64 rows, and up to
// 512 when 256 x 256 tiles would leave CUs without a tile (at N = K = 6144:
// 27 us instead of 105 us at M = 128, 74 us instead of 106 us at M = 512; the
// two meet near M = 768).
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const bool nt = a.a_kmajor && a.b_kmajor;
  if (nt && a.M <= 64) return launch_small_m(a, st);
  int cus = 256;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  if (nt && a.M <= 512 && ((a.M + 255) / 256) * ((a.N + 255) / 256) < cus)
    return launch_small_m(a, st);
  if (a.K % 128 == 0) return launch_depth<128>(a, cus, st);
  return launch_depth<64>(a, cus, st);
}

// Grouped tiles: routed experts get few rows each (padding a 256-row tile
// wastes most of it), so when the average group has fewer than 512 rows the
// tiles are 128 rows x 256 columns, one 128 x 32 slice per wave (eight waves
// side by side: each B fragment is decoded by one wave, A comes decoded
// from LDS); otherwise 256 x 256.
hipError_t launch_grouped_gemm(const GroupedArgs& a, hipStream_t st) {
  if (a.total_rows == 0 || a.N == 0 || a.groups == 0) return hipSuccess;
  int cus = 256;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const bool small = a.total_rows < 512 * a.groups;
  if (a.K % 128 == 0)
    return small ? launch_grouped<Cfg<128, 256, 1, 8, 128, 128>>(a, cus, st)
                 : launch_grouped<Cfg<256, 256, 2, 4, 128>>(a, cus, st);
  return small ? launch_grouped<Cfg<128, 256, 1, 8, 64>>(a, cus, st)
               : launch_grouped<Cfg<256, 256, 2, 4, 64>>(a, cus, st);
}

// Grouped wgrad: 256 x 256 tiles, stages of 64 k (the groups' token counts
// are ragged, and a partial last stage is work on zeros: the shallow stage
// keeps that small).
hipError_t launch_grouped_wgrad(const WgradArgs& a, hipStream_t st) {
  if (a.groups == 0 || a.M == 0 || a.N == 0) return hipSuccess;
  int cus = 256;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  using C = Cfg<256, 256, 2, 4, 64>;
  const int64_t tiles = a.groups * ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
  const int64_t grid = tiles < cus ? tiles : cus;
  grouped_wgrad_kernel<C><<<(unsigned)grid, C::NT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
