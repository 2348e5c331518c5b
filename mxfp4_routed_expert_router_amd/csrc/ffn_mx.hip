// MX mode of the grouped SwiGLU expert FFN (prefill).  The FP4 weights are used as they are stored
// (E2M1 codes with one E8M0 scale per 32 values along K, "DeepSeek-V4-Flash on a four-GPU Ampere
// workstation", section "MXFP4 is not NVFP4") and the activations -- x, then h -- are quantised on
// the fly to an MX element format with their own E8M0 scale per 32 values along K.  Gate/up and
// down then run as scaled MFMAs, v_mfma_scale_f32_16x16x128_f8f6f4, which multiply FP4 weights by
// FP8/FP6/FP4 activations and apply both block scales in the matrix core.
//
// The activation formats are the OCP Microscaling element formats E4M3, E2M3 and E2M1 with the
// scale rule X = 2^(floor(log2 amax) - emax) (emax = 8, 2, 2) and round-to-nearest-even,
// saturating element encoding.  They are not on the pages; this mode trades accuracy against the
// exact path for matrix-core rate and is checked against a quantisation-aware oracle.
//
// Packed codes: a 32-value block takes 4 * bits bytes; FP4 element j in nibble j of the block's
// little-endian 128-bit string, FP6 element j in bits 6j..6j+5 of its 192-bit string, FP8 one
// byte per element.  The MFMA operand layout is stated next to mx_tile.
//
// Work split.  A workgroup (8 waves, two per SIMD) takes one 128-token tile of an expert (the tile
// table of the exact path, built with 128 rows per tile) and 8 * 32 rows of I (gate/up: 32 rows
// of each matrix per wave) or 8 * 64 rows of H (down).  Each wave loads its FP4 weight rows as
// whole 128-byte lines two steps ahead, stages them in registers, and transposes them through a
// private LDS copy into MFMA layout; the tile's activation codes and scales go through a
// two-stage LDS ring shared by the eight waves, with one barrier per step.  Workgroups are
// numbered tile-major with the row blocks padded to a multiple of 8, so row block j of every tile
// runs on XCD j % 8 and the tiles of a hot expert read each weight row from one L2.  Only the
// 16-token column tiles that hold rows of the tile (rounded up to 32 tokens) are computed.
//
// The gate/up epilogue forms h = SiLU(g) * u in fp32; each lane holds 8 consecutive values of h
// for its token (a quarter of a K-block) and writes their codes, one lane per token the block's
// E8M0 scale -- the layout the down phase reads.  The down epilogue writes fp32 y_slots through
// the wave's private LDS copy, whole token rows per store.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// Element formats: code bits, MFMA operand format code, exponent/fraction bits, bias, exponent of
// the largest normal, largest code and value.
template <int F>
struct Mx;
template <>
struct Mx<MOE_MX_FP8_E4M3> {
  static constexpr int kBits = 8, kMfma = 0, kMBits = 3, kBias = 7, kEmax = 8;
  static constexpr uint32_t kMaxCode = 0x7E;  // 448 (0x7F is NaN)
  static constexpr float kMax = 448.0f;
};
template <>
struct Mx<MOE_MX_FP4_E2M1> {
  static constexpr int kBits = 4, kMfma = 4, kMBits = 1, kBias = 1, kEmax = 2;
  static constexpr uint32_t kMaxCode = 0x7;  // 6
  static constexpr float kMax = 6.0f;
};
template <>
struct Mx<MOE_MX_FP6_E2M3> {
  static constexpr int kBits = 6, kMfma = 2, kMBits = 3, kBias = 1, kEmax = 2;
  static constexpr uint32_t kMaxCode = 0x1F;  // 7.5
  static constexpr float kMax = 7.5f;
};
constexpr int kWFmtFp4 = 4;  // MFMA operand format code of the E2M1 weights

// E8M0 code of a block whose largest magnitude is amax (finite, >= 0):
// floor(log2 amax) - emax + 127 clamped to [0, 254]; 0 for an all-zero block.  floor(log2) comes
// from the binary32 exponent field, or from the leading fraction bit for a subnormal amax.
template <int F>
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0) return 0;
  const uint32_t ef = u >> 23;
  const int e = ef ? (int)ef - 127 : (31 - (int)__builtin_clz(u)) - 149;
  const int c = e - Mx<F>::kEmax + 127;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}
// 2^(127 - c), the reciprocal of the block scale, as a binary32 value (exact).
__device__ __forceinline__ float mx_inv_scale(uint32_t c) {
  return __uint_as_float(c <= 253 ? (254u - c) << 23 : 0x00400000u);
}

// Nearest element code to q (ties to the even code), saturating at the largest value, with q's
// sign.  Subnormal range: q / 2^(1 - bias - m_bits) rounded to an integer (which reaches the
// smallest normal code exactly when it rounds up to 2^m_bits).  Normal range: the fraction of q
// rounded to m_bits; a carry out of the fraction lands on the next exponent's code.
template <int F>
__device__ __forceinline__ uint32_t mx_encode(float q) {
  typedef Mx<F> M;
  const uint32_t u = __float_as_uint(q);
  const float a = fabsf(q);
  uint32_t c;
  if (a >= M::kMax) {
    c = M::kMaxCode;
  } else if (a < __uint_as_float((uint32_t)(127 + 1 - M::kBias) << 23)) {
    c = (uint32_t)__builtin_rintf(a * __uint_as_float((uint32_t)(127 + M::kBias - 1 + M::kMBits) << 23));
  } else {
    const int e = (int)((u >> 23) & 0xFF) - 127;
    const float r = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u);
    const uint32_t m = (uint32_t)__builtin_rintf((r - 1.0f) * (float)(1 << M::kMBits));
    c = ((uint32_t)(e + M::kBias) << M::kMBits) + m;
  }
  return c | ((u >> 31) << (M::kBits - 1));
}

// Codes of 2 * NP values q (already divided by the block scale), packed as in the block layout,
// with the hardware conversions at scale 1: over every code's value, every midpoint between
// neighbouring codes and the floats next to them, signed zeros and a million log-spread values,
// they give the codes of mx_encode exactly -- FP6 and FP4 everywhere, FP8 once the input is
// clamped to the largest value (past it the conversion returns the NaN code).  The FP6
// conversion takes 32 values as two halves and interleaves them (field 2i from the first half,
// 2i + 1 from the second), so the halves are the even and the odd values.
typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
template <int F, int NP>
__device__ __forceinline__ void mx_hw_pack(const float* q, uint32_t* dw) {
  static_assert(NP == 4 || NP == 16, "a quarter block or a whole block");
  static_assert(NP == 16 || Mx<F>::kBits != 6, "FP6 quarters take the software encoder");
  if constexpr (Mx<F>::kBits == 4) {
#pragma unroll
    for (int w = 0; w < NP / 4; ++w) {
      const float* p = q + 8 * w;  // byte i of the dword from values 2i, 2i + 1
      uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[0], p[1], 1.0f, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[2], p[3], 1.0f, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[4], p[5], 1.0f, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[6], p[7], 1.0f, 3);
      dw[w] = d;
    }
  } else if constexpr (Mx<F>::kBits == 8) {
    auto cl = [](float x) { return fminf(fmaxf(x, -Mx<F>::kMax), Mx<F>::kMax); };
#pragma unroll
    for (int w = 0; w < NP / 2; ++w) {
      v2s d = {0, 0};
      d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, cl(q[4 * w]), cl(q[4 * w + 1]), 1.0f, false);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, cl(q[4 * w + 2]), cl(q[4 * w + 3]), 1.0f, true);
      dw[w] = __builtin_bit_cast(uint32_t, d);
    }
  } else {
    v16f a = {}, b = {};
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      a[i] = q[2 * i];
      b[i] = q[2 * i + 1];
    }
    const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
#pragma unroll
    for (int w = 0; w < (NP == 16 ? 6 : 2); ++w) dw[w] = (uint32_t)r[w];
    if constexpr (NP == 4) dw[1] &= 0xFFFFu;  // fields 8 .. 31 are codes of zero anyway
  }
}

// One 32-value block: E8M0 code and the packed element codes (4 * bits bytes in dw[0 .. bits/2)).
template <int F>
__device__ __forceinline__ uint32_t mx_pack_block(const float (&v)[32], uint32_t (&dw)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t sc = mx_scale_code<F>(amax);
  const float inv = mx_inv_scale(sc);
  float q[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) q[j] = v[j] * inv;
#pragma unroll
  for (int i = 0; i < 8; ++i) dw[i] = 0;
  mx_hw_pack<F, 16>(q, dw);
  return sc;
}

// Stores the 4 * bits bytes of a packed block (dst aligned to 8 bytes, and to 16 for FP8/FP4).
template <int F>
__device__ __forceinline__ void mx_store_block(uint8_t* dst, const uint32_t (&dw)[8]) {
  if constexpr (Mx<F>::kBits == 6) {
#pragma unroll
    for (int i = 0; i < 3; ++i) *reinterpret_cast<u32x2*>(dst + 8 * i) = u32x2{dw[2 * i], dw[2 * i + 1]};
  } else {
#pragma unroll
    for (int i = 0; i < Mx<F>::kBits / 4; ++i) st16(dst + 16 * i, u32x4{dw[4 * i], dw[4 * i + 1], dw[4 * i + 2], dw[4 * i + 3]});
  }
}

// ---- activation quantisation: one thread per 32-value block of a contiguous [rows][K] matrix ----
template <int F, bool XF16>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t n_blocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 p = ld16(x + b * 32 + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = p[j];
      if constexpr (XF16) {
        const f16x2 h = bitcast<f16x2>(w);
        v[8 * i + 2 * j] = (float)h[0];
        v[8 * i + 2 * j + 1] = (float)h[1];
      } else {
        v[8 * i + 2 * j] = __uint_as_float(w << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
  }
  uint32_t dw[8];
  const uint32_t sc = mx_pack_block<F>(v, dw);
  mx_store_block<F>(codes + b * (4 * Mx<F>::kBits), dw);
  scales[b] = (uint8_t)sc;
}

// ---- the scaled-MFMA FFN kernels ----
constexpr int kMxNW = 8;       // waves per workgroup (two per SIMD)
constexpr int kMxTok = 128;    // sorted rows (tokens) per tile
constexpr int kMxStepK = 256;  // K per step: 8 blocks of 32 (two MFMA K positions of 128)

// Weight rows of a wave: 32 rows of I of each of gate and up (gate/up), or 64 rows of H (down), as
// four 16-row MFMA tiles: two of gate then two of up, or four of down.
template <bool GU>
struct WRows {
  static constexpr int kPerMatrix = GU ? 32 : 64;  // rows per wave of each matrix
  static constexpr int kTiles = kPerMatrix / 16;   // MFMA tiles per matrix
};
constexpr int kMxRows = 64;  // weight rows per wave (both phases)

template <int F>
struct MxTile {
  static constexpr int kBB = 4 * Mx<F>::kBits;             // bytes per 32-value block
  static constexpr int kRowStep = 8 * kBB;                 // code bytes of one token per step
  // LDS row stride.  FP6 fragments are read as 8-byte pieces, 16 lanes (16 consecutive rows) at a
  // time: a 200-byte stride (50 dwords, 18 mod 32 banks) puts the 16 rows on 16 distinct bank
  // pairs.  FP8 and FP4 fragments are read as 16-byte pieces, 8 lanes at a time: 16 bytes of
  // padding (a stride of 4 mod 32 banks) spreads 8 rows over all 32 banks.
  static constexpr int kRS = kRowStep + (Mx<F>::kBits == 6 ? 8 : 16);
  static constexpr int kCodes = kMxTok * kRS;              // code bytes of a stage
  static constexpr int kScales = kCodes;                   // 8 scale bytes per token
  static constexpr int kStage = kScales + kMxTok * 8;      // one stage of the shared activation ring
  // After the two stages: per wave, a private copy of its 64 weight rows for one step (128 bytes
  // per row, 16-byte pieces XOR-swizzled by row) and their scale bytes of two steps (16 per row).
  static constexpr int kPrivA = 2 * kStage;
  static constexpr int kPrivS = kPrivA + kMxNW * kMxRows * 128;
  static constexpr int kLds = kPrivS + kMxNW * kMxRows * 16;
  static constexpr int kPieces = kRowStep / 16;            // 16-byte pieces per token per step
  static constexpr int kLPT = kMxTok * kPieces / (64 * kMxNW);  // fill loads per thread per step
  static_assert(kLPT * 64 * kMxNW == kMxTok * kPieces, "a step of codes over the workgroup");
};

// Codes of 8 consecutive values (a quarter block) packed as in the block layout: bits bytes, in
// dw[0] and (FP6, FP8) dw[1].
template <int F>
// (FP6 quarters take the software encoder: the 32-value FP6 conversion's two 16-register halves
// made the gate/up kernel spill inside its main loop, 3.75 -> 3.79 ms; FP4 with the hardware
// conversion 3.58 -> 3.49 ms.)
__device__ __forceinline__ void mx_pack_quarter(const float (&v)[8], float inv, uint32_t (&dw)[2]) {
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = v[j] * inv;
  dw[0] = 0;
  dw[1] = 0;
  if constexpr (Mx<F>::kBits == 6) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = mx_encode<F>(q[j]);
      const int bit = 6 * j, w = bit >> 5, o = bit & 31;
      dw[w] |= c << o;
      if (o + 6 > 32) dw[w + 1] |= c >> (32 - o);
    }
  } else {
    mx_hw_pack<F, 4>(q, dw);
  }
}

// MFMA layout (v_mfma_scale_f32_16x16x128_f8f6f4, lane l, row/column l%16, quarter q = l/16):
//   FP4/FP6 operand: K-block q of the 128-wide position (32 contiguous values);
//   FP8 operand: values 16(q%2)..+15 of K-blocks q/2 and 2 + q/2;
//   E8M0 scale of a lane: K-block q of its row or column;
//   D: lane l holds column l%16, rows 4q + i in accumulator i.
// A 256-wide step holds positions p = 0, 1 over its K-blocks 4p .. 4p+3 in memory order.
//
// Weight rows are assigned to tile rows so that a lane quarter's accumulators cover consecutive
// rows: row 4q + i of the wave's tile t of a matrix is the matrix row n0 + (R/4) q + 4t + i (R =
// the wave's rows of that matrix).  Lane quarter q then holds rows n0 + (R/4) q .. + R/4 - 1 of
// its column (token): a quarter of h's 32-value block in the gate/up epilogue, 64 contiguous
// bytes of y in the down epilogue.
template <int F, bool GU, int NB>
__device__ __forceinline__ void mx_tile(const TileInfo ti, int nblk, const uint8_t* __restrict__ act,
                                        const uint8_t* __restrict__ act_s, int n_act_rows, int k_total, int K,
                                        int N, const ProjDev& w0, const ProjDev& w1,
                                        const int32_t* __restrict__ sorted_slot, int n_slots,
                                        uint8_t* __restrict__ h_codes, uint8_t* __restrict__ h_scales,
                                        float* __restrict__ y_slots) {
  typedef MxTile<F> P;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, q = lane >> 4;
  constexpr int R = WRows<GU>::kPerMatrix, TM = WRows<GU>::kTiles, TA = 4;
  const int n0 = (nblk * kMxNW + wave) * R;
  const bool active = n0 < N;  // N % R == 0, so a wave's rows are all in or all out
  const int e = ti.e;
  const int n_steps = K / kMxStepK;
  const int RB = (K / 32) * P::kBB, KB = K / 32;

  // ---- LDS fill addressing: piece i of a thread -> token (threadIdx.x + 512 i) / kPieces
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(act, (int64_t)n_act_rows * RB);
  const __amdgpu_buffer_rsrc_t asr = make_rsrc(act_s, (int64_t)n_act_rows * KB);
  auto act_row = [&](int tok) -> int {
    if (tok >= ti.nr) return -1;
    if constexpr (GU) {
      const int sl = sorted_slot[ti.r0 + tok];
      return (sl >= 0 && sl < n_slots) ? sl / k_total : -1;
    } else {
      return ti.r0 + tok;
    }
  };
  uint32_t aoff[P::kLPT];
#pragma unroll
  for (int i = 0; i < P::kLPT; ++i) {
    const int qq = threadIdx.x + 64 * kMxNW * i, tok = qq / P::kPieces, col = qq % P::kPieces;
    const int row = act_row(tok);
    aoff[i] = row >= 0 ? (uint32_t)row * (uint32_t)RB + 16u * col : kOutOfRange;
  }
  auto aw = [&](int i) -> uint32_t {  // LDS offset of fill piece i (recomputed, no register held)
    const int qq = threadIdx.x + 64 * kMxNW * i, tok = qq / P::kPieces, col = qq % P::kPieces;
    return (uint32_t)(tok * P::kRS + 16 * col);
  };
  // The tile's 128 x 8 scale bytes of a step: one dword per thread of the first four waves.
  const bool sfill = threadIdx.x < 2 * kMxTok;
  uint32_t asoff, asw;
  {
    const int tok = (threadIdx.x >> 1) & (kMxTok - 1), half = threadIdx.x & 1;
    const int row = act_row(tok);
    asoff = row >= 0 ? (uint32_t)row * (uint32_t)KB + 4u * half : kOutOfRange;
    asw = (uint32_t)(P::kCodes + tok * 8 + 4 * half);
  }

  // ---- weights: wave row r (0..63) is row r of gate (r < 32) / up for gate/up, row n0 + r of
  //      down.  A step's 128 bytes of the wave's rows are loaded as whole 128-byte lines (8 lanes
  //      per row, 8 rows per instruction), written to the wave's private LDS copy with piece c of
  //      row r in slot c ^ (r & 7), and read back in MFMA layout (conflict-free both ways).  Loads
  //      run two steps ahead of the MFMAs: staged in registers one step, in LDS the next.
  const int64_t wrows = (int64_t)N - 1;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(w0.w + (int64_t)e * w0.we, wrows * w0.wr + K / 2);
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(w1.w + (int64_t)e * w1.we, wrows * w1.wr + K / 2);
  const __amdgpu_buffer_rsrc_t sr0 = make_rsrc(w0.s + (int64_t)e * w0.se, wrows * w0.sr + K / 32);
  const __amdgpu_buffer_rsrc_t sr1 = make_rsrc(w1.s + (int64_t)e * w1.se, wrows * w1.sr + K / 32);
  const int lr = lane >> 3, lc = lane & 7;  // line loads: row lr of 8, 16-byte piece lc
  const uint32_t lv0 = active ? (uint32_t)((n0 + lr) * w0.wr) + 16u * lc : kOutOfRange;
  const uint32_t lv1 = active ? (uint32_t)((n0 + lr) * w1.wr) + 16u * lc : kOutOfRange;
  // scale row of lane l: wave row l (gate/up: gate row l for l < 32, up row l - 32)
  const bool sup = GU && lane >= 32;
  const uint32_t sv = active ? (uint32_t)((n0 + (GU ? (lane & 31) : lane)) * (sup ? w1.sr : w0.sr)) : kOutOfRange;
  // Scales: with an even step count (and 16-byte aligned scale rows), the 16 scale bytes of steps
  // (s, s+1) of a row come in one load at even s and the load at odd s reads nothing (out of
  // range): half the scale requests.  Otherwise 8 bytes every step.  Either way one load per step, so the wait counts
  // do not depend on the step.
  const bool spair = (n_steps & 1) == 0 && ((w0.sr | w1.sr) & 15) == 0 &&
                     ((((uintptr_t)(w0.s + (int64_t)e * w0.se)) | ((uintptr_t)(w1.s + (int64_t)e * w1.se))) & 15) == 0;
  u32x4 ast[8];
  u32x4 sst;
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // rows 8i .. 8i+7 of the wave
      const bool second = GU && i >= 4;
      const uint32_t ii = (uint32_t)(second ? i - 4 : i);
      const uint32_t wrs = (uint32_t)(second ? w1.wr : w0.wr);
      ast[i] = bld16s(second ? wr1 : wr0, second ? lv1 : lv0, 8u * wrs * ii + (uint32_t)(s * 128));
    }
    const __amdgpu_buffer_rsrc_t srr = sup ? sr1 : sr0;
    if (spair) {
      sst = bld16(srr, (s & 1) ? kOutOfRange : sv + (uint32_t)(s * 8));
    } else {
      const u32x2 v = bld8(srr, sv + (uint32_t)(s * 8));
      sst = u32x4{v[0], v[1], 0u, 0u};
    }
  };
  uint8_t* const privA = lds + P::kPrivA + wave * (kMxRows * 128);
  uint8_t* const privS = lds + P::kPrivS + wave * (kMxRows * 16);
  // Private copy layout: piece c of wave row r in 16-byte slot c ^ sw(r), sw(r) = 2 ((r >> S) & 3)
  // + ((r >> 1) & 1), S = log2(R/4).  Writes: the 16 lanes of a bank pass hold 2 rows x 8 pieces,
  // conflict-free for any sw.  Reads (MFMA layout): the 16 lanes l16 of a bank pass read rows
  // (R/4)(l16 / 4) + l16 % 4 + c, for which (r & 1, sw(r)) takes 16 distinct values: no conflicts.
  constexpr int S = GU ? 3 : 4;
  const uint32_t wrow = (uint32_t)(lr * 128);                   // + 1024 per instruction
  const uint32_t wlc = (uint32_t)(lc ^ ((lr >> 1) & 1));         // ^ 2 ((row >> S) & 3)
  auto store_a = [&](int s) {  // s: the step the staged registers were loaded for
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t hi = (uint32_t)(((8 * i) >> S) & 3) << 1;  // rows 8i + lr: (r >> S) & 3
      *reinterpret_cast<u32x4*>(privA + 1024 * i + wrow + 16 * (wlc ^ hi)) = ast[i];
    }
    if (spair) {
      if ((s & 1) == 0) *reinterpret_cast<u32x4*>(privS + 16 * lane) = sst;
    } else {
      *reinterpret_cast<u32x2*>(privS + 16 * lane + 8 * (s & 1)) = u32x2{sst[0], sst[1]};
    }
  };
  // MFMA-layout reads: tile t (tile tt = t % TM of matrix m = t / TM for gate/up), lane row l16 ->
  // wave row r = 32 m + (R/4)(l16 / 4) + 4 tt + l16 % 4, piece 4p + q.  For these rows sw(r) =
  // g = 2 (l16 / 4) + ((l16 / 2) & 1) whatever m and tt, so the slot (4p + q) ^ g is
  // 4 (p ^ (g >> 2)) + ((q ^ g) & 3): every read is one of two per-lane bases plus a constant.
  const int rbase = (R / 4) * (l16 >> 2) + (l16 & 3);
  const int g = 2 * (l16 >> 2) + ((l16 >> 1) & 1);
  const uint8_t* const abase0 = privA + 128 * rbase + 16 * ((q ^ g) & 3) + 64 * (g >> 2);
  const uint8_t* const abase1 = privA + 128 * rbase + 16 * ((q ^ g) & 3) + 64 * ((g >> 2) ^ 1);
  const uint8_t* const sbase = privS + 16 * rbase;

  // A step's fill goes in two parts (pieces [0, H0), then [H0, kLPT) and the scales) through the
  // same staging registers, so the two parts' lifetimes (load to LDS store) must not overlap; the
  // pipeline below loads part 1 after storing part 0 and part 0 after storing part 1.
  constexpr int H0 = (P::kLPT + 1) / 2;
  u32x4 fill[H0];
  uint32_t fills;
  auto load_b = [&](int s, int part) {
#pragma unroll
    for (int i = part ? H0 : 0; i < (part ? P::kLPT : H0); ++i)
      fill[i - (part ? H0 : 0)] = bld16(ar, aoff[i] + (uint32_t)(s * P::kRowStep));
    if (part && sfill) fills = bld4(asr, asoff + (uint32_t)(s * 8));
  };
  auto store_b = [&](int stage, int part) {
    uint8_t* base = lds + stage * P::kStage;
#pragma unroll
    for (int i = part ? H0 : 0; i < (part ? P::kLPT : H0); ++i) {
      const u32x4 f = fill[i - (part ? H0 : 0)];
      if constexpr (Mx<F>::kBits == 6) {  // 8-byte aligned rows
        *reinterpret_cast<u32x2*>(base + aw(i)) = u32x2{f[0], f[1]};
        *reinterpret_cast<u32x2*>(base + aw(i) + 8) = u32x2{f[2], f[3]};
      } else {
        *reinterpret_cast<u32x4*>(base + aw(i)) = f;
      }
    }
    if (part && sfill) *reinterpret_cast<uint32_t*>(base + asw) = fills;
  };

  f32x4 acc[TA][NB];
#pragma unroll
  for (int t = 0; t < TA; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step of MFMAs over the stage's activations and the wave's private weight copy, position
  // by position.  After the last reads of the private copy, the next step's weights (staged in
  // registers) are written in their place and the loads of the step after that are started.
  auto step = [&](int stage, int s_cur, int s_next1, int s_next2) {
    const uint8_t* base = lds + stage * P::kStage;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // activation fill of step s+1 into the other stage: part p stored, then the next part loaded
      // (part 1 of step s+1 at p = 0, part 0 of step s+2 at p = 1)
      store_b(stage ^ 1, p);
      load_b(p ? s_next2 : s_next1, p ^ 1);
      // A wave past the last row (ragged N) reads and writes its private copy like the others
      // (its loads are out of range and return zeros) and skips only the MFMAs and the epilogue:
      // the same loads stay pending on every path, so the wait counts are exact.
      u32x4 af4[TA];
      uint32_t was[TA];
#pragma unroll
      for (int t = 0; t < TA; ++t) {
        const int m = GU ? (t / TM) : 0, tt = GU ? (t % TM) : t;
        af4[t] = *reinterpret_cast<const u32x4*>((p ? abase1 : abase0) + 128 * (32 * m + 4 * tt));
        was[t] = *reinterpret_cast<const uint32_t*>(sbase + 16 * (32 * m + 4 * tt) + 8 * (s_cur & 1) + 4 * p);
      }
      if (p == 1) {
        store_a(s_next1);  // LDS accesses of a wave stay in order: the reads above come first
        load_a(s_next2);
      }
      if (!active) continue;
      // B fragment (column tile b, position p) and its scale byte; the next tile's fragment is
      // read before the current tile's MFMAs, so LDS latency overlaps the matrix work
      auto load_bf = [&](int b, v8i& bf, int& sb) {
        const uint8_t* row = base + (16 * b + l16) * P::kRS;
        const uint32_t bsc = *reinterpret_cast<const uint32_t*>(base + P::kCodes + (16 * b + l16) * 8 + 4 * p);
        if constexpr (Mx<F>::kBits == 8) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 128 * p + 16 * q);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 128 * p + 64 + 16 * q);
          bf = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else if constexpr (Mx<F>::kBits == 6) {
          const uint8_t* pp = row + 24 * (4 * p + q);
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(pp);
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(pp + 8);
          const u32x2 x2 = *reinterpret_cast<const u32x2*>(pp + 16);
          bf = v8i{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
        } else {
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(row + 16 * (4 * p + q));
          bf = v8i{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
        }
        sb = (int)((bsc >> (8 * q)) & 0xFFu);
      };
      v8i bf[2];
      int sb[2];
      load_bf(0, bf[0], sb[0]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b + 1 < NB) load_bf(b + 1, bf[(b + 1) & 1], sb[(b + 1) & 1]);
#pragma unroll
        for (int t = 0; t < TA; ++t) {
          const u32x4 c = af4[t];
          const v8i af = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
          const int sa = (int)((was[t] >> (8 * q)) & 0xFFu);
          acc[t][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b & 1], acc[t][b], kWFmtFp4,
                                                                       Mx<F>::kMfma, 0, sa, 0, sb[b & 1]);
        }
      }
    }
  };

  // ---- pipeline.  Step s: at each position, a part of step s+1's activations goes into the other
  //      ring stage and the next part's loads start; the MFMAs of step s (its weights were written
  //      to the private copy during step s-1), replacing them with step s+1's and starting the
  //      loads of step s+2's weights; barrier.  Loads are issued unconditionally (a step past the
  //      end re-reads the last one), and in the same order before the loop as inside it, so the
  //      wait counts at the loop head hold for both of its entries.
  const int last = n_steps - 1;
  load_a(0);
  load_b(0, 0);
  store_a(0);
  store_b(0, 0);
  load_b(0, 1);
  store_b(0, 1);
  load_b(min(1, last), 0);
  load_a(min(1, last));
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    step(s & 1, s, min(s + 1, last), min(s + 2, last));
    __syncthreads();
  }
  if (!active) return;

  // ---- epilogue ----
  // Down: the slots of the lane's tokens, all loaded before the first store (a load between stores
  // would wait for every store before it).
  int yslot[GU ? 1 : NB];
  if constexpr (!GU) {
#pragma unroll
    for (int b = 0; b < NB; ++b) yslot[b] = sorted_slot[ti.r0 + min(16 * b + l16, ti.nr - 1)];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int sl = yslot[b];
      yslot[b] = (16 * b + l16 < ti.nr && sl >= 0 && sl < n_slots) ? sl : -1;
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int tok = 16 * b + l16;
    const bool ok = tok < ti.nr;
    if constexpr (GU) {
      // rows n0 + 8q + j (j = 4t + i) of this token: a quarter of h's block n0 / 32
      float v[8];
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // SiLU(g) * u with the hardware exp2 and reciprocal (about 2 ulp; -0 or 0 for g << 0)
          const float g = acc[t][b][i], u = acc[TM + t][b][i];
          const float ex = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
          v[4 * t + i] = g * u * __builtin_amdgcn_rcpf(1.0f + ex);
        }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const uint32_t sc = mx_scale_code<F>(amax);
      uint32_t dw[2];
      mx_pack_quarter<F>(v, mx_inv_scale(sc), dw);
      const int kb = n0 / 32;
      uint8_t* const blk = h_codes + (int64_t)(ti.r0 + tok) * ((N / 32) * P::kBB) + kb * P::kBB;
      if constexpr (Mx<F>::kBits == 6) {
        // 6 bytes per quarter: quarter pairs join into 12 bytes (4-byte aligned)
        const uint32_t o0 = (uint32_t)__shfl_xor((int)dw[0], 16, kWave);
        const uint32_t o1 = (uint32_t)__shfl_xor((int)dw[1], 16, kWave);
        if (ok && (q & 1) == 0) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(blk + 12 * (q >> 1));
          dst[0] = dw[0];
          dst[1] = (dw[1] & 0xFFFFu) | (o0 << 16);
          dst[2] = (o0 >> 16) | (o1 << 16);
        }
      } else if constexpr (Mx<F>::kBits == 8) {
        if (ok) *reinterpret_cast<u32x2*>(blk + 8 * q) = u32x2{dw[0], dw[1]};
      } else {
        if (ok) *reinterpret_cast<uint32_t*>(blk + 4 * q) = dw[0];
      }
      if (ok && q == 0) h_scales[(int64_t)(ti.r0 + tok) * (N / 32) + kb] = (uint8_t)sc;
    } else {
      // The 16 tokens x 64 rows of column tile b go through the wave's private LDS copy (free
      // after the last step): lane (token, q) writes rows 16q .. 16q+15 of its token, then each
      // store instruction writes 4 whole token rows (256 contiguous bytes each) of y.
      constexpr int kYS = 272;  // LDS bytes per token row (256 + 16: the 16 tokens on distinct banks)
      uint8_t* const ybuf = privA;
#pragma unroll
      for (int t = 0; t < TA; ++t) *reinterpret_cast<f32x4*>(ybuf + l16 * kYS + 64 * q + 16 * t) = acc[t][b];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tk = 4 * j + (lane >> 4), piece = lane & 15;  // token of the tile, 16-byte piece
        const int sl = __shfl(yslot[b], tk, kWave);
        const f32x4 v = *reinterpret_cast<const f32x4*>(ybuf + tk * kYS + 16 * piece);
        if (sl >= 0) *reinterpret_cast<f32x4*>(y_slots + (int64_t)sl * N + n0 + 4 * piece) = v;
      }
    }
  }
}

template <int F, bool GU>
__global__ __launch_bounds__(kMxNW * 64, 2) void ffn_mx_kernel(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_s, int n_act_rows, int k_total, int K, int N,
    ProjDev w0, ProjDev w1, const TileEntry* __restrict__ tiles, int n_experts,
    const int32_t* __restrict__ sorted_slot, int n_slots, int n_nblk, int n_items, uint8_t* __restrict__ h_codes,
    uint8_t* __restrict__ h_scales, float* __restrict__ y_slots) {
  // two workgroups per CU: a chunk of 64 items is what one XCD holds at once
  const int item = grouped_item(blockIdx.x, 2 * kCusPerXcd);
  if (item >= n_items) return;
  const int tile = item / n_nblk, nblk = item - tile * n_nblk;
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, kMxTok);
  if (ti.nr <= 0) return;
  // 16-token column tiles computed: the rows of the tile rounded up to 32
  switch ((ti.nr + 31) >> 5) {
    case 1:
      mx_tile<F, GU, 2>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    case 2:
      mx_tile<F, GU, 4>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    case 3:
      mx_tile<F, GU, 6>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    default:
      mx_tile<F, GU, 8>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
  }
}

template <int F>
hipError_t quantize_fmt(const void* x, bool x_fp16, int64_t n_blocks, uint8_t* codes, uint8_t* scales,
                        hipStream_t stream) {
  const unsigned grid = (unsigned)((n_blocks + 255) / 256);
  if (x_fp16)
    mx_quantize_kernel<F, true><<<grid, 256, 0, stream>>>((const uint16_t*)x, n_blocks, codes, scales);
  else
    mx_quantize_kernel<F, false><<<grid, 256, 0, stream>>>((const uint16_t*)x, n_blocks, codes, scales);
  return hipGetLastError();
}

template <int F>
hipError_t ffn_mx_fmt(const MxFfnArgs& a, hipStream_t stream) {
  const int n_slots = a.T * a.k_total;
  hipError_t err = quantize_fmt<F>(a.x, false, (int64_t)a.T * a.H / 32, a.xq, a.xs, stream);
  if (err != hipSuccess) return err;
  const int64_t tiles = mx_tiles(a.T, a.k_total, a.n_experts);
  err = launch_ffn_tiles(a.offsets, a.n_experts, n_slots, kMxTok, tiles, a.table, stream);
  if (err != hipSuccess) return err;
  const size_t lds = (size_t)MxTile<F>::kLds;
  constexpr int64_t kGroup = (int64_t)kXcds * 2 * kCusPerXcd;  // grid granule of the grouped item map
  {
    const int nb = (a.I + kMxNW * 32 - 1) / (kMxNW * 32);
    const int64_t items = tiles * nb;
    ffn_mx_kernel<F, true><<<dim3((unsigned)((items + kGroup - 1) / kGroup * kGroup)), kMxNW * 64, lds, stream>>>(
        a.xq, a.xs, a.T, a.k_total, a.H, a.I, a.gate, a.up, (const TileEntry*)a.table, a.n_experts,
        a.sorted_slot, n_slots, nb, (int)items, a.hq, a.hs, nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  {
    const int nb = (a.H + kMxNW * 64 - 1) / (kMxNW * 64);
    const int64_t items = tiles * nb;
    ffn_mx_kernel<F, false><<<dim3((unsigned)((items + kGroup - 1) / kGroup * kGroup)), kMxNW * 64, lds, stream>>>(
        a.hq, a.hs, n_slots, a.k_total, a.I, a.H, a.down, a.down, (const TileEntry*)a.table, a.n_experts,
        a.sorted_slot, n_slots, nb, (int)items, nullptr, nullptr, a.y_slots);
  }
  return hipGetLastError();
}

}  // namespace

int mx_bits(int fmt) {
  return fmt == MOE_MX_FP8_E4M3 ? 8 : (fmt == MOE_MX_FP6_E2M3 ? 6 : (fmt == MOE_MX_FP4_E2M1 ? 4 : 0));
}

int64_t mx_tiles(int T, int k_total, int n_experts) {
  return (max_tiles((int64_t)T * k_total, n_experts, kMxTok) + kXcds - 1) / kXcds * kXcds;
}

hipError_t launch_mx_quantize(const void* x, bool x_fp16, int64_t n_rows, int K, int fmt, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  const int64_t n_blocks = n_rows * (K / 32);
  switch (fmt) {
    case MOE_MX_FP8_E4M3: return quantize_fmt<MOE_MX_FP8_E4M3>(x, x_fp16, n_blocks, codes, scales, stream);
    case MOE_MX_FP6_E2M3: return quantize_fmt<MOE_MX_FP6_E2M3>(x, x_fp16, n_blocks, codes, scales, stream);
    case MOE_MX_FP4_E2M1: return quantize_fmt<MOE_MX_FP4_E2M1>(x, x_fp16, n_blocks, codes, scales, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ffn_mx(const MxFfnArgs& a, hipStream_t stream) {
  switch (a.fmt) {
    case MOE_MX_FP8_E4M3: return ffn_mx_fmt<MOE_MX_FP8_E4M3>(a, stream);
    case MOE_MX_FP6_E2M3: return ffn_mx_fmt<MOE_MX_FP6_E2M3>(a, stream);
    case MOE_MX_FP4_E2M1: return ffn_mx_fmt<MOE_MX_FP4_E2M1>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
