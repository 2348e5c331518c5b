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
// Work split.  A workgroup (4 waves) takes one 128-token tile of an expert (the tile table of the
// exact path, built with 128 rows per tile) and 4 * 64 rows of I (gate/up: 64 rows of each matrix
// per wave) or 4 * 128 rows of H (down: 128 rows per wave).  Each wave streams its FP4 weight rows
// straight from memory into registers, one step ahead, every instruction reading whole 64-byte
// pieces of 16 rows; the tile's activation codes and scales go through a two-stage LDS ring
// shared by the four waves, written one step ahead, with one barrier per step.  Workgroups are
// numbered tile-major with the row blocks padded to a multiple of 8, so row block j of every tile
// runs on XCD j % 8 and the tiles of a hot expert read each weight row from one L2.  Only the
// 16-token column tiles that hold rows of the tile (rounded up to 32 tokens) are computed.
//
// The gate/up epilogue forms h = SiLU(g) * u in fp32, exchanges values between the four lane
// quarters so that each lane holds 16 consecutive values of h for its token (half a K-block), and
// writes their codes and the block's E8M0 scale -- the layout the down phase reads.
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

// One 32-value block: E8M0 code and the packed element codes (4 * bits bytes in dw[0 .. bits/2)).
template <int F>
__device__ __forceinline__ uint32_t mx_pack_block(const float (&v)[32], uint32_t (&dw)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t sc = mx_scale_code<F>(amax);
  const float inv = mx_inv_scale(sc);
#pragma unroll
  for (int i = 0; i < 8; ++i) dw[i] = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t c = mx_encode<F>(v[j] * inv);
    constexpr int B = Mx<F>::kBits;
    const int bit = B * j, w = bit >> 5, o = bit & 31;
    dw[w] |= c << o;
    if (o + B > 32) dw[w + 1] |= c >> (32 - o);
  }
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
constexpr int kMxNW = 4;       // waves per workgroup
constexpr int kMxTok = 128;    // sorted rows (tokens) per tile
constexpr int kMxStepK = 256;  // K per step: 8 blocks of 32 (two MFMA K positions of 128)

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
  // After the two stages: per wave, a private copy of its 128 weight rows for one step (128 bytes
  // per row, 16-byte pieces XOR-swizzled by row) and their 8 scale bytes.
  static constexpr int kPrivA = 2 * kStage;
  static constexpr int kPrivS = kPrivA + kMxNW * 128 * 128;
  static constexpr int kLds = kPrivS + kMxNW * 128 * 8;
  static constexpr int kPieces = kRowStep / 16;            // 16-byte pieces per token per step
  static constexpr int kLPT = kMxTok * kPieces / (64 * kMxNW);  // fill loads per thread per step
  static_assert(kLPT * 64 * kMxNW == kMxTok * kPieces, "a step of codes over the workgroup");
};

template <int GU>
struct WRows {
  static constexpr int kPerWave = GU ? 64 : 128;  // rows of I (of each of gate, up) or of H
};

// Codes of 16 consecutive values (half a block) packed as in the block layout: 2 * bits bytes.
template <int F>
__device__ __forceinline__ void mx_pack_half(const float (&v)[16], float inv, uint32_t (&dw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dw[i] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t c = mx_encode<F>(v[j] * inv);
    constexpr int B = Mx<F>::kBits;
    const int bit = B * j, w = bit >> 5, o = bit & 31;
    dw[w] |= c << o;
    if (o + B > 32) dw[w + 1] |= c >> (32 - o);
  }
}

// MFMA layout (v_mfma_scale_f32_16x16x128_f8f6f4, lane l, row/column l%16, quarter q = l/16):
//   FP4/FP6 operand: K-block q of the 128-wide position (32 contiguous values);
//   FP8 operand: values 16(q%2)..+15 of K-blocks q/2 and 2 + q/2;
//   E8M0 scale of a lane: K-block q of its row or column;
//   D: lane l holds column l%16, rows 4q + i in accumulator i.
// A 256-wide step holds positions p = 0, 1 over its K-blocks 4p .. 4p+3 in memory order, so the
// four lanes of a weight row read one contiguous 64-byte piece per position.
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
  constexpr int RPW = WRows<GU>::kPerWave;
  const int n0 = (nblk * kMxNW + wave) * RPW;
  const bool active = n0 < N;  // N % RPW == 0, so a wave's rows are all in or all out
  const int e = ti.e;
  const int n_steps = K / kMxStepK;
  const int RB = (K / 32) * P::kBB, KB = K / 32;

  // ---- LDS fill addressing: piece i of a thread -> token (threadIdx.x + 256 i) / kPieces
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
  uint32_t aoff[P::kLPT], aw[P::kLPT];
#pragma unroll
  for (int i = 0; i < P::kLPT; ++i) {
    const int qq = threadIdx.x + 64 * kMxNW * i, tok = qq / P::kPieces, col = qq % P::kPieces;
    const int row = act_row(tok);
    aoff[i] = row >= 0 ? (uint32_t)row * (uint32_t)RB + 16u * col : kOutOfRange;
    aw[i] = (uint32_t)(tok * P::kRS + 16 * col);
  }
  uint32_t asoff, asw;
  {
    const int tok = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int row = act_row(tok);
    asoff = row >= 0 ? (uint32_t)row * (uint32_t)KB + 4u * half : kOutOfRange;
    asw = (uint32_t)(P::kCodes + tok * 8 + 4 * half);
  }

  // ---- weights: wave row r (0..127) is row r % 16 of tile t = r / 16, i.e. row n0 + 16*(t % 4) +
  //      r % 16 of gate (t < 4) / up (t >= 4) for gate/up, row n0 + r of down.  A step's 128 bytes
  //      of the wave's rows are loaded as whole 128-byte lines (8 lanes per row, 8 rows per
  //      instruction), written to the wave's private LDS copy with piece c of row r in slot
  //      c ^ (r & 7), and read back in MFMA layout (conflict-free both ways).  Loads run two steps
  //      ahead of the MFMAs: staged in registers one step, in LDS the next.
  const int64_t wrows = (int64_t)N - 1;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(w0.w + (int64_t)e * w0.we, wrows * w0.wr + K / 2);
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(w1.w + (int64_t)e * w1.we, wrows * w1.wr + K / 2);
  const __amdgpu_buffer_rsrc_t sr0 = make_rsrc(w0.s + (int64_t)e * w0.se, wrows * w0.sr + K / 32);
  const __amdgpu_buffer_rsrc_t sr1 = make_rsrc(w1.s + (int64_t)e * w1.se, wrows * w1.sr + K / 32);
  const int lr = lane >> 3, lc = lane & 7;  // line loads: row lr of 8, 16-byte piece lc
  const uint32_t lv0 = active ? (uint32_t)((n0 + lr) * w0.wr) + 16u * lc : kOutOfRange;
  const uint32_t lv1 = active ? (uint32_t)((n0 + lr) * w1.wr) + 16u * lc : kOutOfRange;
  const uint32_t wt0 = (uint32_t)(16 * w0.wr), wt1 = (uint32_t)(16 * w1.wr);  // per 16-row tile
  // scale rows of lane l: wave rows l and 64 + l
  const uint32_t sv0 = active ? (uint32_t)((n0 + lane) * w0.sr) : kOutOfRange;
  const uint32_t sv1 = active ? (GU ? (uint32_t)((n0 + lane) * w1.sr) : (uint32_t)((n0 + 64 + lane) * w0.sr)) : kOutOfRange;
  u32x4 ast[16];
  u32x2 sst[2];
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = i >> 1;
      const bool second = GU && t >= 4;
      const uint32_t tt = GU ? (uint32_t)(t & 3) : (uint32_t)t;
      const uint32_t wt = second ? wt1 : wt0;
      ast[i] = bld16s(second ? wr1 : wr0, second ? lv1 : lv0, wt * tt + (wt >> 1) * (uint32_t)(i & 1) + (uint32_t)(s * 128));
    }
    sst[0] = bld8(sr0, sv0 + (uint32_t)(s * 8));
    sst[1] = bld8(GU ? sr1 : sr0, sv1 + (uint32_t)(s * 8));
  };
  uint8_t* const privA = lds + P::kPrivA + wave * (128 * 128);
  uint8_t* const privS = lds + P::kPrivS + wave * (128 * 8);
  const uint32_t wslot = (uint32_t)(lr * 128 + 16 * (lc ^ lr));  // + 1024 per instruction
  auto store_a = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(privA + 1024 * i + wslot) = ast[i];
    *reinterpret_cast<u32x2*>(privS + 8 * lane) = sst[0];
    *reinterpret_cast<u32x2*>(privS + 8 * (64 + lane)) = sst[1];
  };
  // MFMA-layout reads: tile t, position p -> row 16t + l16, piece 4p + q in slot (4p + q) ^ (l16 & 7)
  const uint32_t rslot0 = (uint32_t)(l16 * 128 + 16 * ((0 + q) ^ (l16 & 7)));
  const uint32_t rslot1 = (uint32_t)(l16 * 128 + 16 * ((4 + q) ^ (l16 & 7)));

  u32x4 fill[P::kLPT];
  uint32_t fills;
  auto load_b = [&](int s) {
#pragma unroll
    for (int i = 0; i < P::kLPT; ++i) fill[i] = bld16(ar, aoff[i] + (uint32_t)(s * P::kRowStep));
    fills = bld4(asr, asoff + (uint32_t)(s * 8));
  };
  auto store_b = [&](int stage) {
    uint8_t* base = lds + stage * P::kStage;
#pragma unroll
    for (int i = 0; i < P::kLPT; ++i) {
      if constexpr (Mx<F>::kBits == 6) {  // 8-byte aligned rows
        *reinterpret_cast<u32x2*>(base + aw[i]) = u32x2{fill[i][0], fill[i][1]};
        *reinterpret_cast<u32x2*>(base + aw[i] + 8) = u32x2{fill[i][2], fill[i][3]};
      } else {
        *reinterpret_cast<u32x4*>(base + aw[i]) = fill[i];
      }
    }
    *reinterpret_cast<uint32_t*>(base + asw) = fills;
  };

  f32x4 acc[8][NB];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step of MFMAs over the stage's activations and the wave's private weight copy, position
  // by position (so only one position's weight operands are in registers).  After the last reads
  // of the private copy, the next step's weights (staged in registers) are written in their place
  // and the loads of the step after that are started.
  auto step = [&](int stage, int s_next2) {
    const uint8_t* base = lds + stage * P::kStage;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4 af4[8];
      uint32_t was[8];
      if (active) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          af4[t] = *reinterpret_cast<const u32x4*>(privA + 2048 * t + (p ? rslot1 : rslot0));
          was[t] = *reinterpret_cast<const uint32_t*>(privS + 8 * (16 * t + l16) + 4 * p);
        }
      }
      if (p == 1) {
        if (active) store_a();  // LDS accesses of a wave stay in order: the reads above come first
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
        for (int t = 0; t < 8; ++t) {
          const u32x4 c = af4[t];
          const v8i af = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
          const int sa = (int)((was[t] >> (8 * q)) & 0xFFu);
          acc[t][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b & 1], acc[t][b], kWFmtFp4,
                                                                       Mx<F>::kMfma, 0, sa, 0, sb[b & 1]);
        }
      }
    }
  };

  // ---- pipeline.  Step s: write step s+1's activations (loaded during step s-1) into the other
  //      ring stage and start loading step s+2's; MFMAs of step s (its weights were written to the
  //      private copy during step s-1), replacing them with step s+1's and starting the loads of
  //      step s+2's weights; barrier.  Loads are issued unconditionally (a step past the end
  //      re-reads the last one), so every iteration has the same outstanding loads.
  load_a(0);
  load_b(0);
  if (active) store_a();
  store_b(0);
  load_a(min(1, n_steps - 1));
  load_b(min(1, n_steps - 1));
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    store_b((s + 1) & 1);
    load_b(min(s + 2, n_steps - 1));
    __builtin_amdgcn_sched_barrier(0);
    step(s & 1, min(s + 2, n_steps - 1));
    __syncthreads();
  }
  if (!active) return;

  // ---- epilogue ----
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int tok = 16 * b + l16;
    const bool ok = tok < ti.nr;
    if constexpr (GU) {
      // h of the wave's 64 rows for this token: lane quarter q' holds rows 16t + 4q' + i (t = 0..3).
      // A 4 x 4 exchange over the quarters leaves quarter q with rows 16q .. 16q+15, i.e. half
      // q % 2 of block q / 2 of the wave.
      float h[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[t][b][i], u = acc[4 + t][b][i];
          h[t][i] = (g / (1.0f + expf(-g))) * u;
        }
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // round r: send the rows of tile q ^ r (the tile of the receiving quarter q ^ r), receive
        // the rows 4 (q ^ r) + i of tile q from quarter q ^ r
        const int ts = q ^ r;
        float got[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float snd = ts == 0 ? h[0][i] : (ts == 1 ? h[1][i] : (ts == 2 ? h[2][i] : h[3][i]));
          got[i] = r == 0 ? snd : __shfl_xor(snd, 16 * r, kWave);
        }
        // source quarter j = q ^ r: place at v[4j + i] with a select over j
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * j + i] = (j == (q ^ r)) ? got[i] : v[4 * j + i];
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));  // the block's other half: quarter q ^ 1
      const uint32_t sc = mx_scale_code<F>(amax);
      uint32_t dw[4];
      mx_pack_half<F>(v, mx_inv_scale(sc), dw);
      if (ok) {
        const int row = ti.r0 + tok, kb = n0 / 32 + (q >> 1);
        uint8_t* dst = h_codes + (int64_t)row * ((N / 32) * P::kBB) + kb * P::kBB + (q & 1) * (P::kBB / 2);
        if constexpr (Mx<F>::kBits == 8) {
          st16(dst, u32x4{dw[0], dw[1], dw[2], dw[3]});
        } else if constexpr (Mx<F>::kBits == 6) {
#pragma unroll
          for (int i = 0; i < 3; ++i) *reinterpret_cast<uint32_t*>(dst + 4 * i) = dw[i];
        } else {
          *reinterpret_cast<u32x2*>(dst) = u32x2{dw[0], dw[1]};
        }
        if ((q & 1) == 0) h_scales[(int64_t)row * (N / 32) + kb] = (uint8_t)sc;
      }
    } else {
      const int sl = ok ? sorted_slot[ti.r0 + tok] : -1;
      if (sl >= 0 && sl < n_slots) {
        float* dst = y_slots + (int64_t)sl * N + n0 + 4 * q;
#pragma unroll
        for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t) = acc[t][b];
      }
    }
  }
}

template <int F, bool GU>
__global__ __launch_bounds__(kMxNW * 64, 1) void ffn_mx_kernel(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_s, int n_act_rows, int k_total, int K, int N,
    ProjDev w0, ProjDev w1, const TileEntry* __restrict__ tiles, int n_experts,
    const int32_t* __restrict__ sorted_slot, int n_slots, int n_nblk, int n_nblk_pad, uint8_t* __restrict__ h_codes,
    uint8_t* __restrict__ h_scales, float* __restrict__ y_slots) {
  const int tile = blockIdx.x / n_nblk_pad, nblk = blockIdx.x - tile * n_nblk_pad;
  if (nblk >= n_nblk) return;
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
  {
    const int nb = (a.I + kMxNW * 64 - 1) / (kMxNW * 64), nbp = (nb + kXcds - 1) / kXcds * kXcds;
    ffn_mx_kernel<F, true><<<dim3((unsigned)(tiles * nbp)), kMxNW * 64, lds, stream>>>(
        a.xq, a.xs, a.T, a.k_total, a.H, a.I, a.gate, a.up, (const TileEntry*)a.table, a.n_experts,
        a.sorted_slot, n_slots, nb, nbp, a.hq, a.hs, nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  {
    const int nb = (a.H + kMxNW * 128 - 1) / (kMxNW * 128), nbp = (nb + kXcds - 1) / kXcds * kXcds;
    ffn_mx_kernel<F, false><<<dim3((unsigned)(tiles * nbp)), kMxNW * 64, lds, stream>>>(
        a.hq, a.hs, n_slots, a.k_total, a.I, a.H, a.down, a.down, (const TileEntry*)a.table, a.n_experts,
        a.sorted_slot, n_slots, nb, nbp, nullptr, nullptr, a.y_slots);
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
