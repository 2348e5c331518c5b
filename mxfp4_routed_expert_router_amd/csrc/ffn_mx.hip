// MX mode of the grouped SwiGLU expert FFN (prefill).  The FP4 weights are used as they are stored
// (E2M1 codes with one E8M0 scale per 32 values along K, "DeepSeek-V4-Flash on a four-GPU Ampere
// workstation", section "MXFP4 is not NVFP4") and the activations -- x, then h -- are quantised on
// the fly to an MX element format with their own E8M0 scale per 32 values along K.  Gate/up and
// down then run as scaled MFMAs, v_mfma_scale_f32_32x32x64_f8f6f4, which multiply FP4 weights by
// FP8/FP6/FP4 activations and apply both block scales in the matrix core.
//
// The activation formats are the OCP Microscaling element formats E4M3, E2M3 and E2M1 with the
// scale rule X = 2^(floor(log2 amax) - emax) (emax = 8, 2, 2) and round-to-nearest-even,
// saturating element encoding.  They are not on the pages; this mode trades accuracy against the
// exact path for matrix-core rate and is checked against a quantisation-aware oracle.
//
// Operand layout of the 32x32x64 scaled MFMA (lane l, row/column l%32, half g = l/32):
//   FP4 or FP6 operand: lane holds the 32 contiguous values of K-block g (FP4: 16 bytes, element
//     j in nibble j of the little-endian 128-bit string; FP6: 24 bytes, element j in bits
//     6j..6j+5 of the little-endian 192-bit string);
//   FP8 operand: lane holds values 16g..16g+15 of K-block 0 in bytes 0..15 and values
//     16g..16g+15 of K-block 1 in bytes 16..31;
//   the E8M0 scale of a lane applies to K-block g of its row (A) or column (B);
//   D: lane l holds column l%32, rows 8*(i/4) + 4*g + i%4 in accumulator i.
// MFMA m (0..3) of a 256-wide K step covers the step's K-blocks 2m and 2m+1 in memory order, so
// weights, activation codes and scales are all read in their stored order.
//
// Work split.  A workgroup (4 waves) takes one 128-token tile of an expert (the tile table of the
// exact path, built with 128 rows per tile) and 4 * 64 rows of I (gate/up: 64 rows of each matrix
// per wave) or 4 * 128 rows of H (down: 128 rows per wave).  Each wave streams its FP4 weight rows
// straight from memory into registers, one step ahead; the tile's activation codes and scales go
// through a two-stage LDS ring shared by the four waves, written one step ahead, with one barrier
// per step.  Workgroups are numbered tile-major with the row blocks padded to a multiple of 8, so
// row block j of every tile runs on XCD j % 8 and the tiles of a hot expert read each weight row
// from one L2.  Only the 32-token column tiles that hold rows of the tile are computed.
//
// The gate/up epilogue forms h = SiLU(g) * u in fp32, exchanges half of each 32-row block between
// lane halves so that every lane holds one whole K-block of h for its token, and writes that
// block's codes and E8M0 scale -- the layout the down phase reads.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
constexpr int kMxStepK = 256;  // K per step: 8 blocks of 32

template <int F>
struct MxTile {
  static constexpr int kBB = 4 * Mx<F>::kBits;             // bytes per 32-value block
  static constexpr int kRowStep = 8 * kBB;                 // code bytes of one token per step
  static constexpr int kRS = kRowStep + 16;                // LDS row stride (padded)
  static constexpr int kCodes = kMxTok * kRS;              // code bytes of a stage
  static constexpr int kStage = kCodes + kMxTok * 8;       // + 8 scale bytes per token
  static constexpr int kPieces = kRowStep / 16;            // 16-byte pieces per token per step
  static constexpr int kLPT = kMxTok * kPieces / (64 * kMxNW);  // fill loads per thread per step
  static_assert(kLPT * 64 * kMxNW == kMxTok * kPieces, "a step of codes over the workgroup");
};

template <int GU>
struct WRows {
  static constexpr int kPerWave = GU ? 64 : 128;  // rows of I (of each of gate, up) or of H
};

// Weight registers of one step: 4 row tiles x 4 MFMAs x 16 bytes, plus 8 scale bytes per tile.
struct MxA {
  u32x4 c[4][4];
  uint32_t s[4][2];
};

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
  const int l32 = lane & 31, g = lane >> 5;
  constexpr int RPW = WRows<GU>::kPerWave;
  const int n0 = (nblk * kMxNW + wave) * RPW;
  const bool active = n0 < N;  // N % RPW == 0, so a wave's rows are all in or all out
  const int e = ti.e;
  const int n_steps = K / kMxStepK;
  const int RB = (K / 32) * P::kBB, KB = K / 32;

  // ---- LDS fill addressing: piece q = threadIdx.x + 256 i -> token q / kPieces, column q % kPieces
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
    const int q = threadIdx.x + 64 * kMxNW * i, tok = q / P::kPieces, col = q % P::kPieces;
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

  // ---- weight addressing: tile a covers rows n0 + 32*(a % 2) + l32 of gate (a < 2) / up (a >= 2)
  //      for gate/up, rows n0 + 32*a + l32 of down
  const int64_t wrows = (int64_t)N - 1;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(w0.w + (int64_t)e * w0.we, wrows * w0.wr + K / 2);
  const __amdgpu_buffer_rsrc_t sr0 = make_rsrc(w0.s + (int64_t)e * w0.se, wrows * w0.sr + K / 32);
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(w1.w + (int64_t)e * w1.we, wrows * w1.wr + K / 2);
  const __amdgpu_buffer_rsrc_t sr1 = make_rsrc(w1.s + (int64_t)e * w1.se, wrows * w1.sr + K / 32);
  uint32_t woff[4], soff[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int row = GU ? n0 + 32 * (a & 1) + l32 : n0 + 32 * a + l32;
    const ProjDev& p = (GU && a >= 2) ? w1 : w0;
    woff[a] = active ? (uint32_t)(row * p.wr) + 16u * g : kOutOfRange;
    soff[a] = active ? (uint32_t)(row * p.sr) : kOutOfRange;
  }
  auto load_a = [&](int s, MxA& A) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const __amdgpu_buffer_rsrc_t wr = (GU && a >= 2) ? wr1 : wr0;
      const __amdgpu_buffer_rsrc_t sr = (GU && a >= 2) ? sr1 : sr0;
#pragma unroll
      for (int m = 0; m < 4; ++m) A.c[a][m] = bld16(wr, woff[a] + (uint32_t)(s * 128 + 32 * m));
      A.s[a][0] = bld4(sr, soff[a] + (uint32_t)(s * 8));
      A.s[a][1] = bld4(sr, soff[a] + (uint32_t)(s * 8 + 4));
    }
  };
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
    for (int i = 0; i < P::kLPT; ++i) *reinterpret_cast<u32x4*>(base + aw[i]) = fill[i];
    *reinterpret_cast<uint32_t*>(base + asw) = fills;
  };

  f32x16 acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};

  // byte 2m + g of a step's 8 scale bytes (dwords lo, hi)
  auto sbyte = [&](uint32_t lo, uint32_t hi, int m) -> int {
    return (int)(((m < 2 ? lo : hi) >> (8 * (2 * (m & 1) + g))) & 0xFFu);
  };
  auto compute = [&](int stage, const MxA& A) {
    if (!active) return;
    const uint8_t* base = lds + stage * P::kStage;
    uint32_t bs[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const u32x2 t = *reinterpret_cast<const u32x2*>(base + P::kCodes + (32 * b + l32) * 8);
      bs[b][0] = t[0];
      bs[b][1] = t[1];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v8i bf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t* row = base + (32 * b + l32) * P::kRS;
        if constexpr (Mx<F>::kBits == 8) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 64 * m + 16 * g);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 64 * m + 32 + 16 * g);
          bf[b] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else if constexpr (Mx<F>::kBits == 6) {
          const uint8_t* p = row + 24 * (2 * m + g);
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(p);
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(p + 8);
          const u32x2 x2 = *reinterpret_cast<const u32x2*>(p + 16);
          bf[b] = v8i{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
        } else {
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(row + 16 * (2 * m + g));
          bf[b] = v8i{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int sb = sbyte(bs[b][0], bs[b][1], m);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x4 c = A.c[a][m];
          const v8i af = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af, bf[b], acc[a][b], kWFmtFp4, Mx<F>::kMfma, 0, sbyte(A.s[a][0], A.s[a][1], m), 0, sb);
        }
      }
    }
  };

  // ---- pipeline: weights one step ahead in registers, activations one step ahead in LDS.  The
  //      loads are issued unconditionally (a step past the end re-reads the last one) so every
  //      iteration has the same outstanding-load pattern.
  MxA A0, A1;
  load_b(0);
  load_a(0, A0);
  store_b(0);
  load_b(min(1, n_steps - 1));
  __syncthreads();
  for (int s = 0; s < n_steps; s += 2) {
    load_a(min(s + 1, n_steps - 1), A1);
    store_b((s + 1) & 1);
    load_b(min(s + 2, n_steps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s & 1, A0);
    __syncthreads();
    if (s + 1 >= n_steps) break;
    load_a(min(s + 2, n_steps - 1), A0);
    store_b(s & 1);
    load_b(min(s + 3, n_steps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute((s + 1) & 1, A1);
    __syncthreads();
  }
  if (!active) return;

  // ---- epilogue ----
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int tok = 32 * b + l32;
    const bool ok = tok < ti.nr;
    if constexpr (GU) {
      // h of the wave's two 32-row blocks; lanes g = 0 keep block 0, lanes g = 1 block 1
      float own[16], rcv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float g0 = acc[0][b][i], u0 = acc[2][b][i], g1 = acc[1][b][i], u1 = acc[3][b][i];
        const float h0 = (g0 / (1.0f + expf(-g0))) * u0;
        const float h1 = (g1 / (1.0f + expf(-g1))) * u1;
        own[i] = g ? h1 : h0;
        rcv[i] = __shfl_xor(g ? h0 : h1, 32, kWave);
      }
      // block element 8q + 4g' + r sits in lane half g' at accumulator 4q + r
      float blk[32];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          blk[8 * q + r] = g ? rcv[4 * q + r] : own[4 * q + r];
          blk[8 * q + 4 + r] = g ? own[4 * q + r] : rcv[4 * q + r];
        }
      uint32_t dw[8];
      const uint32_t sc = mx_pack_block<F>(blk, dw);
      if (ok) {
        const int row = ti.r0 + tok, kb = n0 / 32 + g;
        mx_store_block<F>(h_codes + (int64_t)row * ((N / 32) * P::kBB) + kb * P::kBB, dw);
        h_scales[(int64_t)row * (N / 32) + kb] = (uint8_t)sc;
      }
    } else {
      const int sl = ok ? sorted_slot[ti.r0 + tok] : -1;
      if (sl >= 0 && sl < n_slots) {
        float* dst = y_slots + (int64_t)sl * N + n0 + 4 * g;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(dst + 32 * a + 8 * q) =
                f32x4{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]};
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
  switch ((ti.nr + 31) >> 5) {
    case 1:
      mx_tile<F, GU, 1>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    case 2:
      mx_tile<F, GU, 2>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    case 3:
      mx_tile<F, GU, 3>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
                        h_scales, y_slots);
      break;
    default:
      mx_tile<F, GU, 4>(ti, nblk, act, act_s, n_act_rows, k_total, K, N, w0, w1, sorted_slot, n_slots, h_codes,
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
  const size_t lds = 2 * (size_t)MxTile<F>::kStage;
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
