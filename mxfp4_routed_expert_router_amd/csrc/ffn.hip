// Grouped SwiGLU expert FFN over the buckets (Cascadia, Sec. 3.1), with the MXFP4 weights decoded
// in registers as part of each dot product and summed in FP32 (FreeToken DeepSeek-V4-Flash post,
// "MXFP4 is not NVFP4"): every lane fetches a block's scale byte together with its 16 code bytes,
// and the decoded weights exist only as MFMA operands, never as a bf16 matrix in memory.
//
// Work unit.  A "tile" is up to 16*MT consecutive sorted rows (tokens) of one expert; tiles are
// numbered expert by expert, so an expert with n rows owns ceil(n / (16*MT)) tiles.  A workgroup
// takes one tile and one block of weight rows and covers the full reduction dimension K, so the
// weights are read from HBM once per tile -- once per active expert when an expert has at most
// 16*MT tokens, which is the decode regime.  Four kernel families split that work differently:
//   K-split (general and streaming kernels): the NW waves reduce contiguous shares of K's
//     128-wide chunks for the same 16*RT rows, and the partial sums meet in LDS (few tiles);
//   row-split streaming kernels: the waves own different rows over the whole K and share the
//     tile's activations (or h) through LDS (many small tiles: the decode sweep);
//   tile kernels: 128-token tiles for experts with many rows (prefill).
//
// MFMA mapping (v_mfma_f32_16x16x32_{bf16,f16}).  A = 16 weight rows x 32 k, B = 32 k x 16 tokens,
// D = 16 rows x 16 tokens.  Lane l holds A row l%16 and B column l%16 with k slots
// 8*(l/16) .. +8.  Per 128-wide chunk, lane l loads ONE 16-byte MXFP4 block: 32 codes of row l%16
// covering k = chunk*128 + 32*(l/16) + [0, 32), plus that block's scale byte; step s of the
// four MFMAs of the chunk uses codes 8s .. 8s+7 of the block (one dword, decoded by
// v_cvt_scalef32_pk_bf16_fp4 -- exact for every finite result).  B is loaded with the same k
// permutation, so every product pairs the right weight with the right activation.
// D: lane l holds rows 4*(l/16) + i (i = 0..3) of token l%16.
//
// Precision.  Decoded weights and bf16 activations are exact MFMA operands; products are exact in
// fp32 and accumulate in fp32.  h = SiLU(g)*u is formed in fp32 and stored as a bf16 high part and
// a bf16 low part (h - hi); the down projection runs one MFMA on each, so h keeps ~16 significant
// bits.  FP16 weights use the f16 MFMA with fp16 activations and an fp16 high/low pair for h.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {

// Builds the tile table (TileEntry, tiles.hpp) from the bucket offsets: one thread per expert
// (MOE_MAX_EXPERTS <= 1024), a block-wide scan of the tile counts, then each expert's entries.
__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t* __restrict__ offsets, int n_experts,
                                                         int n_rows_max, int rows_per_tile, int n_entries,
                                                         TileEntry* __restrict__ table) {
  __shared__ int wsum[16];
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // tiles of expert tid (offsets clamped, so corrupt device data cannot produce rows outside
  // [0, n_rows_max))
  int a = 0, n = 0, cnt = 0;
  if (tid < n_experts) {
    a = min(max(offsets[tid], 0), n_rows_max);
    const int b = min(max(offsets[tid + 1], 0), n_rows_max);
    n = max(b - a, 0);
    cnt = (n + rows_per_tile - 1) / rows_per_tile;
  }
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int v = wsum[w];
      wsum[w] = run;
      run += v;
    }
    s_total = run;
  }
  __syncthreads();
  const int first = wsum[wave] + incl - cnt;
  // (the bound on n_entries holds for offsets from moe_bucket; the guard keeps inconsistent offsets
  // from writing past the table)
  for (int p = 0; p < cnt && first + p < n_entries; ++p) {
    const int r0 = a + p * rows_per_tile;
    table[first + p] = TileEntry{tid, r0, min(rows_per_tile, a + n - r0), 0};
  }
  const int total = s_total;
  for (int t = total + tid; t < n_entries; t += blockDim.x) table[t] = TileEntry{0, 0, 0, 0};
}

template <int FMT>
struct Op;  // operand types per weight format

template <>
struct Op<MOE_W_MXFP4> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // h -> (hi, lo) pair in the operand type
  static __device__ __forceinline__ void split(float h, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(h);
    lo = f32_to_bf16_bits(h - bf16_bits_to_f32(hi));
  }
};
template <>
struct Op<MOE_W_FP16> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(float h, uint16_t& hi, uint16_t& lo) {
    _Float16 a = (_Float16)h;
    _Float16 b = (_Float16)(h - (float)a);
    hi = bitcast<uint16_t>(a);
    lo = bitcast<uint16_t>(b);
  }
};

// Cascadia's group-32 INT4 and NVFP4 weights run on the bf16 MFMA like MXFP4.
template <>
struct Op<MOE_W_INT4_G32> : Op<MOE_W_MXFP4> {};
template <>
struct Op<MOE_W_NVFP4> : Op<MOE_W_MXFP4> {};

// Decoded A operands of one MFMA step: NP planes whose sum is the exact weight.  INT4 group-32
// weights (code - zero) * scale carry up to 15 significant bits, so they take a bf16 high and a
// bf16 low plane (two MFMAs); every other format is exact in one operand.
template <int FMT>
struct Planes {
  static constexpr int n = FMT == MOE_W_INT4_G32 ? 2 : 1;
};
template <int FMT>
struct Dec {
  typename Op<FMT>::V p[Planes<FMT>::n];
};

// Raw weight data of one lane for one chunk and one 16-row tile: the 16-byte block of 32 codes
// and its scale data (MXFP4: the E8M0 byte; INT4: the group's binary16 scale and zero point;
// NVFP4: the E4M3 scales of its two 16-value blocks), or 4 x 16 bytes of fp16.
template <int FMT>
struct RawW;
template <>
struct RawW<MOE_W_MXFP4> {
  u32x4 q;
  uint32_t e;
};
template <>
struct RawW<MOE_W_FP16> {
  u32x4 q[4];
};
template <>
struct RawW<MOE_W_INT4_G32> {
  u32x4 q;
  float scale, zs;  // zs = -zero * scale (exact: 4 x 11 significant bits)
};
template <>
struct RawW<MOE_W_NVFP4> {
  u32x4 q;
  float s0, s1;
};

// E4M3 (bias 7, subnormals at exponent field 0; the NaN codes are outside the contract) -> fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, fr = c & 7u;
  const float mag = ex ? __uint_as_float(((ex + 120u) << 23) | (fr << 20)) : (float)fr * 0.001953125f;  // fr * 2^-9
  return (c & 0x80u) ? -mag : mag;
}

// Load lane's raw weights: row pointer `row` (already offset to expert and row), its scale row
// and (INT4) zero-point row, k = this lane's block start; ok = row and block inside the matrix.
template <int FMT>
__device__ __forceinline__ RawW<FMT> load_w(const uint8_t* row, const uint8_t* srow, const uint8_t* zrow, int k,
                                            bool ok) {
  RawW<FMT> r;
  if constexpr (FMT == MOE_W_MXFP4) {
    if (ok) {
      r.q = ld16(row + (k >> 1));
      r.e = srow[k >> 5];
    } else {
      r.q = u32x4{0, 0, 0, 0};
      r.e = 127;
    }
  } else if constexpr (FMT == MOE_W_INT4_G32) {
    if (ok) {
      const int g = k >> 5;
      r.q = ld16(row + (k >> 1));
      const uint32_t sb = (uint32_t)srow[2 * g] | ((uint32_t)srow[2 * g + 1] << 8);
      r.scale = (float)bitcast<_Float16>((uint16_t)sb);
      const uint32_t z = (zrow[g >> 1] >> (4 * (g & 1))) & 15u;
      r.zs = -(float)z * r.scale;
    } else {
      r.q = u32x4{0, 0, 0, 0};
      r.scale = 0.0f;
      r.zs = 0.0f;
    }
  } else if constexpr (FMT == MOE_W_NVFP4) {
    if (ok) {
      r.q = ld16(row + (k >> 1));
      r.s0 = e4m3_to_f32(srow[k >> 4]);
      r.s1 = e4m3_to_f32(srow[(k >> 4) + 1]);
    } else {
      r.q = u32x4{0, 0, 0, 0};
      r.s0 = r.s1 = 0.0f;
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) r.q[s] = ok ? ld16(row + 2 * (k + 8 * s)) : u32x4{0, 0, 0, 0};
  }
  return r;
}

// Two fp32 values whose low 16 bits are zero (at most 8 significant bits) -> a packed bf16 pair.
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// MFMA operands for step s of a lane's block: codes 8s .. 8s+7 (dword s).
template <int FMT>
__device__ __forceinline__ Dec<FMT> decode_step(const RawW<FMT>& r, int s) {
  Dec<FMT> d;
  if constexpr (FMT == MOE_W_MXFP4) {
    d.p[0] = decode8_bf16(r.q[s], e8m0_to_f32(r.e));
  } else if constexpr (FMT == MOE_W_INT4_G32) {
    // (code - zero) * scale = fma(code, scale, -zero * scale), exact in fp32 (at most 15
    // significant bits); truncating to bf16 keeps its top 8 bits, the remainder (at most 7 more)
    // is exact in bf16 too.
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[2], h[2], l[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t c = (r.q[s] >> (8 * i + 4 * j)) & 15u;
        v[j] = __builtin_fmaf((float)c, r.scale, r.zs);
        h[j] = __uint_as_float(__float_as_uint(v[j]) & 0xFFFF0000u);
        l[j] = v[j] - h[j];
      }
      hi[i] = pack_bf16_exact(h[0], h[1]);
      lo[i] = pack_bf16_exact(l[0], l[1]);
    }
    d.p[0] = bitcast<bf16x8>(u32x4{hi[0], hi[1], hi[2], hi[3]});
    d.p[1] = bitcast<bf16x8>(u32x4{lo[0], lo[1], lo[2], lo[3]});
  } else if constexpr (FMT == MOE_W_NVFP4) {
    // exact E2M1 values times the block's E4M3 scale: at most 2 x 4 = 6 significant bits, inside
    // bf16's range, so exact in bf16
    const float sc = s < 2 ? r.s0 : r.s1;
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q[s], 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q[s], 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q[s], 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q[s], 1.0f, 3);
    d.p[0] = bitcast<bf16x8>(u32x4{pack_bf16_exact(v0[0] * sc, v0[1] * sc), pack_bf16_exact(v1[0] * sc, v1[1] * sc),
                                   pack_bf16_exact(v2[0] * sc, v2[1] * sc), pack_bf16_exact(v3[0] * sc, v3[1] * sc)});
  } else {
    d.p[0] = bitcast<f16x8>(r.q[s]);
  }
  return d;
}

// The NVFP4 tensor scale of expert e of a projection (applied to the fp32 sums); 1 otherwise.
template <int FMT>
__device__ __forceinline__ float tensor_scale(const ProjDev& p, int e) {
  if constexpr (FMT == MOE_W_NVFP4) return p.ts[e];
  return 1.0f;
}

// ------------------------------------------------------------------------------------------------
// gate/up + SwiGLU:  h[r, n] = SiLU(sum_k Wg[e,n,k] x[t,k]) * (sum_k Wu[e,n,k] x[t,k])
// ------------------------------------------------------------------------------------------------
// u_scale and h_f16 serve the range-managed path (Cascadia Sec. 3.3, Eq. 1): u is multiplied by
// the layer's attenuation 1/A = u_scale (a power of two, so exact), and h is rounded to binary16
// before it is split, as the FP16 intermediate of that path.  u_scale = 1, h_f16 = 0 is the plain
// FFN.
template <int FMT, int NW, int RT, int MT>
__global__ __launch_bounds__(NW * 64) void ffn_gateup_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, float u_scale, int h_f16) {
  typedef typename Op<FMT>::V V;
  __shared__ float s_red[NW][RT][2][256];
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16 * MT);
  if (ti.nr <= 0) return;  // uniform across the workgroup
  // wave index in an SGPR: the K-share loop bounds are then wave-uniform (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;

  // B sources: the activation row of each of this lane's tokens
  const uint16_t* xrow[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    bool ok = m < ti.nr;
    int s = ok ? sorted_slot[ti.r0 + m] : -1;
    ok = ok && s >= 0 && s < n_slots;
    tok_ok[mt] = ok;
    xrow[mt] = x + (int64_t)(ok ? s / k_total : 0) * H;
  }
  // A sources: weight rows n0 + rt*16 + l16 of expert e
  const uint8_t *grow[RT], *urow[RT], *gsrow[RT], *usrow[RT], *gzrow[RT], *uzrow[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + rt * 16 + l16;
    row_ok[rt] = n < I;
    const int nn = row_ok[rt] ? n : 0;
    grow[rt] = gate.w + (int64_t)ti.e * gate.we + (int64_t)nn * gate.wr;
    urow[rt] = up.w + (int64_t)ti.e * up.we + (int64_t)nn * up.wr;
    gsrow[rt] = gate.s ? gate.s + (int64_t)ti.e * gate.se + (int64_t)nn * gate.sr : nullptr;
    usrow[rt] = up.s ? up.s + (int64_t)ti.e * up.se + (int64_t)nn * up.sr : nullptr;
    gzrow[rt] = gate.z ? gate.z + (int64_t)ti.e * gate.ze + (int64_t)nn * gate.zr : nullptr;
    uzrow[rt] = up.z ? up.z + (int64_t)ti.e * up.ze + (int64_t)nn * up.zr : nullptr;
  }

  const int n_chunks = (H + 127) >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);

  f32x4 accg[MT][RT], accu[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      accg[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // Software pipeline: the weights and activations of chunk c+1 are requested before chunk c is
  // decoded and multiplied.
  RawW<FMT> wg[RT], wu[RT];
  V xb[MT][4];
  auto load_x = [&](int k, V (&dst)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (tok_ok[mt] && k < H) v = ld16(xrow[mt] + k + 8 * s);
        dst[mt][s] = bitcast<V>(v);
      }
  };
  if (c0 < c1) {
    const int k = c0 * 128 + 32 * lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wg[rt] = load_w<FMT>(grow[rt], gsrow[rt], gzrow[rt], k, row_ok[rt] && k < H);
      wu[rt] = load_w<FMT>(urow[rt], usrow[rt], uzrow[rt], k, row_ok[rt] && k < H);
    }
    load_x(k, xb);
  }
  for (int c = c0; c < c1; ++c) {
    const int k = c * 128 + 32 * lq;
    RawW<FMT> ng[RT], nu[RT];
    V nx[MT][4];
    if (c + 1 < c1) {
      const int kn = k + 128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        ng[rt] = load_w<FMT>(grow[rt], gsrow[rt], gzrow[rt], kn, row_ok[rt] && kn < H);
        nu[rt] = load_w<FMT>(urow[rt], usrow[rt], uzrow[rt], kn, row_ok[rt] && kn < H);
      }
      load_x(kn, nx);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const Dec<FMT> ag = decode_step<FMT>(wg[rt], s);
        const Dec<FMT> au = decode_step<FMT>(wu[rt], s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < Planes<FMT>::n; ++p) {
            accg[mt][rt] = Op<FMT>::mfma(ag.p[p], xb[mt][s], accg[mt][rt]);
            accu[mt][rt] = Op<FMT>::mfma(au.p[p], xb[mt][s], accu[mt][rt]);
          }
      }
    }
    if (c + 1 < c1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        wg[rt] = ng[rt];
        wu[rt] = nu[rt];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[mt][s] = nx[mt][s];
    }
  }

  // cross-wave reduction of the K shares, one 16-token tile at a time, then SwiGLU
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();  // previous tile's reads of s_red are done
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_red[wave][rt][0][lane * 4 + i] = accg[mt][rt][i];
        s_red[wave][rt][1][lane * 4 + i] = accu[mt][rt][i];
      }
    __syncthreads();
    for (int o = threadIdx.x; o < RT * 256; o += NW * 64) {
      const int row = o & 15, tok = (o >> 4) & 15, rt = o >> 8;
      const int q = (16 * (row >> 2) + tok) * 4 + (row & 3);  // D layout: lane 16*(row/4)+tok, elem row%4
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        g += s_red[w][rt][0][q];
        u += s_red[w][rt][1][q];
      }
      g *= tensor_scale<FMT>(gate, ti.e);
      u *= tensor_scale<FMT>(up, ti.e);
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < I && m < ti.nr) {
        float h = (g / (1.0f + expf(-g))) * (u * u_scale);
        if (h_f16) h = (float)(_Float16)h;
        uint16_t hi, lo;
        Op<FMT>::split(h, hi, lo);
        const int64_t idx = (int64_t)(ti.r0 + m) * I + n;
        h_hi[idx] = hi;
        h_lo[idx] = lo;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// down:  y_slots[s, n] = sum_k Wd[e,n,k] (h_hi[r,k] + h_lo[r,k])
// ------------------------------------------------------------------------------------------------
// y16 (the range-managed path): when non-null, each output is rounded to binary16 and stored
// there instead of y_slots.
template <int FMT, int NW, int RT, int MT>
__global__ __launch_bounds__(NW * 64) void ffn_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    float* __restrict__ y_slots, uint16_t* __restrict__ y16) {
  typedef typename Op<FMT>::V V;
  __shared__ float s_red[NW][RT][256];
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16 * MT);
  if (ti.nr <= 0) return;
  // wave index in an SGPR: the K-share loop bounds are then wave-uniform (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;

  const uint16_t *hrow_hi[MT], *hrow_lo[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    tok_ok[mt] = m < ti.nr;
    const int64_t r = tok_ok[mt] ? ti.r0 + m : 0;
    hrow_hi[mt] = h_hi + r * I;
    hrow_lo[mt] = h_lo + r * I;
  }
  const uint8_t *drow[RT], *dsrow[RT], *dzrow[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + rt * 16 + l16;
    row_ok[rt] = n < H;
    const int nn = row_ok[rt] ? n : 0;
    drow[rt] = down.w + (int64_t)ti.e * down.we + (int64_t)nn * down.wr;
    dsrow[rt] = down.s ? down.s + (int64_t)ti.e * down.se + (int64_t)nn * down.sr : nullptr;
    dzrow[rt] = down.z ? down.z + (int64_t)ti.e * down.ze + (int64_t)nn * down.zr : nullptr;
  }

  const int n_chunks = (I + 127) >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);

  f32x4 acc[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  RawW<FMT> wd[RT];
  V bh[MT][4], bl[MT][4];
  auto load_h = [&](int k, V (&hi)[MT][4], V (&lo)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a = u32x4{0, 0, 0, 0}, b = u32x4{0, 0, 0, 0};
        if (tok_ok[mt] && k < I) {
          a = ld16(hrow_hi[mt] + k + 8 * s);
          b = ld16(hrow_lo[mt] + k + 8 * s);
        }
        hi[mt][s] = bitcast<V>(a);
        lo[mt][s] = bitcast<V>(b);
      }
  };
  if (c0 < c1) {
    const int k = c0 * 128 + 32 * lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wd[rt] = load_w<FMT>(drow[rt], dsrow[rt], dzrow[rt], k, row_ok[rt] && k < I);
    load_h(k, bh, bl);
  }
  for (int c = c0; c < c1; ++c) {
    const int k = c * 128 + 32 * lq;
    RawW<FMT> nd[RT];
    V nh[MT][4], nl[MT][4];
    if (c + 1 < c1) {
      const int kn = k + 128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) nd[rt] = load_w<FMT>(drow[rt], dsrow[rt], dzrow[rt], kn, row_ok[rt] && kn < I);
      load_h(kn, nh, nl);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const Dec<FMT> a = decode_step<FMT>(wd[rt], s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < Planes<FMT>::n; ++p) {
            acc[mt][rt] = Op<FMT>::mfma(a.p[p], bh[mt][s], acc[mt][rt]);
            acc[mt][rt] = Op<FMT>::mfma(a.p[p], bl[mt][s], acc[mt][rt]);
          }
      }
    }
    if (c + 1 < c1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wd[rt] = nd[rt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bh[mt][s] = nh[mt][s];
          bl[mt][s] = nl[mt][s];
        }
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[wave][rt][lane * 4 + i] = acc[mt][rt][i];
    __syncthreads();
    for (int o = threadIdx.x; o < RT * 256; o += NW * 64) {
      const int row = o & 15, tok = (o >> 4) & 15, rt = o >> 8;
      const int q = (16 * (row >> 2) + tok) * 4 + (row & 3);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_red[w][rt][q];
      v *= tensor_scale<FMT>(down, ti.e);
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < H && m < ti.nr) {
        const int s = sorted_slot[ti.r0 + m];
        if (s >= 0 && s < n_slots) {
          if (y16)
            y16[(int64_t)s * H + n] = bitcast<uint16_t>((_Float16)v);
          else
            y_slots[(int64_t)s * H + n] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Streaming variants for MXFP4 with 128-aligned K and 4-byte aligned scale rows (every workload
// shape).  Weights, activations and h are read with MUBUF buffer loads into registers, two chunks
// deep (ping-pong register sets, so no register copy forces an early wait); the loads go through
// buffer descriptors whose ranges bound every access.  Each wave keeps the scale bytes of its K
// share for the workgroup's 64 (matrix, row) pairs in a private LDS table filled once per work
// item with row-contiguous dword loads, instead of one scale load per row and chunk.
// ------------------------------------------------------------------------------------------------
// Two chunks in flight over the chunks [c0, c1) of a wave: register set A holds chunk c, B chunk
// c+1, and A is refilled with c+2 right after chunk c is consumed.  The steady-state loop issues
// its loads unconditionally (a load skipped on some path would make the compiler's vmcnt
// bookkeeping at the loop header fall back to waiting for everything); the last 1-3 chunks are
// peeled.  fill() (the wave's scale table) runs once the first two chunks' loads are out, so its
// own loads overlap them.
template <typename Chunk, typename Load, typename Compute, typename Fill>
__device__ __forceinline__ void run_pipeline_impl(int c0, int c1, Load& load, Compute& compute, Fill& fill) {
  if (c0 >= c1) return;
  Chunk A, B;
  load(c0, A);
  if (c1 - c0 == 1) {
    fill();
    compute(c0, A);
    return;
  }
  load(c0 + 1, B);
  fill();
  int c = c0;
  for (; c + 3 < c1; c += 2) {
    // scheduling barriers keep each refill right behind the compute that frees its registers
    compute(c, A);
    load(c + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(c + 1, B);
    load(c + 3, B);
    __builtin_amdgcn_sched_barrier(0);
  }
  compute(c, A);
  if (c + 2 < c1) load(c + 2, A);
  compute(c + 1, B);
  if (c + 2 < c1) compute(c + 2, A);
}

constexpr int kMaxChunksPerWave = 64;  // K share of one wave <= 8192
// Scale table of one wave: [pairs][cpw dwords]
__host__ __device__ constexpr int stab_bytes(int pairs, int cpw) { return pairs * cpw * 4; }
// Row stride (dwords) of the row-split kernels' scale tables: odd, so that the 16 rows a wave's
// lanes read at once fall on 16 different LDS banks (with n_chunks dwords per row, e.g. 16 or 56,
// they shared 2 or 4 banks, and each read waited on 8- or 4-way bank conflicts).
__host__ __device__ constexpr int rows_stab_stride(int n_chunks) { return n_chunks | 1; }

// Fills a wave's scale table: NM matrices of `total` units each; unit f of matrix m is read by
// ld(m, f) (which must read nothing for f >= total) and written by st(m, f, v).  PER units of every
// matrix are in flight per lane, all matrices together.  The first batch is straight-line code:
// in front of a loop that loads, the compiler waits for every load in flight, which would put the
// table's round trip behind that of the weight loads issued before it instead of beside it.
template <int NM, int PER, typename U, typename Ld, typename St>
__device__ __forceinline__ void fill_table(int total, int lane, const Ld& ld, const St& st) {
  auto batch = [&](int f0) {
    U v[NM][PER];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < PER; ++i) v[m][i] = ld(m, f0 + 64 * i + lane);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int f = f0 + 64 * i + lane;
        if (f < total) st(m, f, v[m][i]);
      }
  };
  batch(0);
  for (int f0 = 64 * PER; f0 < total; f0 += 64 * PER) batch(f0);
}

template <int NW, int MT, int RT>
__global__ __launch_bounds__(NW * 64) void ffn_gateup_stream_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int NM = 2, NP = NM * RT * 16;  // (matrix, row) pairs of the row block
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16 * MT);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;
  const int e = __builtin_amdgcn_readfirstlane(ti.e);

  // activations: rows of this lane's tokens.  Padded token lanes get an offset past the
  // descriptor's range: their loads are still issued (a uniform instruction count keeps the
  // compiler's vmcnt accounting exact) but return zeros without touching memory; their output
  // columns are never stored anyway.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  uint32_t xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    bool ok = m < ti.nr;
    const int sl = ok ? sorted_slot[ti.r0 + m] : -1;
    ok = ok && sl >= 0 && sl < n_slots;
    xoff[mt] = ok ? (uint32_t)(sl / k_total) * (uint32_t)H * 2u + 64u * lq : kOutOfRange;
  }
  const __amdgpu_buffer_rsrc_t wr[NM] = {make_rsrc(gate.w + (int64_t)e * gate.we, (int64_t)(I - 1) * gate.wr + H / 2),
                                         make_rsrc(up.w + (int64_t)e * up.we, (int64_t)(I - 1) * up.wr + H / 2)};
  const __amdgpu_buffer_rsrc_t sr[NM] = {make_rsrc(gate.s + (int64_t)e * gate.se, (int64_t)(I - 1) * gate.sr + H / 32),
                                         make_rsrc(up.s + (int64_t)e * up.se, (int64_t)(I - 1) * up.sr + H / 32)};
  uint32_t coff[NM][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min(n0 + rt * 16 + l16, I - 1);  // rows past I repeat the last row; never stored
    coff[0][rt] = (uint32_t)(n * gate.wr) + 16u * lq;
    coff[1][rt] = (uint32_t)(n * up.wr) + 16u * lq;
  }

  const int n_chunks = H >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + wave * stab_bytes(NP, cpw));

  // scale table: dword f = pair * cpw + j holds the scales of blocks 4*(c0+j) .. +3 of the pair's
  // row (pair = matrix * 16*RT + row); consecutive lanes read consecutive dwords of one row, 8
  // loads in flight per lane (4 of each matrix).
  auto fill = [&]() {
    const int total = 16 * RT * cpw;  // dwords per matrix
    fill_table<2, 4, uint32_t>(
        total, lane,
        [&](int m, int f) {
          const int r = f / cpw, j = f - r * cpw;
          const int n = min(n0 + r, I - 1), c = min(c0 + j, n_chunks - 1);
          return bld4(sr[m], f < total ? (uint32_t)(n * (m ? up.sr : gate.sr)) + 4u * c : kOutOfRange);
        },
        [&](int m, int f, uint32_t v) { stab[m * total + f] = v; });
  };

  f32x4 accg[MT][RT], accu[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      accg[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  struct Chunk {
    u32x4 q[NM][RT];
    V xb[MT][4];
  };
  auto load = [&](int c, Chunk& d) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) d.q[m][rt] = bld16(wr[m], coff[m][rt] + 64u * c);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) d.xb[mt][s] = bitcast<V>(bld16(xr, xoff[mt] + 256u * c + 16u * s));
  };
  auto compute = [&](int c, const Chunk& d) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * (c - c0) + lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float sg = e8m0_to_f32(sc[4 * cpw * (0 * 16 * RT + rt * 16 + l16)]);
      const float su = e8m0_to_f32(sc[4 * cpw * (1 * 16 * RT + rt * 16 + l16)]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const V ag = decode8_bf16(d.q[0][rt][s], sg), au = decode8_bf16(d.q[1][rt][s], su);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          accg[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, d.xb[mt][s], accg[mt][rt], 0, 0, 0);
          accu[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, d.xb[mt][s], accu[mt][rt], 0, 0, 0);
        }
      }
    }
  };
  run_pipeline_impl<Chunk>(c0, c1, load, compute, fill);

  // cross-wave reduction of the K shares, then SwiGLU
  float* red = reinterpret_cast<float*>(lds + NW * stab_bytes(NP, cpw));  // [NW][RT][2][256]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[((wave * RT + rt) * 2 + 0) * 256 + lane * 4 + i] = accg[mt][rt][i];
        red[((wave * RT + rt) * 2 + 1) * 256 + lane * 4 + i] = accu[mt][rt][i];
      }
    __syncthreads();
    for (int o = threadIdx.x; o < RT * 256; o += NW * 64) {
      const int row = o & 15, tok = (o >> 4) & 15, rt = o >> 8;
      const int q = (16 * (row >> 2) + tok) * 4 + (row & 3);
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        g += red[((w * RT + rt) * 2 + 0) * 256 + q];
        u += red[((w * RT + rt) * 2 + 1) * 256 + q];
      }
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < I && m < ti.nr) {
        const float h = (g / (1.0f + expf(-g))) * u;
        uint16_t hi, lo;
        Op<MOE_W_MXFP4>::split(h, hi, lo);
        const int64_t idx = (int64_t)(ti.r0 + m) * I + n;
        h_hi[idx] = hi;
        h_lo[idx] = lo;
      }
    }
  }
}

// FMT: MXFP4 (one 16-byte load of 32 codes per row and chunk, decoded with the block scale; K
// permuted within a chunk so that lane quarter lq holds values 32 lq .. + 31, as in the gate/up
// kernel) or FP16 (four 16-byte loads per row and chunk in the matrix core's own K order: k-step
// s, quarter lq takes values 32 s + 8 lq .. + 7, so one load covers 64 contiguous bytes of 16
// rows; no scales).  The h planes follow the same K order.
template <int FMT, int NW, int MT, int RT>
__global__ __launch_bounds__(NW * 64) void ffn_down_stream_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    float* __restrict__ y_slots) {
  constexpr int NP = RT * 16;  // rows of the row block
  constexpr bool MX = FMT == MOE_W_MXFP4;
  constexpr int WQ = MX ? 1 : 4;
  constexpr uint32_t kCW = MX ? 64u : 256u;
  constexpr uint32_t kHQ = MX ? 64u : 16u, kHS = MX ? 16u : 64u;
  typedef typename Op<FMT>::V V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16 * MT);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;
  const int ex = __builtin_amdgcn_readfirstlane(ti.e);

  const __amdgpu_buffer_rsrc_t hr_hi = make_rsrc(h_hi, (int64_t)n_slots * I * 2);
  const __amdgpu_buffer_rsrc_t hr_lo = make_rsrc(h_lo, (int64_t)n_slots * I * 2);
  uint32_t hoff[MT];  // padded token lanes: out-of-range offsets (see the gate/up kernel)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    hoff[mt] = m < ti.nr ? (uint32_t)(ti.r0 + m) * (uint32_t)I * 2u + kHQ * lq : kOutOfRange;
  }
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(down.w + (int64_t)ex * down.we, (int64_t)(H - 1) * down.wr + (MX ? I / 2 : (int64_t)I * 2));
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(MX ? down.s + (int64_t)ex * down.se : nullptr, MX ? (int64_t)(H - 1) * down.sr + I / 32 : 0);
  uint32_t coff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) coff[rt] = (uint32_t)(min(n0 + rt * 16 + l16, H - 1) * down.wr) + 16u * lq;

  const int n_chunks = I >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + wave * stab_bytes(NP, cpw));
  auto fill = [&]() {  // as in gate/up
    if constexpr (!MX) return;
    const int total = NP * cpw;
    fill_table<1, 8, uint32_t>(
        total, lane,
        [&](int, int f) {
          const int row = f / cpw, j = f - row * cpw, c = min(c0 + j, n_chunks - 1);
          return bld4(sr, f < total ? (uint32_t)(min(n0 + row, H - 1) * down.sr) + 4u * c : kOutOfRange);
        },
        [&](int, int f, uint32_t v) { stab[f] = v; });
  };

  f32x4 acc[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Chunk {
    u32x4 q[RT][WQ];
    V hi[MT][4], lo[MT][4];
  };
  auto load = [&](int c, Chunk& d) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int w = 0; w < WQ; ++w) d.q[rt][w] = bld16(wr, coff[rt] + kCW * c + 64u * w);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        d.hi[mt][s] = bitcast<V>(bld16(hr_hi, hoff[mt] + 256u * c + kHS * s));
        d.lo[mt][s] = bitcast<V>(bld16(hr_lo, hoff[mt] + 256u * c + kHS * s));
      }
  };
  auto compute = [&](int c, const Chunk& d) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * (c - c0) + lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float scale = 1.0f;
      if constexpr (MX) scale = e8m0_to_f32(sc[4 * cpw * (rt * 16 + l16)]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        V a;
        if constexpr (MX) a = decode8_bf16(d.q[rt][0][s], scale);
        else a = bitcast<V>(d.q[rt][s]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][rt] = Op<FMT>::mfma(a, d.hi[mt][s], acc[mt][rt]);
          acc[mt][rt] = Op<FMT>::mfma(a, d.lo[mt][s], acc[mt][rt]);
        }
      }
    }
  };
  run_pipeline_impl<Chunk>(c0, c1, load, compute, fill);

  float* red = reinterpret_cast<float*>(lds + NW * stab_bytes(NP, cpw));  // [NW][RT][256]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * RT + rt) * 256 + lane * 4 + i] = acc[mt][rt][i];
    __syncthreads();
    for (int o = threadIdx.x; o < RT * 256; o += NW * 64) {
      const int row = o & 15, tok = (o >> 4) & 15, rt = o >> 8;
      const int q = (16 * (row >> 2) + tok) * 4 + (row & 3);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[(w * RT + rt) * 256 + q];
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < H && m < ti.nr) {
        const int sl = sorted_slot[ti.r0 + m];
        if (sl >= 0 && sl < n_slots) y_slots[(int64_t)sl * H + n] = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Down for tiny calls (at most kTinyT tokens, so no tile has more rows than that): each wave owns
// 16 rows of H over the whole reduction dimension (no cross-wave sums) and issues its loads ahead
// of its MFMAs -- its share of the tile's h rows straight into LDS (buffer loads with the LDS
// destination, so they hold no registers), then its rows' block scales, then its weight chunks
// (all of them, or the first AHEAD pairs) -- so a wave waits for one memory round trip instead of
// one per pair of chunks.  The hi and lo planes of h are two sets of MFMA columns (token t in
// column t and kTinyT + t), one MFMA per weight operand, summed once at the end; columns past the
// tile's rows take zeros (those lanes read no LDS).
// ------------------------------------------------------------------------------------------------
constexpr int kTinyNC = 16, kTinyNW = 4;  // (kTinyT: launch.hpp)
typedef __attribute__((address_space(3))) void lds_void;

// AHEAD: chunk pairs of weight lines requested before the first MFMA, the next pair requested as
// each pair's first chunk starts (kTinyNC / 2: all at once).  A CU serves its load requests in
// order, so with every line requested at once the last workgroup on a CU receives all of its lines
// at the end and computes all of its chunks after them; requesting a few pairs ahead interleaves
// the workgroups' lines.  Measured, that paid for calls of one token (one row per tile) and was
// slower from two tokens on, which keep the one-shot form.
template <int AHEAD>
__global__ __launch_bounds__(kTinyNW * 64) void ffn_down_tiny_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    float* __restrict__ y_slots) {
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // [plane][kTinyT][I] bf16
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, kTinyT);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = (nblk * kTinyNW + wave) * 16;
  const int ex = __builtin_amdgcn_readfirstlane(ti.e);
  const int nc = I >> 7;  // chunks of 128 along I, at most kTinyNC

  // h rows of the tile: piece f of a plane (16 bytes) is column f % (I/8) of row f / (I/8); the
  // LDS copy holds them in that order, so each wave's load instruction fills 1 KB of LDS in lane
  // order.  Rows past the tile's (and pieces past the plane) read nothing.
  const int hp = I >> 3, per_plane = kTinyT * hp;
  const __amdgpu_buffer_rsrc_t hr[2] = {make_rsrc(h_hi, (int64_t)n_slots * I * 2), make_rsrc(h_lo, (int64_t)n_slots * I * 2)};
#pragma unroll
  for (int plane = 0; plane < 2; ++plane)
#pragma unroll
    for (int j = 0; j < kTinyT * kTinyNC * 16 / (kTinyNW * 64); ++j) {
      const int fw = 256 * j + 64 * wave;  // the wave's first piece (uniform)
      if (fw < per_plane) {
        const int f = fw + lane, t = f / hp, col = f - t * hp;
        const uint32_t off = t < ti.nr ? (uint32_t)(ti.r0 + t) * (uint32_t)I * 2u + 16u * col : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hr[plane], (lds_void*)(lds + plane * per_plane * 16 + 16 * fw), 16,
                                                 off, 0, 0, 0);
      }
    }

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(down.w + (int64_t)ex * down.we, (int64_t)(H - 1) * down.wr + I / 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(down.s + (int64_t)ex * down.se, (int64_t)(H - 1) * down.sr + I / 32);
  const int row = min(n0 + l16, H - 1);
  // the row's block scales, 16 bytes per load (scale rows 16-byte aligned, I / 32 a multiple of
  // 16): block 4c + lq of chunk c is byte lq of dword c
  u32x4 sv[kTinyNC / 4];
#pragma unroll
  for (int u = 0; u < kTinyNC / 4; ++u) sv[u] = bld16(sr, 16 * u < I / 32 ? (uint32_t)(row * down.sr) + 16u * u : kOutOfRange);
  // the weights as whole lines (nontemporal): load 2p + g covers rows n0 + 8g .. + 7 x the 128
  // bytes of chunks 2p and 2p + 1 (lane: row lr of the 8, piece lc; pieces 4-7 are the second
  // chunk); rows past H fall past the buffer's range and read zeros
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t lbase = (uint32_t)((n0 + lr) * down.wr) + 16u * lc;
  u32x4 q[kTinyNC];
  auto load_pair = [&](int p) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      q[2 * p + g] = bld16nt(wr, 2 * p + (lc >> 2) < nc ? lbase + (uint32_t)(8 * g * down.wr) + 128u * p : kOutOfRange);
  };
#pragma unroll
  for (int p = 0; p < AHEAD; ++p) load_pair(p);
  __syncthreads();  // the h pieces of every wave are in LDS
  // chunk c of the wave's 16 rows in MFMA layout (lane: row l16, the chunk's piece lq) through the
  // wave's 1 KB slot after the h copy, as in the row-split down kernel
  uint8_t* const tslot = lds + 2 * per_plane * 16 + wave * 1024;
  auto mfma_layout = [&](int c) -> u32x4 {
    const int p = c >> 1, j = c & 1;
    if ((lc >> 2) == j) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int w = 8 * g + lr;
        *reinterpret_cast<u32x4*>(tslot + 64 * w + 16 * ((lc & 3) ^ ((w >> 1) & 3))) = q[2 * p + g];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v = *reinterpret_cast<const u32x4*>(tslot + 64 * l16 + 16 * (lq ^ ((l16 >> 1) & 3)));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return v;
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  static_assert(2 * kTinyT <= 16, "hi and lo columns of every token in one MFMA");
  const int tcol = l16 < kTinyT ? l16 : l16 - kTinyT;  // token of this lane's column
  const bool tok = l16 < 2 * kTinyT && tcol < ti.nr;
  const uint8_t* hb = lds + (l16 < kTinyT ? 0 : per_plane * 16) + (tok ? tcol : 0) * I * 2 + 64 * lq;
  // B operand: lanes of the tile's rows load it, the other lanes keep what the registers hold
  // (their output columns are never stored)
  V b = V{};
#pragma unroll
  for (int c = 0; c < kTinyNC; ++c) {
    if (c < nc) {  // uniform
      if ((c & 1) == 0 && (c >> 1) + AHEAD < kTinyNC / 2) load_pair((c >> 1) + AHEAD);
      const float scale = e8m0_to_f32((sv[c >> 2][c & 3] >> (8 * lq)) & 0xFFu);
      const u32x4 w = mfma_layout(c);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        if (tok) b = *reinterpret_cast<const V*>(hb + 256 * c + 16 * s4);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(w[s4], scale), b, acc, 0, 0, 0);
      }
    }
  }
  // lane (column l16, quarter lq) holds rows n0 + 4 lq .. + 3 of its column; the lo column of
  // token t takes the hi column's sums (the lane kTinyT to its left in the same 16-lane row)
  static_assert(kTinyT == 4, "the DPP shift below moves columns by kTinyT");
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(dpp_u32<kDppRowShr4, 0xF>(0u, __float_as_uint(acc[i])));
  if (tok && l16 >= kTinyT) {
    const int sl = sorted_slot[ti.r0 + tcol];
    const int n = n0 + 4 * lq;
    if (sl >= 0 && sl < n_slots) {
      float* dst = y_slots + (int64_t)sl * H + n;
      if ((H & 3) == 0 && n + 3 < H) {
        *reinterpret_cast<f32x4*>(dst) = acc;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < H) dst[i] = acc[i];
      }
    }
  }
}

// Gate/up for the same tiny calls: the K-split streaming structure (four waves share a 16-row block
// of each of gate and up, each over a quarter of K, and meet in LDS for SwiGLU), with the whole of
// x -- at most kTinyT rows -- staged once in LDS by buffer loads with the LDS destination, and the
// weights kTinyDepth chunks deep in registers.  The streaming kernel's activation registers (four
// 16-byte loads per chunk) become LDS reads, which leaves room for the deeper weight pipeline.
constexpr int kTinyDepth = 4, kTinyGuT = 2;
// K share (chunks of 128) of one tiny gate/up wave: a quarter of K rounded up to whole pairs
__host__ __device__ constexpr int tiny_gateup_cpw(int H) { return ((H / 128 + kTinyNW - 1) / kTinyNW + 1) & ~1; }

__global__ __launch_bounds__(kTinyNW * 64) void ffn_gateup_tiny_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int NW = kTinyNW, D = kTinyDepth;
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // x [T][H] | scale tables | sums
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, kTinyT);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16;
  const int e = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = H >> 7, cpw = tiny_gateup_cpw(H);  // an even share: whole chunk pairs
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);

  // x: piece f (16 bytes) = token f / (H/8), column f % (H/8), at LDS byte 16 f; T * H / 8 is a
  // multiple of 64 (H % 512 == 0), so every load instruction fills 1 KB inside the x region
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  const int n_x = T * (H >> 3);
  for (int fw = 64 * wave; fw < n_x; fw += 64 * NW)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(lds + 16 * fw), 16, 16u * (uint32_t)(fw + lane), 0, 0, 0);

  const __amdgpu_buffer_rsrc_t wr[2] = {make_rsrc(gate.w + (int64_t)e * gate.we, (int64_t)(I - 1) * gate.wr + H / 2),
                                        make_rsrc(up.w + (int64_t)e * up.we, (int64_t)(I - 1) * up.wr + H / 2)};
  const __amdgpu_buffer_rsrc_t sr[2] = {make_rsrc(gate.s + (int64_t)e * gate.se, (int64_t)(I - 1) * gate.sr + H / 32),
                                        make_rsrc(up.s + (int64_t)e * up.se, (int64_t)(I - 1) * up.sr + H / 32)};
  // The weights as whole lines (nontemporal), a chunk pair per register set: load g of matrix m
  // covers rows n0 + 8g .. + 7 x the 128 bytes of chunks 2p and 2p + 1 (lane: row lr of the 8,
  // piece lc; pieces 4-7 are the second chunk).  Pieces past the wave's share, and rows past I
  // (past the buffer's range), read nothing.
  constexpr int DP = D / 2;  // chunk pairs in flight
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t lbase[2] = {(uint32_t)((n0 + lr) * gate.wr) + 16u * lc, (uint32_t)((n0 + lr) * up.wr) + 16u * lc};
  u32x4 q[DP][2][2];  // [set][matrix][8-row group]
  auto load = [&](int p, u32x4 (&d)[2][2]) {
    const bool in = 2 * p + (lc >> 2) < c1;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t wrm = m ? up.wr : gate.wr;
#pragma unroll
      for (int g = 0; g < 2; ++g) d[m][g] = bld16nt(wr[m], in ? lbase[m] + (uint32_t)(8 * g * wrm) + 128u * p : kOutOfRange);
    }
  };
  const int p0 = c0 >> 1, p1 = (c1 + 1) >> 1;
#pragma unroll
  for (int d = 0; d < DP; ++d) load(p0 + d, q[d]);

  // scale table of the wave's share: dword (m * 16 + r) * cpw + j holds the four block scales of
  // chunk c0 + j of row n0 + r of matrix m (gate, up)
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + (size_t)T * H * 2 + wave * stab_bytes(32, cpw));
  {
    const int total = 16 * cpw;
    fill_table<2, 4, uint32_t>(
        total, lane,
        [&](int m, int f) {
          const int r = f / cpw, j = f - r * cpw;
          const int n = min(n0 + r, I - 1), c = min(c0 + j, n_chunks - 1);
          return bld4(sr[m], f < total ? (uint32_t)(n * (m ? up.sr : gate.sr)) + 4u * c : kOutOfRange);
        },
        [&](int m, int f, uint32_t v) { stab[m * total + f] = v; });
  }
  // the token of this lane's MFMA column (a row of the tile), or -1 past the tile's rows
  int tok = -1;
  if (l16 < ti.nr) {
    const int sl = sorted_slot[ti.r0 + l16];
    if (sl >= 0 && sl < n_slots) tok = sl / k_total;
  }
  const uint8_t* xrow = lds + (size_t)(tok > 0 ? tok : 0) * H * 2 + 64 * lq;
  __syncthreads();  // x in LDS

  // chunk j of a matrix's 16 rows in MFMA layout (lane: row l16, the chunk's piece lq) through the
  // wave's 1 KB slot after the reduction area, as in the row-split down kernel
  uint8_t* const tslot = lds + (size_t)T * H * 2 + NW * stab_bytes(32, cpw) + NW * 2 * 256 * 4 + wave * 1024;
  auto mfma_layout = [&](const u32x4 (&dm)[2], int j) -> u32x4 {
    if ((lc >> 2) == j) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int w = 8 * g + lr;
        *reinterpret_cast<u32x4*>(tslot + 64 * w + 16 * ((lc & 3) ^ ((w >> 1) & 3))) = dm[g];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v = *reinterpret_cast<const u32x4*>(tslot + 64 * l16 + 16 * (lq ^ ((l16 >> 1) & 3)));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return v;
  };
  f32x4 accg = f32x4{0.f, 0.f, 0.f, 0.f}, accu = f32x4{0.f, 0.f, 0.f, 0.f};
  // B operand: lanes of the tile's rows load it, the others keep zeros (no refill per step)
  V b = V{};
  auto compute = [&](int c, const u32x4 (&d)[2][2]) {  // chunk c of the pair held in d
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * (c - c0) + lq;
    const float sg = e8m0_to_f32(sc[4 * cpw * l16]);
    const float su = e8m0_to_f32(sc[4 * cpw * (16 + l16)]);
    const u32x4 wg = mfma_layout(d[0], c & 1), wu = mfma_layout(d[1], c & 1);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (tok >= 0) b = *reinterpret_cast<const V*>(xrow + 256 * c + 16 * s4);
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(wg[s4], sg), b, accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(wu[s4], su), b, accu, 0, 0, 0);
    }
  };
  // ring of DP register sets: pair p in set (p - p0) % DP, refilled with pair p + DP once used
  for (int p = p0; p < p1; p += DP) {
#pragma unroll
    for (int d = 0; d < DP; ++d) {
      if (p + d < p1) {  // uniform
        compute(2 * (p + d), q[d]);
        if (2 * (p + d) + 1 < c1) compute(2 * (p + d) + 1, q[d]);
      }
      load(p + d + DP, q[d]);
    }
  }

  // cross-wave sums of the K shares, then SwiGLU
  float* red = reinterpret_cast<float*>(lds + (size_t)T * H * 2 + NW * stab_bytes(32, cpw));  // [NW][2][256]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[(wave * 2 + 0) * 256 + lane * 4 + i] = accg[i];
    red[(wave * 2 + 1) * 256 + lane * 4 + i] = accu[i];
  }
  __syncthreads();
  {
    const int o = threadIdx.x;  // one (row, token) per thread: 256 = 16 rows x 16 tokens
    const int rr = o & 15, tt = o >> 4;
    const int qq = (16 * (rr >> 2) + tt) * 4 + (rr & 3);
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      g += red[(w * 2 + 0) * 256 + qq];
      u += red[(w * 2 + 1) * 256 + qq];
    }
    const int n = n0 + rr;
    if (n < I && tt < ti.nr) {
      const float h = (g / (1.0f + expf(-g))) * u;
      uint16_t hi, lo;
      Op<MOE_W_MXFP4>::split(h, hi, lo);
      const int64_t idx = (int64_t)(ti.r0 + tt) * I + n;
      h_hi[idx] = hi;
      h_lo[idx] = lo;
    }
  }
}

// Gate/up of the K-split calls with one token tile (too few tiles for the row-split kernels, more
// tokens than the tiny kernel stages, e.g. 3 to about 10 tokens of the sweep layer): the tiny
// kernel's structure -- four waves share a 16-row block of each of gate and up, each over a
// quarter of K in whole chunk pairs, and meet in LDS for SwiGLU; weights as whole 128-byte lines
// with the nontemporal hint, turned into MFMA layout through a per-wave LDS slot -- with the
// tile's activations read per chunk pair from global memory (the tokens' rows stay in L2) into the
// same register ring as the weights, DP chunk pairs deep.  (Against the K-split kernel with
// half-line loads, side by side: sweep T = 4 180.5 -> 175.5 us, T = 8 265.2 -> 259.3 us.)
template <int DP>
__global__ __launch_bounds__(kTinyNW * 64) void ffn_gateup_split_lines_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int NW = kTinyNW;
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // scale tables | sums | slots
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16;
  const int e = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = H >> 7, cpw = tiny_gateup_cpw(H);  // an even share: whole chunk pairs
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);

  // the x row of this lane's MFMA column (a row of the tile), quarter lq of each chunk; columns
  // past the tile's rows take an offset past the descriptor's range (zeros, no memory access)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  uint32_t xoff = kOutOfRange;
  if (l16 < ti.nr) {
    const int sl = sorted_slot[ti.r0 + l16];
    if (sl >= 0 && sl < n_slots) xoff = (uint32_t)(sl / k_total) * (uint32_t)H * 2u + 64u * lq;
  }
  const __amdgpu_buffer_rsrc_t wr[2] = {make_rsrc(gate.w + (int64_t)e * gate.we, (int64_t)(I - 1) * gate.wr + H / 2),
                                        make_rsrc(up.w + (int64_t)e * up.we, (int64_t)(I - 1) * up.wr + H / 2)};
  const __amdgpu_buffer_rsrc_t sr[2] = {make_rsrc(gate.s + (int64_t)e * gate.se, (int64_t)(I - 1) * gate.sr + H / 32),
                                        make_rsrc(up.s + (int64_t)e * up.se, (int64_t)(I - 1) * up.sr + H / 32)};
  // load g of matrix m covers rows n0 + 8g .. + 7 x the 128 bytes of chunks 2p and 2p + 1 (lane:
  // row lr of the 8, piece lc; pieces 4-7 are the second chunk); pieces past the wave's share and
  // rows past I (past the buffer's range) read nothing
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t lbase[2] = {(uint32_t)((n0 + lr) * gate.wr) + 16u * lc, (uint32_t)((n0 + lr) * up.wr) + 16u * lc};
  u32x4 q[DP][2][2];   // [set][matrix][8-row group]
  u32x4 xq[DP][2][4];  // [set][chunk of the pair][k-step]
  auto load = [&](int p, u32x4 (&d)[2][2], u32x4 (&dx)[2][4]) {
    const bool in = 2 * p + (lc >> 2) < c1;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t wrm = m ? up.wr : gate.wr;
#pragma unroll
      for (int g = 0; g < 2; ++g) d[m][g] = bld16nt(wr[m], in ? lbase[m] + (uint32_t)(8 * g * wrm) + 128u * p : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 2 * p + j;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) dx[j][s4] = bld16(xr, c < c1 ? xoff + 256u * c + 16u * s4 : kOutOfRange);
    }
  };
  const int p0 = c0 >> 1, p1 = (c1 + 1) >> 1;
#pragma unroll
  for (int d = 0; d < DP; ++d) load(p0 + d, q[d], xq[d]);

  // scale table of the wave's share: dword (m * 16 + r) * cpw + j holds the four block scales of
  // chunk c0 + j of row n0 + r of matrix m (gate, up)
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + wave * stab_bytes(32, cpw));
  {
    const int total = 16 * cpw;
    fill_table<2, 4, uint32_t>(
        total, lane,
        [&](int m, int f) {
          const int r = f / cpw, j = f - r * cpw;
          const int n = min(n0 + r, I - 1), c = min(c0 + j, n_chunks - 1);
          return bld4(sr[m], f < total ? (uint32_t)(n * (m ? up.sr : gate.sr)) + 4u * c : kOutOfRange);
        },
        [&](int m, int f, uint32_t v) { stab[m * total + f] = v; });
  }

  // chunk j of a matrix's 16 rows in MFMA layout (lane: row l16, the chunk's piece lq) through the
  // wave's 1 KB slot after the reduction area
  uint8_t* const tslot = lds + NW * stab_bytes(32, cpw) + NW * 2 * 256 * 4 + wave * 1024;
  auto mfma_layout = [&](const u32x4 (&dm)[2], int j) -> u32x4 {
    if ((lc >> 2) == j) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int w = 8 * g + lr;
        *reinterpret_cast<u32x4*>(tslot + 64 * w + 16 * ((lc & 3) ^ ((w >> 1) & 3))) = dm[g];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v = *reinterpret_cast<const u32x4*>(tslot + 64 * l16 + 16 * (lq ^ ((l16 >> 1) & 3)));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return v;
  };
  f32x4 accg = f32x4{0.f, 0.f, 0.f, 0.f}, accu = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int c, const u32x4 (&d)[2][2], const u32x4 (&dx)[2][4]) {  // chunk c of the pair in d
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * (c - c0) + lq;
    const float sg = e8m0_to_f32(sc[4 * cpw * l16]);
    const float su = e8m0_to_f32(sc[4 * cpw * (16 + l16)]);
    const u32x4 wg = mfma_layout(d[0], c & 1), wu = mfma_layout(d[1], c & 1);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const V b = bitcast<V>(dx[c & 1][s4]);
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(wg[s4], sg), b, accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(wu[s4], su), b, accu, 0, 0, 0);
    }
  };
  // ring of DP register sets: pair p in set (p - p0) % DP, refilled with pair p + DP once used
  for (int p = p0; p < p1; p += DP) {
#pragma unroll
    for (int d = 0; d < DP; ++d) {
      if (p + d < p1) {  // uniform
        compute(2 * (p + d), q[d], xq[d]);
        if (2 * (p + d) + 1 < c1) compute(2 * (p + d) + 1, q[d], xq[d]);
      }
      load(p + d + DP, q[d], xq[d]);
    }
  }

  // cross-wave sums of the K shares, then SwiGLU
  float* red = reinterpret_cast<float*>(lds + NW * stab_bytes(32, cpw));  // [NW][2][256]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[(wave * 2 + 0) * 256 + lane * 4 + i] = accg[i];
    red[(wave * 2 + 1) * 256 + lane * 4 + i] = accu[i];
  }
  __syncthreads();
  {
    const int o = threadIdx.x;  // one (row, token) per thread: 256 = 16 rows x 16 tokens
    const int rr = o & 15, tt = o >> 4;
    const int qq = (16 * (rr >> 2) + tt) * 4 + (rr & 3);
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      g += red[(w * 2 + 0) * 256 + qq];
      u += red[(w * 2 + 1) * 256 + qq];
    }
    const int n = n0 + rr;
    if (n < I && tt < ti.nr) {
      const float h = (g / (1.0f + expf(-g))) * u;
      uint16_t hi, lo;
      Op<MOE_W_MXFP4>::split(h, hi, lo);
      const int64_t idx = (int64_t)(ti.r0 + tt) * I + n;
      h_hi[idx] = hi;
      h_lo[idx] = lo;
    }
  }
}
size_t gateup_split_lines_lds(int H) {  // scale tables, reduction, transposition slots
  return (size_t)kTinyNW * stab_bytes(32, tiny_gateup_cpw(H)) + (size_t)kTinyNW * 2 * 256 * 4 + (size_t)kTinyNW * 1024;
}
// One chunk pair in flight per wave: 100 registers and five waves per SIMD were faster than two
// pairs at 156 registers and three waves (side by side, sweep T = 4 182 -> 175 us, decode workload
// T = 8 136 -> 129 us, sweep T = 8 unchanged).
constexpr int kSplitLinesDP = 1;

// ------------------------------------------------------------------------------------------------
// Row-split streaming variants (many active experts).  The waves of a workgroup (4 or 8) own
// different weight rows, each over the whole reduction dimension, so no cross-wave reduction is
// needed; the activation (or h) chunk of the tile's tokens is shared: each wave loads a part of
// it into registers, writes it to an LDS stage, and every wave reads its MFMA operands from LDS.
// This cuts the L1 requests spent on activations 4-8x (the L1 request rate, more than HBM, bounds
// these kernels).  Each wave keeps the block scales of its rows over the whole reduction in an
// LDS table filled once: refilling a smaller table in windows re-fetches the partial 128-byte
// lines that straddle the windows (scale rows are 224 bytes for a 7168-wide matrix).
// ------------------------------------------------------------------------------------------------
constexpr int kRowsRT2 = 4;  // 16-row tiles per down wave (gate/up: one tile of each matrix)

// Gate/up: a step covers two 128-K chunks, i.e. a whole 128-byte line of every weight row, so the
// two halves of a line are requested together (one step apart, a line's second half was often
// evicted from L2 and fetched again).  The activation ring has two stages of two chunks; with the
// stage written right after the step's barrier, one barrier per step orders both the writes
// before their reads (next step) and the reads before the stage's rewrite (the step after).
constexpr int kGuXRow = 2 * 256 + 16;     // one token's two chunks of x + padding
constexpr int kGuXStage = 16 * kGuXRow;  // bytes of one stage

template <int NW, int RT>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 4 : 1) void ffn_gateup_rows_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int NM = 2, NP = NM * RT * 16;
  constexpr int XPT = 512 / (64 * NW);  // 16-byte lane-loads of x per thread per step
  static_assert(XPT * 64 * NW == 512 && (XPT == 1 || XPT == 2), "a step's x: 16 tokens x 2 chunks x 256 bytes");
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = (nblk * NW + wave) * 16 * RT;  // this wave's first row
  const int e = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = H >> 7, n_steps = (n_chunks + 1) >> 1;

  uint8_t* xs = lds;  // [2][kGuXStage]
  const int sstr = rows_stab_stride(n_chunks);
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + 2 * kGuXStage + wave * stab_bytes(NP, sstr));

  // Activations: thread q = 64*wave + lane moves 16-byte column q%16 of token q/16, both chunks of
  // a step (4 waves), or of token q/32, chunk (q/16)%2 (8 waves).  Padded tokens get an
  // out-of-range offset (reads zeros, no memory access).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  const int q = 64 * wave + lane;
  const int q_tok = XPT == 2 ? q >> 4 : q >> 5, q_col = q & 15, q_j = XPT == 2 ? 0 : (q >> 4) & 1;
  uint32_t xoff;
  {
    bool ok = q_tok < ti.nr;
    const int sl = ok ? sorted_slot[ti.r0 + q_tok] : -1;
    ok = ok && sl >= 0 && sl < n_slots;
    xoff = ok ? (uint32_t)(sl / k_total) * (uint32_t)H * 2u + 256u * q_j + 16u * q_col : kOutOfRange;
  }
  const uint32_t xs_w = (uint32_t)(q_tok * kGuXRow + 256 * q_j + 16 * q_col);  // + 256 * lane-load
  const uint32_t xs_r = (uint32_t)(l16 * kGuXRow + 64 * lq);        // + 256 * chunk + 16 * s

  const __amdgpu_buffer_rsrc_t wr[NM] = {make_rsrc(gate.w + (int64_t)e * gate.we, (int64_t)(I - 1) * gate.wr + H / 2),
                                         make_rsrc(up.w + (int64_t)e * up.we, (int64_t)(I - 1) * up.wr + H / 2)};
  const __amdgpu_buffer_rsrc_t sr[NM] = {make_rsrc(gate.s + (int64_t)e * gate.se, (int64_t)(I - 1) * gate.sr + H / 32),
                                         make_rsrc(up.s + (int64_t)e * up.se, (int64_t)(I - 1) * up.sr + H / 32)};
  // Weights come as whole lines: a load instruction covers 8 rows x the 128 bytes of a step (lane:
  // row lr of the 8, 16-byte piece lc; pieces 0-3 are the step's first chunk, 4-7 its second),
  // with the nontemporal hint.  Rows past I fall past the buffer's range and read zeros.  Each
  // 16-row tile is turned into MFMA layout through the wave's 512-byte LDS slot, 8 rows at a time.
  const int lr = lane >> 3, lc = lane & 7;
  const bool lsecond = lc >= 4;  // the lane's piece is in the step's second chunk
  const uint32_t lbase[NM] = {(uint32_t)((n0 + lr) * gate.wr) + 16u * lc, (uint32_t)((n0 + lr) * up.wr) + 16u * lc};
  uint8_t* const tslot = lds + 2 * kGuXStage + NW * stab_bytes(NP, sstr) + wave * 512;

  f32x4 accg[RT], accu[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    accg[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct Step {
    u32x4 q[NM][RT][2];  // [matrix][row tile][8-row group]: whole lines of the step
  };
  // (a piece of a missing second chunk of the last step reads nothing)
  auto load = [&](int s, Step& d) {
    const bool in = 2 * s + (lsecond ? 1 : 0) < n_chunks;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int64_t wrm = m ? up.wr : gate.wr;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int g = 0; g < 2; ++g)
          d.q[m][rt][g] = bld16nt(wr[m], in ? lbase[m] + (uint32_t)((16 * rt + 8 * g) * wrm) + 128u * s : kOutOfRange);
    }
  };
  // chunk j of row tile rt of matrix m in MFMA layout (lane: row l16, the chunk's piece lq), in two
  // rounds through the 512-byte slot: round g holds rows 8g .. 8g + 7 (piece c of slot row w at
  // 64 w + 16 (c ^ ((w >> 1) & 3))), which the lanes of those rows read.  Lanes read what other
  // lanes wrote: wavefront-scope fences and wave barriers keep the compiler's order (a wave's LDS
  // operations run in order).
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto mfma_layout = [&](const Step& d, int m, int rt, int j) -> u32x4 {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (lsecond == (j == 1))
        *reinterpret_cast<u32x4*>(tslot + 64 * lr + 16 * ((lc & 3) ^ ((lr >> 1) & 3))) = d.q[m][rt][g];
      wave_sync();
      if ((l16 >> 3) == g) {
        const int w = l16 & 7;
        v = *reinterpret_cast<const u32x4*>(tslot + 64 * w + 16 * (lq ^ ((w >> 1) & 3)));
      }
      wave_sync();
    }
    return v;
  };
  // Activations are fetched two steps ahead, like the weights: X[s % 2] holds step s's chunks
  // until they are written to their stage, then is refilled with step s + 2's.
  u32x4 X[2][XPT];
  auto fetch_x = [&](int s, u32x4 (&r)[XPT]) {
#pragma unroll
    for (int j = 0; j < XPT; ++j)
      r[j] = bld16(xr, 2 * s + q_j + j < n_chunks ? xoff + 512u * s + 256u * j : kOutOfRange);
  };
  auto put_x = [&](int s, const u32x4 (&r)[XPT]) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) *reinterpret_cast<u32x4*>(xs + (s & 1) * kGuXStage + xs_w + 256 * j) = r[j];
  };
  auto compute_chunk = [&](int s, int j, const Step& d) {
    const int c = 2 * s + j;
    const uint8_t* xst = xs + (s & 1) * kGuXStage + xs_r + 256 * j;
    V xb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xb[k] = *reinterpret_cast<const V*>(xst + 16 * k);
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * c + lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float sg = e8m0_to_f32(sc[4 * sstr * (0 * 16 * RT + rt * 16 + l16)]);
      const float su = e8m0_to_f32(sc[4 * sstr * (1 * 16 * RT + rt * 16 + l16)]);
      {
        const u32x4 w = mfma_layout(d, 0, rt, j);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          accg[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(w[k], sg), xb[k], accg[rt], 0, 0, 0);
      }
      {
        const u32x4 w = mfma_layout(d, 1, rt, j);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          accu[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8_bf16(w[k], su), xb[k], accu[rt], 0, 0, 0);
      }
    }
  };
  // Step s: sync, publish step s+1's activations (held in Xn), compute step s from register set D,
  // refill D with step s+2's weights and Xn with step s+3's activations.  Every step issues its
  // loads in one order (the weights, then the activations), so the wait counts the compiler derives
  // at the loop head are the steady ones.
  auto step = [&](int s, Step& D, u32x4 (&Xn)[XPT]) {
    __syncthreads();
    put_x(s + 1, Xn);
    compute_chunk(s, 0, D);
    compute_chunk(s, 1, D);
    load(s + 2, D);
    __builtin_amdgcn_sched_barrier(0);  // keep the load order fixed
    fetch_x(s + 3, Xn);
  };
  Step A, B;
  // The first two steps' weights go out before their activations, whose offsets wait for the
  // sorted-slot read (measured: T = 176 668 -> 663 us, T = 32 436 -> 432 us).
  load(0, A);
  __builtin_amdgcn_sched_barrier(0);
  load(n_steps > 1 ? 1 : 0, B);
  __builtin_amdgcn_sched_barrier(0);
  fetch_x(0, X[0]);
  __builtin_amdgcn_sched_barrier(0);
  fetch_x(1, X[1]);
  __builtin_amdgcn_sched_barrier(0);
  // The scale table is filled while the first steps' loads are in flight: one memory round trip
  // before the first MFMA instead of two.
  // Scale table [pair][n_chunks] dwords (a dword: the four block scales of one row in one chunk),
  // pair = m * 16 * RT + row offset; read in 16-byte units when rows allow it.
  {
    const int rows = 16 * RT;
    auto vec_ok = [&](const ProjDev& p) {
      return (n_chunks & 3) == 0 && (p.sr & 15) == 0 && ((uintptr_t)(p.s + (int64_t)e * p.se) & 15) == 0;
    };
    if (vec_ok(gate) && vec_ok(up)) {
      const int upr = n_chunks >> 2, total = rows * upr;
      fill_table<NM, 4, u32x4>(
          total, lane,
          [&](int m, int f) {
            const int r = f / upr, u = f - r * upr;
            return bld16(sr[m], f < total ? (uint32_t)(min(n0 + r, I - 1) * (m ? up.sr : gate.sr)) + 16u * u : kOutOfRange);
          },
          [&](int m, int f, const u32x4& v) {
            const int r = f / upr, u = f - r * upr;
            uint32_t* d = stab + (m * rows + r) * sstr + 4 * u;
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = v[i];
          });
    } else {
      const int total = rows * n_chunks;
      fill_table<NM, 4, uint32_t>(
          total, lane,
          [&](int m, int f) {
            const int r = f / n_chunks, j = f - r * n_chunks;
            return bld4(sr[m], f < total ? (uint32_t)(min(n0 + r, I - 1) * (m ? up.sr : gate.sr)) + 4u * j : kOutOfRange);
          },
          [&](int m, int f, uint32_t v) {
            const int r = f / n_chunks, j = f - r * n_chunks;
            stab[(m * rows + r) * sstr + j] = v;
          });
    }
  }
  put_x(0, X[0]);
  fetch_x(2, X[0]);
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;  // even: step s's weights in A, step s+1's in B
  for (; s + 3 < n_steps; s += 2) {
    step(s, A, X[1]);
    __builtin_amdgcn_sched_barrier(0);
    step(s + 1, B, X[0]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // last 1-3 steps: no loads past the end
  __syncthreads();
  if (s + 1 < n_steps) put_x(s + 1, X[1]);
  compute_chunk(s, 0, A);
  if (2 * s + 1 < n_chunks) compute_chunk(s, 1, A);
  if (s + 2 < n_steps) load(s + 2, A);
  if (s + 1 < n_steps) {
    __syncthreads();
    if (s + 2 < n_steps) put_x(s + 2, X[0]);
    compute_chunk(s + 1, 0, B);
    if (2 * s + 3 < n_chunks) compute_chunk(s + 1, 1, B);
  }
  if (s + 2 < n_steps) {
    __syncthreads();
    compute_chunk(s + 2, 0, A);
    if (2 * s + 5 < n_chunks) compute_chunk(s + 2, 1, A);
  }

  // SwiGLU on the wave's own rows: lane holds rows n0 + rt*16 + 4*lq + i of token l16
  const int m = l16;
  if (m < ti.nr) {
    const int64_t base = (int64_t)(ti.r0 + m) * I;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
    {  // four consecutive h values of one token: one 8-byte store per plane
      const int nb = n0 + rt * 16 + 4 * lq;
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = accg[rt][i], u = accu[rt][i];
        const float h = (g / (1.0f + expf(-g))) * u;
        uint16_t hi, lo;
        Op<MOE_W_MXFP4>::split(h, hi, lo);
        if (i & 1) { ph[i >> 1] |= (uint32_t)hi << 16; pl[i >> 1] |= (uint32_t)lo << 16; }
        else { ph[i >> 1] = hi; pl[i >> 1] = lo; }
      }
      if ((I & 3) == 0 && nb + 3 < I) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2*>(h_hi + base + nb) = u32x2{ph[0], ph[1]};
        *reinterpret_cast<u32x2*>(h_lo + base + nb) = u32x2{pl[0], pl[1]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < I) {
            h_hi[base + nb + i] = (uint16_t)(ph[i >> 1] >> (16 * (i & 1)));
            h_lo[base + nb + i] = (uint16_t)(pl[i >> 1] >> (16 * (i & 1)));
          }
      }
    }
  }
}

// Down: whole lines per step.  A step covers two 128-K chunks -- one whole 128-byte line of every
// weight row -- for half of the wave's row tiles, and the next step the same two chunks for the
// other half, so both halves of a line are requested by one pair of loads.  (With one chunk of all
// the row tiles per step, the half-read lines of a workgroup's rows stayed open for a whole step,
// more of them than an XCD's L2 holds, and about 9% of the lines were fetched twice.)  A step's
// weights are four 16-byte loads per lane.  The h ring (two stages, written after the barrier as
// in gate/up) advances every two steps: a stage holds the hi and lo planes of both chunks of a
// pair of steps, with one barrier per pair.  The scale table covers the whole K.
struct DnStage {
  static constexpr int kRow = 2 * 256 + 16;    // one token's two chunks of one h plane + padding
  static constexpr int kBytes = 2 * 16 * kRow;  // hi plane, then lo plane
};

template <int NW>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 4 : 1) void ffn_down_lines_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    float* __restrict__ y_slots) {
  constexpr int RT = kRowsRT2, HT = RT / 2, NP = RT * 16;
  constexpr int LPT = 1024 / (64 * NW);  // 16-byte lane-loads of h per thread per pair
  static_assert(LPT * 64 * NW == 1024, "a pair's h: 2 planes x 16 tokens x 2 chunks x 256 bytes");
  static_assert(RT % 2 == 0, "two halves of the row tiles");
  constexpr int kRow = DnStage::kRow, kStage = DnStage::kBytes;
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, 16);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = (nblk * NW + wave) * 16 * RT;
  const int ex = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = I >> 7, n_pairs = (n_chunks + 1) >> 1;

  uint8_t* xs = lds;  // [2][kStage]
  const int sstr = rows_stab_stride(n_chunks);
  uint32_t* stab = reinterpret_cast<uint32_t*>(lds + 2 * kStage + wave * stab_bytes(NP, sstr));

  // h lane-load i: q = 64 * (NW * i + wave) + lane covers 16-byte column q % 16 of chunk (q / 16) % 2
  // of the pair, token (q / 32) % 16 and plane q / 512 (uniform over a wave's load).
  const __amdgpu_buffer_rsrc_t hr[2] = {make_rsrc(h_hi, (int64_t)n_slots * I * 2), make_rsrc(h_lo, (int64_t)n_slots * I * 2)};
  uint32_t hoff[LPT], hs_w[LPT];
  int hplane[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int q = 64 * (NW * i + wave) + lane;
    const int plane = q >> 9, tok = (q >> 5) & 15, j = (q >> 4) & 1, col = q & 15;
    hplane[i] = __builtin_amdgcn_readfirstlane(plane);
    hoff[i] = tok < ti.nr ? (uint32_t)(ti.r0 + tok) * (uint32_t)I * 2u + 256u * j + 16u * col : kOutOfRange;
    hs_w[i] = (uint32_t)(plane * 16 * kRow + tok * kRow + 256 * j + 16 * col);
  }
  const int hj = (lane >> 4) & 1;  // the chunk of the pair that this lane's h loads cover
  const uint32_t hs_r = (uint32_t)(l16 * kRow + 64 * lq);  // + 256 * chunk + 16 * k (+ lo plane)

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(down.w + (int64_t)ex * down.we, (int64_t)(H - 1) * down.wr + I / 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(down.s + (int64_t)ex * down.se, (int64_t)(H - 1) * down.sr + I / 32);
  // Weights come as whole lines: a load instruction covers 8 rows x the 128 bytes of a pair (lane:
  // row lr of the 8, 16-byte piece lc; pieces 0-3 are the pair's first chunk, 4-7 its second), with
  // the nontemporal hint.  Rows past H fall past the buffer's range and read zeros.  Each row tile
  // is turned into MFMA layout through the wave's 1 KB LDS slot, one chunk at a time.
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t lbase = (uint32_t)((n0 + lr) * down.wr) + 16u * lc;
  const bool lsecond = lc >= 4;  // the lane's piece is in the pair's second chunk
  uint8_t* const tslot = lds + 2 * kStage + NW * stab_bytes(NP, rows_stab_stride(n_chunks)) + wave * 1024;
  f32x4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Half {
    u32x4 q[HT][2];  // [row tile of the half][8-row group]: whole lines of the pair
  };
  // pair p, half th: row tiles HT * th .. HT * th + HT - 1, chunks 2p and 2p + 1 (a piece of a
  // missing second chunk reads nothing)
  auto load = [&](int p, int th, Half& d) {
    const bool in = 2 * p + (lsecond ? 1 : 0) < n_chunks;
#pragma unroll
    for (int r = 0; r < HT; ++r)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        d.q[r][g] = bld16nt(wr, in ? lbase + (uint32_t)((16 * (HT * th + r) + 8 * g) * down.wr) + 128u * p
                                   : kOutOfRange);
  };
  // chunk j of row tile r of d in MFMA layout (lane: row l16, the chunk's 16-byte piece lq),
  // through the wave's slot (piece c of slot row w at 64 w + 16 (c ^ ((w >> 1) & 3)): the 8 rows
  // a read pass touches sit on distinct banks).  A lane reads what other lanes of its wave wrote:
  // wavefront-scope fences and wave barriers keep the compiler from moving the read above the
  // writes or the next writes above the read (a wave's LDS operations run in order, so no wait
  // is needed in hardware).
  auto mfma_layout = [&](const Half& d, int r, int j) -> u32x4 {
    if (lsecond == (j == 1)) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int w = 8 * g + lr;
        *reinterpret_cast<u32x4*>(tslot + 64 * w + 16 * ((lc & 3) ^ ((w >> 1) & 3))) = d.q[r][g];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v = *reinterpret_cast<const u32x4*>(tslot + 64 * l16 + 16 * (lq ^ ((l16 >> 1) & 3)));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return v;
  };
  auto fetch_h = [&](int p, u32x4 (&r)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) r[i] = bld16(hr[hplane[i]], 2 * p + hj < n_chunks ? hoff[i] + 512u * p : kOutOfRange);
  };
  auto put_h = [&](int p, const u32x4 (&r)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<u32x4*>(xs + (p & 1) * kStage + hs_w[i]) = r[i];
  };
  // tail: the pair may be the last one, whose second chunk is missing for an odd chunk count
  auto compute = [&](int p, int th, const Half& d, bool tail) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j == 1 && tail && 2 * p + 1 >= n_chunks) break;
      const int c = 2 * p + j;
      const uint8_t* st = xs + (p & 1) * kStage + hs_r + 256 * j;
      const uint8_t* sc = reinterpret_cast<const uint8_t*>(stab) + 4 * c + lq;
      float scale[HT];
#pragma unroll
      for (int r = 0; r < HT; ++r) scale[r] = e8m0_to_f32(sc[4 * sstr * ((HT * th + r) * 16 + l16)]);
      u32x4 w[HT];
#pragma unroll
      for (int r = 0; r < HT; ++r) w[r] = mfma_layout(d, r, j);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const V bh = *reinterpret_cast<const V*>(st + 16 * k);
        const V bl = *reinterpret_cast<const V*>(st + 16 * kRow + 16 * k);
#pragma unroll
        for (int r = 0; r < HT; ++r) {
          const V a = decode8_bf16(w[r][k], scale[r]);
          acc[HT * th + r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[HT * th + r], 0, 0, 0);
          acc[HT * th + r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[HT * th + r], 0, 0, 0);
        }
      }
    }
  };
  // Pair p: sync, publish pair p+1's h (held in Hn), compute both halves of pair p, each followed by
  // the load of the same half of pair p+1 into its registers, then fetch pair p+3's h into Hn.  The
  // prologue issues its loads in the same order.
  auto pair = [&](int p, Half& A, Half& B, u32x4 (&Hn)[LPT]) {
    __syncthreads();
    put_h(p + 1, Hn);
    compute(p, 0, A, false);
    load(p + 1, 0, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(p, 1, B, false);
    load(p + 1, 1, B);
    __builtin_amdgcn_sched_barrier(0);
    fetch_h(p + 3, Hn);
  };
  Half A, B;
  u32x4 Hc[2][LPT];
  fetch_h(0, Hc[0]);
  __builtin_amdgcn_sched_barrier(0);
  load(0, 0, A);
  __builtin_amdgcn_sched_barrier(0);
  fetch_h(1, Hc[1]);
  __builtin_amdgcn_sched_barrier(0);
  load(0, 1, B);
  __builtin_amdgcn_sched_barrier(0);
  // scale table [row][n_chunks] dwords, filled while the first pair's loads are in flight, in
  // 16-byte units when rows allow it
  {
    const bool vec = (n_chunks & 3) == 0 && (down.sr & 15) == 0 &&
                     ((uintptr_t)(down.s + (int64_t)ex * down.se) & 15) == 0;
    if (vec) {
      const int upr = n_chunks >> 2, total = NP * upr;
      fill_table<1, 4, u32x4>(
          total, lane,
          [&](int, int f) {
            const int r = f / upr, u = f - r * upr;
            return bld16(sr, f < total ? (uint32_t)(min(n0 + r, H - 1) * down.sr) + 16u * u : kOutOfRange);
          },
          [&](int, int f, const u32x4& v) {
            const int r = f / upr, u = f - r * upr;
            uint32_t* d = stab + r * sstr + 4 * u;
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = v[i];
          });
    } else {
      const int total = NP * n_chunks;
      fill_table<1, 8, uint32_t>(
          total, lane,
          [&](int, int f) {
            const int r = f / n_chunks, j = f - r * n_chunks;
            return bld4(sr, f < total ? (uint32_t)(min(n0 + r, H - 1) * down.sr) + 4u * j : kOutOfRange);
          },
          [&](int, int f, uint32_t v) {
            const int r = f / n_chunks, j = f - r * n_chunks;
            stab[r * sstr + j] = v;
          });
    }
  }
  put_h(0, Hc[0]);
  fetch_h(2, Hc[0]);
  __builtin_amdgcn_sched_barrier(0);
  int p = 0;  // even: Hc[1] holds pair p+1's h, Hc[0] pair p+2's
  for (; p + 3 < n_pairs; p += 2) {
    pair(p, A, B, Hc[1]);
    __builtin_amdgcn_sched_barrier(0);
    pair(p + 1, A, B, Hc[0]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // last 1-3 pairs: no loads past the end
  __syncthreads();
  if (p + 1 < n_pairs) put_h(p + 1, Hc[1]);
  compute(p, 0, A, true);
  if (p + 1 < n_pairs) load(p + 1, 0, A);
  compute(p, 1, B, true);
  if (p + 1 < n_pairs) {
    load(p + 1, 1, B);
    __syncthreads();
    if (p + 2 < n_pairs) put_h(p + 2, Hc[0]);
    compute(p + 1, 0, A, true);
    if (p + 2 < n_pairs) load(p + 2, 0, A);
    compute(p + 1, 1, B, true);
    if (p + 2 < n_pairs) load(p + 2, 1, B);
  }
  if (p + 2 < n_pairs) {
    __syncthreads();
    compute(p + 2, 0, A, true);
    compute(p + 2, 1, B, true);
  }

  const int m = l16;
  if (m < ti.nr) {
    const int sl = sorted_slot[ti.r0 + m];
    if (sl >= 0 && sl < n_slots) {
      float* dst = y_slots + (int64_t)sl * H;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int n = n0 + rt * 16 + 4 * lq;
        if ((H & 3) == 0 && n + 3 < H) {
          // streaming stores: y_slots is read by the next call, not by this kernel, and keeping it
          // out of L2 shortens the end-of-kernel write-back (T = 176: 378 -> 374 us)
          __builtin_nontemporal_store(acc[rt], reinterpret_cast<f32x4*>(dst + n));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < H) dst[n + i] = acc[rt][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Tile kernels for calls with many rows per expert (prefill, or FP16 slices with many tokens):
// 128-token tiles.  A gate/up wave decodes its 16 rows of each matrix once per chunk and applies
// them to all eight 16-token sub-tiles (a down wave: 32 rows, a 64-token half of a tile), so the
// work is MFMA-bound rather than decode- or HBM-bound.  The tile's activations (or h) go through a
// two-stage LDS ring, written right after each step's barrier.  MXFP4 block scales are loaded with
// the weights (one dword per row and chunk); FP16 weights are four 16-byte loads per row and chunk.  Workgroups are numbered tile-major with the row blocks
// padded to a multiple of 8, so row block j of every tile runs on XCD j % 8: the tiles of a hot
// expert that run together read each weight row from one L2.  Gate/up computes sub-tiles past the
// tile's rows on zero activations (branching around their MFMAs split its scheduled loop and was
// slower); the down kernel skips them.
// ------------------------------------------------------------------------------------------------
constexpr int kTileMT = 8;                     // 16-token sub-tiles per gate/up tile
constexpr int kTileRT = 1;                     // 16-row tiles of each matrix per gate/up wave
constexpr int kDnTileMT = 4;                   // 16-token sub-tiles per down work item (half a tile)
constexpr int kTileRow = 128 * 2 + 16;         // LDS bytes per token row of one plane of a stage

// Weights of one lane for one 16-row tile in one 128-K chunk, as the tile kernels load them: the
// 16-byte MXFP4 block plus the row's four block scales of the chunk (byte lq is the lane's), or
// 4 x 16 bytes of fp16 (the lane's 32 consecutive K values).
template <int FMT>
struct TileW;
template <>
struct TileW<MOE_W_MXFP4> {
  u32x4 q;
  uint32_t sc;
  static constexpr uint32_t kLaneBytes = 16;  // per lane-quarter of a row, per chunk
};
template <>
struct TileW<MOE_W_FP16> {
  u32x4 q[4];
  static constexpr uint32_t kLaneBytes = 64;
};
template <int FMT>
__device__ __forceinline__ void tile_load(TileW<FMT>& d, __amdgpu_buffer_rsrc_t w, __amdgpu_buffer_rsrc_t s,
                                          uint32_t coff, uint32_t soff, int c) {
  if constexpr (FMT == MOE_W_MXFP4) {
    d.q = bld16(w, coff + 64u * c);
    d.sc = bld4(s, soff + 4u * c);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) d.q[k] = bld16(w, coff + 256u * c + 16u * k);
  }
}
// k-th MFMA operand (K values 32*lq + 8k .. +7 of the chunk); scale = the lane's block scale
template <int FMT>
__device__ __forceinline__ typename Op<FMT>::V tile_operand(const TileW<FMT>& d, int k, float scale) {
  if constexpr (FMT == MOE_W_MXFP4) return decode8_bf16(d.q[k], scale);
  else return bitcast<f16x8>(d.q[k]);
}
template <int FMT>
__device__ __forceinline__ float tile_scale(const TileW<FMT>& d, int lq) {
  if constexpr (FMT == MOE_W_MXFP4) return e8m0_to_f32((d.sc >> (8 * lq)) & 255u);
  else return 1.0f;
}
// Buffer descriptors of one expert's weight matrix (rows x K) and its scale grid (MXFP4 only).
template <int FMT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_wrsrc(const ProjDev& p, int e, int rows, int K) {
  return make_rsrc(p.w + (int64_t)e * p.we, (int64_t)(rows - 1) * p.wr + (FMT == MOE_W_MXFP4 ? K / 2 : 2 * K));
}
template <int FMT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_srsrc(const ProjDev& p, int e, int rows, int K) {
  return FMT == MOE_W_MXFP4 ? make_rsrc(p.s + (int64_t)e * p.se, (int64_t)(rows - 1) * p.sr + K / 32)
                            : make_rsrc(p.w, 0);
}

template <int FMT, int NW, int RT, int MT>
__global__ __launch_bounds__(NW * 64, FMT == MOE_W_MXFP4 ? 2 : 1) void ffn_gateup_tile_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    int n_nblk_pad, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int NM = 2, NTOK = 16 * MT;
  constexpr int kStage = NTOK * kTileRow;
  constexpr int LPT = NTOK * 16 / (64 * NW);  // 16-byte lane-loads of x per thread per chunk
  static_assert(LPT * 64 * NW == NTOK * 16, "a chunk of x over the workgroup");
  typedef typename Op<FMT>::V V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_slots = T * k_total;
  const int tile = blockIdx.x / n_nblk_pad, nblk = blockIdx.x - tile * n_nblk_pad;
  if (nblk >= n_nblk) return;
  const TileInfo ti = get_tile(tiles, tile, n_experts, n_slots, NTOK);
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = (nblk * NW + wave) * 16 * RT;
  const int e = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = H >> 7;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  uint32_t xoff[LPT], xs_w[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int q = threadIdx.x + 64 * NW * i, tok = q >> 4, col = q & 15;
    bool ok = tok < ti.nr;
    const int sl = ok ? sorted_slot[ti.r0 + tok] : -1;
    ok = ok && sl >= 0 && sl < n_slots;
    xoff[i] = ok ? (uint32_t)(sl / k_total) * (uint32_t)H * 2u + 16u * col : kOutOfRange;
    xs_w[i] = (uint32_t)(tok * kTileRow + 16 * col);
  }
  const uint32_t xs_r = (uint32_t)(l16 * kTileRow + 64 * lq);

  const __amdgpu_buffer_rsrc_t wr[NM] = {tile_wrsrc<FMT>(gate, e, I, H), tile_wrsrc<FMT>(up, e, I, H)};
  const __amdgpu_buffer_rsrc_t sr[NM] = {tile_srsrc<FMT>(gate, e, I, H), tile_srsrc<FMT>(up, e, I, H)};
  uint32_t coff[NM][RT], soff[NM][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min(n0 + rt * 16 + l16, I - 1);
    coff[0][rt] = (uint32_t)(n * gate.wr) + TileW<FMT>::kLaneBytes * lq;
    coff[1][rt] = (uint32_t)(n * up.wr) + TileW<FMT>::kLaneBytes * lq;
    soff[0][rt] = (uint32_t)(n * gate.sr);
    soff[1][rt] = (uint32_t)(n * up.sr);
  }

  f32x4 accg[RT][MT], accu[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accg[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  struct Step {
    TileW<FMT> w[NM][RT];
  };
  auto load = [&](int c, Step& d) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) tile_load<FMT>(d.w[m][rt], wr[m], sr[m], coff[m][rt], soff[m][rt], c);
  };
  // x is fetched one chunk ahead (the next chunk's piece of this thread)
  u32x4 Xr[LPT];
  auto fetch_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) Xr[i] = bld16(xr, c < n_chunks ? xoff[i] + 256u * c : kOutOfRange);
  };
  auto put_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<u32x4*>(lds + (c & 1) * kStage + xs_w[i]) = Xr[i];
  };
  auto compute = [&](int c, const Step& d) {
    const uint8_t* st = lds + (c & 1) * kStage + xs_r;
    float scl[NM][RT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) scl[m][rt] = tile_scale<FMT>(d.w[m][rt], lq);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      V ag[RT], au[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        ag[rt] = tile_operand<FMT>(d.w[0][rt], k, scl[0][rt]);
        au[rt] = tile_operand<FMT>(d.w[1][rt], k, scl[1][rt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const V xb = *reinterpret_cast<const V*>(st + mt * 16 * kTileRow + 16 * k);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          accg[rt][mt] = Op<FMT>::mfma(ag[rt], xb, accg[rt][mt]);
          accu[rt][mt] = Op<FMT>::mfma(au[rt], xb, accu[rt][mt]);
        }
      }
    }
  };
  // Weights three chunks deep (register sets A, B, C; two waves per SIMD for MXFP4 needs the
  // register cap in the launch bounds), activations one chunk ahead.  Measured on the prefill
  // layer: 6.0 -> 5.66 ms; the same for the down kernel gave nothing and cost FP16 occupancy.
  auto step = [&](int c, Step& D) {  // D holds chunk c; refilled with chunk c + 3
    __syncthreads();
    put_x(c + 1);
    fetch_x(c + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(c, D);
    load(c + 3, D);
  };
  // the last 1-5 chunks: no loads past the end
  auto tail_step = [&](int c, Step& D) {
    __syncthreads();
    if (c + 1 < n_chunks) put_x(c + 1);
    if (c + 2 < n_chunks) fetch_x(c + 2);
    compute(c, D);
    if (c + 3 < n_chunks) load(c + 3, D);
  };
  Step A, B, C;
  fetch_x(0);
  load(0, A);
  load(min(1, n_chunks - 1), B);
  load(min(2, n_chunks - 1), C);
  put_x(0);
  fetch_x(1);
  __builtin_amdgcn_sched_barrier(0);
  int c = 0;
  for (; c + 5 < n_chunks; c += 3) {
    step(c, A);
    __builtin_amdgcn_sched_barrier(0);
    step(c + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    step(c + 2, C);
    __builtin_amdgcn_sched_barrier(0);
  }
  tail_step(c, A);
  if (c + 1 < n_chunks) tail_step(c + 1, B);
  if (c + 2 < n_chunks) tail_step(c + 2, C);
  if (c + 3 < n_chunks) tail_step(c + 3, A);
  if (c + 4 < n_chunks) tail_step(c + 4, B);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    if (m >= ti.nr) continue;
    const int64_t base = (int64_t)(ti.r0 + m) * I;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + rt * 16 + 4 * lq + i;
        if (n < I) {
          const float g = accg[rt][mt][i], u = accu[rt][mt][i];
          const float h = (g / (1.0f + expf(-g))) * u;
          uint16_t hi, lo;
          Op<FMT>::split(h, hi, lo);
          h_hi[base + n] = hi;
          h_lo[base + n] = lo;
        }
      }
  }
}

template <int FMT, int NW>
__global__ __launch_bounds__(NW * 64) void ffn_down_tile_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const TileEntry* __restrict__ tiles, int n_experts, const int32_t* __restrict__ sorted_slot, int n_nblk,
    int n_nblk_pad, float* __restrict__ y_slots) {
  constexpr int RT = 2, MT = kDnTileMT, NTOK = 16 * MT;
  constexpr int HALVES = kTileMT / kDnTileMT;     // work items per tile
  constexpr int kStage = 2 * NTOK * kTileRow;     // hi plane, then lo plane
  constexpr int LPT = 2 * NTOK * 16 / (64 * NW);  // 16-byte lane-loads of h per thread per chunk
  typedef typename Op<FMT>::V V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int item = blockIdx.x / n_nblk_pad, nblk = blockIdx.x - item * n_nblk_pad;
  if (nblk >= n_nblk) return;
  TileInfo ti = get_tile(tiles, item / HALVES, n_experts, n_slots, NTOK * HALVES);
  {  // this item's part of the tile's rows
    const int skip = (item % HALVES) * NTOK;
    ti.r0 += skip;
    ti.nr = min(ti.nr - skip, NTOK);
  }
  if (ti.nr <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = (nblk * NW + wave) * 16 * RT;
  const int ex = __builtin_amdgcn_readfirstlane(ti.e);
  const int n_chunks = I >> 7;

  // lane-load q = threadIdx.x + 64 * NW * i: plane q / (16 * NTOK) (uniform per load), token
  // (q / 16) % NTOK, column q % 16
  const __amdgpu_buffer_rsrc_t hr[2] = {make_rsrc(h_hi, (int64_t)n_slots * I * 2), make_rsrc(h_lo, (int64_t)n_slots * I * 2)};
  uint32_t hoff[LPT], hs_w[LPT];
  int hplane[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int q = threadIdx.x + 64 * NW * i, plane = q / (16 * NTOK), tok = (q >> 4) % NTOK, col = q & 15;
    hplane[i] = __builtin_amdgcn_readfirstlane(plane);
    hoff[i] = tok < ti.nr ? (uint32_t)(ti.r0 + tok) * (uint32_t)I * 2u + 16u * col : kOutOfRange;
    hs_w[i] = (uint32_t)(plane * NTOK * kTileRow + tok * kTileRow + 16 * col);
  }
  const uint32_t hs_r = (uint32_t)(l16 * kTileRow + 64 * lq);

  const __amdgpu_buffer_rsrc_t wr = tile_wrsrc<FMT>(down, ex, H, I);
  const __amdgpu_buffer_rsrc_t sr = tile_srsrc<FMT>(down, ex, H, I);
  uint32_t coff[RT], soff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min(n0 + rt * 16 + l16, H - 1);
    coff[rt] = (uint32_t)(n * down.wr) + TileW<FMT>::kLaneBytes * lq;
    soff[rt] = (uint32_t)(n * down.sr);
  }

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    TileW<FMT> w[RT];
  };
  auto load = [&](int c, Step& d) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) tile_load<FMT>(d.w[rt], wr, sr, coff[rt], soff[rt], c);
  };
  // h is fetched one chunk ahead (its rows are shared by every row block of the tile and mostly
  // come from L2)
  u32x4 Hr[LPT];
  auto fetch_h = [&](int c) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) Hr[i] = bld16(hr[hplane[i]], c < n_chunks ? hoff[i] + 256u * c : kOutOfRange);
  };
  auto put_h = [&](int c) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<u32x4*>(lds + (c & 1) * kStage + hs_w[i]) = Hr[i];
  };
  auto compute = [&](int c, const Step& d) {
    const uint8_t* st = lds + (c & 1) * kStage + hs_r;
    float scl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) scl[rt] = tile_scale<FMT>(d.w[rt], lq);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      V bh[MT], bl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // uniform: 16-token column tiles past the rows hold nothing (prefill layer: down 4.90 ->
        // 4.66 ms; the same skip in the gate/up tile kernel was slower, 5.66 -> 5.80 ms)
        if (16 * mt >= ti.nr) break;
        bh[mt] = *reinterpret_cast<const V*>(st + mt * 16 * kTileRow + 16 * k);
        bl[mt] = *reinterpret_cast<const V*>(st + NTOK * kTileRow + mt * 16 * kTileRow + 16 * k);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const V a = tile_operand<FMT>(d.w[rt], k, scl[rt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (16 * mt >= ti.nr) break;
          acc[rt][mt] = Op<FMT>::mfma(a, bh[mt], acc[rt][mt]);
          acc[rt][mt] = Op<FMT>::mfma(a, bl[mt], acc[rt][mt]);
        }
      }
    }
  };
  auto step = [&](int c, Step& D) {
    __syncthreads();
    put_h(c + 1);
    fetch_h(c + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(c, D);
    load(c + 2, D);
  };
  Step A, B;
  fetch_h(0);
  load(0, A);
  load(n_chunks > 1 ? 1 : 0, B);
  put_h(0);
  fetch_h(1);
  __builtin_amdgcn_sched_barrier(0);
  int c = 0;
  for (; c + 3 < n_chunks; c += 2) {
    step(c, A);
    __builtin_amdgcn_sched_barrier(0);
    step(c + 1, B);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if (c + 1 < n_chunks) put_h(c + 1);
  if (c + 2 < n_chunks) fetch_h(c + 2);
  compute(c, A);
  if (c + 2 < n_chunks) load(c + 2, A);
  if (c + 1 < n_chunks) {
    __syncthreads();
    if (c + 2 < n_chunks) put_h(c + 2);
    compute(c + 1, B);
  }
  if (c + 2 < n_chunks) {
    __syncthreads();
    compute(c + 2, A);
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    if (m >= ti.nr) continue;
    const int sl = sorted_slot[ti.r0 + m];
    if (sl < 0 || sl >= n_slots) continue;
    float* dst = y_slots + (int64_t)sl * H;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = n0 + rt * 16 + 4 * lq;
      if ((H & 3) == 0 && n + 3 < H) {
        *reinterpret_cast<f32x4*>(dst + n) = acc[rt][mt];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < H) dst[n + i] = acc[rt][mt][i];
      }
    }
  }
}


constexpr int kNW = 4, kRT1 = 2, kRT2 = 4;
// Row tiles per wave of the K-split streaming kernels (few tiles, e.g. T = 1): one per matrix for
// gate/up, two for down -- twice the workgroups of kRT1 / kRT2 (measured at T = 1 / 4 on the sweep
// workload: gate/up 26.1 -> 25.2 / 108 -> 104 us, down 20.5 -> 18.6 us at T = 1).
constexpr int kStRT1 = 1, kStRT2 = 2;

inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
// The streaming kernels need whole 128-wide chunks, dword-aligned scale rows, a K share per wave
// within the scale table, and 32-bit buffer offsets.
inline bool stream_ok(const ProjDev& p, int K, int64_t rows) {
  return K % 128 == 0 && K <= 4 * 128 * kMaxChunksPerWave && al4(p.s) && p.se % 4 == 0 && p.sr % 4 == 0 &&
         rows * p.wr < INT32_MAX;
}
// FP16 weights on the K-split streaming kernels: whole 128-wide chunks, 16-byte aligned rows.
inline bool stream_ok_f16(const ProjDev& p, int K, int64_t rows) {
  return K % 128 == 0 && K <= 4 * 128 * kMaxChunksPerWave && ((uintptr_t)p.w & 15u) == 0 && p.wr % 16 == 0 &&
         p.we % 16 == 0 && rows * p.wr < INT32_MAX;
}

// K-split streaming kernels: RT 16-row tiles per workgroup (kStRT1 of each matrix for gate/up,
// kStRT2 for down).  Wider blocks amortise each activation chunk over more weight rows but cost
// occupancy and workgroups.
template <int MT, int RT>
void launch_gateup_stream(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate,
                          ProjDev up, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                          const TileEntry* tiles, hipStream_t stream) {
  const int nb = (I + 16 * RT - 1) / (16 * RT);
  const int cpw = (H / 128 + kNW - 1) / kNW;
  const size_t lds = (size_t)kNW * stab_bytes(2 * 16 * RT, cpw) + (size_t)kNW * RT * 2 * 256 * 4;
  ffn_gateup_stream_kernel<kNW, MT, RT><<<dim3((unsigned)(pl.tiles * nb)), kNW * 64, lds, stream>>>(
      (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb, h_hi, h_lo);
}
template <int FMT, int MT, int RT>
void launch_down_stream(const FfnPlan& pl, int T, int k_total, int H, int I, ProjDev down, const int32_t* sorted_slot,
                        float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo, const TileEntry* tiles,
                        hipStream_t stream) {
  const int nb = (H + 16 * RT - 1) / (16 * RT);
  const int cpw = (I / 128 + kNW - 1) / kNW;
  const size_t lds = (size_t)kNW * stab_bytes(16 * RT, cpw) + (size_t)kNW * RT * 256 * 4;
  ffn_down_stream_kernel<FMT, kNW, MT, RT><<<dim3((unsigned)(pl.tiles * nb)), kNW * 64, lds, stream>>>(
      h_hi, h_lo, T * k_total, H, I, down, tiles, pl.n_experts, sorted_slot, nb, y_slots);
}

// Row-split kernels: worth it once there are enough row blocks to fill the chip with full-K
// streams; below that the K-split kernels spread each expert over more workgroups.
constexpr int64_t kRowsMinBlocks = 1024;
constexpr size_t kMaxLds = 160 * 1024;
size_t gateup_rows_lds(int H, int rt, int nw) {  // x ring, scale tables, a 512-byte transposition slot per wave
  return 2 * (size_t)kGuXStage + nw * (size_t)stab_bytes(2 * 16 * rt, rows_stab_stride(H / 128)) + nw * 512;
}
// Gate/up row-split workgroups: one 16-row tile of each matrix per wave and 8 waves sharing each
// x stage, or 4 waves when 8-wave row blocks would give fewer than kGuSmallBlocks workgroups
// (measured on the sweep workload, 8 waves: T = 176 685 -> 667 us, T = 128 673 -> 657 us,
// T = 64 600 -> 595 us, T = 8 153 -> 159 us; two tiles per wave were slower at every T).
constexpr int64_t kGuSmallBlocks = 4096;
constexpr int kGuNW = 8, kGuNWSmall = 4;
// Waves per down workgroup (they share each h stage): 8 at every T.  (With 64-byte half-line
// loads, 4-wave workgroups were faster below 4,096 eight-wave blocks: T = 32 236 -> 229 us.  With
// whole-line loads 8 waves are faster throughout, side by side: T = 8 88.5 -> 87.2 us, T = 32
// 228 -> 218 us, T = 88 346 -> 326 us.)
constexpr int kDnNW = 8;
size_t down_rows_lds(int I, int nw) {  // h ring, scale tables, a 1 KB transposition slot per wave
  return 2 * (size_t)DnStage::kBytes + nw * (size_t)stab_bytes(16 * kRowsRT2, rows_stab_stride(I / 128)) + nw * 1024;
}

template <int FMT, int MT>
hipError_t gateup_mt(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
                     const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo, const TileEntry* tiles,
                     hipStream_t stream) {
  // (FP16 weights take the general kernel here: on the dense slices the K-split streaming form
  // with FP16 loads was no faster at 1 token and slower at 16, 61.0 -> 64.5 us)
  const bool streamable = FMT == MOE_W_MXFP4 && stream_ok(gate, H, I) && stream_ok(up, H, I) && (int64_t)T * H * 2 < INT32_MAX;
  const int nb8 = (I + 16 * kGuNW - 1) / (16 * kGuNW);
  const bool small = pl.tiles * nb8 < kGuSmallBlocks;
  const int nw = small ? kGuNWSmall : kGuNW;
  const int nb_rows = (I + 16 * nw - 1) / (16 * nw);
  const int tiny_cpw = tiny_gateup_cpw(H);
  const size_t tiny_lds = (size_t)T * H * 2 + (size_t)kTinyNW * stab_bytes(32, tiny_cpw) + (size_t)kTinyNW * 2 * 256 * 4 +
                          (size_t)kTinyNW * 1024;  // x, scale tables, reduction, transposition slots
  // (pl.tiny: T <= kTinyT.)  Measured on the sweep layer against the streaming kernel: T = 1 31.3 ->
  // 29.4 us, T = 2 56.5 -> 52.8 us, but T = 4 105 -> 109 us (x for 4 tokens takes 56 KB of LDS per
  // workgroup and halves the workgroups per CU), so up to kTinyGuT tokens.
  if (MT == 1 && streamable && pl.tiny && T <= kTinyGuT && H % 512 == 0 && tiny_lds <= kMaxLds) {
    const int nb = (I + 15) / 16;
    const size_t lds = tiny_lds;
    ffn_gateup_tiny_kernel<<<dim3((unsigned)(pl.tiles * nb)), kTinyNW * 64, lds, stream>>>(
        (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb, h_hi, h_lo);
  } else if (MT == 1 && streamable && gateup_rows_lds(H, 1, nw) <= kMaxLds && pl.tiles * nb8 >= kRowsMinBlocks) {
    const dim3 grid((unsigned)(pl.tiles * nb_rows));
    if (small)
      ffn_gateup_rows_kernel<kGuNWSmall, 1><<<grid, kGuNWSmall * 64, gateup_rows_lds(H, 1, nw), stream>>>(
          (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb_rows, h_hi, h_lo);
    else
      ffn_gateup_rows_kernel<kGuNW, 1><<<grid, kGuNW * 64, gateup_rows_lds(H, 1, nw), stream>>>(
          (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb_rows, h_hi, h_lo);
  } else if (MT == 1 && streamable) {
    const int nb = (I + 15) / 16;
    ffn_gateup_split_lines_kernel<kSplitLinesDP><<<dim3((unsigned)(pl.tiles * nb)), kTinyNW * 64,
                                                   gateup_split_lines_lds(H), stream>>>(
        (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb, h_hi, h_lo);
  } else if (streamable) {
    launch_gateup_stream<MT, kStRT1>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  } else {
    const int nb = (I + 16 * kRT1 - 1) / (16 * kRT1);
    ffn_gateup_kernel<FMT, kNW, kRT1, MT><<<dim3((unsigned)(pl.tiles * nb)), kNW * 64, 0, stream>>>(
        (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb, h_hi, h_lo, 1.0f, 0);
  }
  return hipGetLastError();
}

template <int FMT, int MT>
hipError_t down_mt(const FfnPlan& pl, int T, int k_total, int H, int I, ProjDev down, const int32_t* sorted_slot,
                   float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo, const TileEntry* tiles,
                   hipStream_t stream) {
  const int n_slots = T * k_total;
  constexpr bool mx = FMT == MOE_W_MXFP4;  // the tiny and row-split down kernels are MXFP4 only
  const bool streamable = (mx ? stream_ok(down, I, H) : FMT == MOE_W_FP16 && stream_ok_f16(down, I, H)) &&
                          (int64_t)n_slots * I * 2 < INT32_MAX;
  const int nw = kDnNW;
  const int nb_rows = (H + 16 * kRowsRT2 * nw - 1) / (16 * kRowsRT2 * nw);
  if (mx && MT == 1 && streamable && pl.tiny) {  // (the plan holds it only for H a multiple of 16 * kTinyNW)
    const int nb = H / (16 * kTinyNW);
    const size_t lds = (size_t)2 * kTinyT * I * 2 + kTinyNW * 1024;
    if (T == 1)
      ffn_down_tiny_kernel<2><<<dim3((unsigned)(pl.tiles * nb)), kTinyNW * 64, lds, stream>>>(
          h_hi, h_lo, n_slots, H, I, down, tiles, pl.n_experts, sorted_slot, nb, y_slots);
    else
      ffn_down_tiny_kernel<kTinyNC / 2><<<dim3((unsigned)(pl.tiles * nb)), kTinyNW * 64, lds, stream>>>(
          h_hi, h_lo, n_slots, H, I, down, tiles, pl.n_experts, sorted_slot, nb, y_slots);
  } else if (mx && MT == 1 && streamable && down_rows_lds(I, nw) <= kMaxLds && pl.tiles * nb_rows >= kRowsMinBlocks / 4) {
    // (kRowsMinBlocks / 4 eight-wave blocks: the 2,048 waves that kRowsMinBlocks / 2 four-wave
    // blocks gave before the down kernel dropped its 4-wave form)
    ffn_down_lines_kernel<kDnNW><<<dim3((unsigned)(pl.tiles * nb_rows)), kDnNW * 64, down_rows_lds(I, nw), stream>>>(
        h_hi, h_lo, n_slots, H, I, down, tiles, pl.n_experts, sorted_slot, nb_rows, y_slots);
  } else if (streamable && (mx || MT == 1)) {
    // (FP16 weights with one token tile: dense slices T = 1 35.6 -> 29.1 us, T = 16 unchanged)
    if constexpr (mx || (FMT == MOE_W_FP16 && MT == 1))
      launch_down_stream<FMT, MT, kStRT2>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  } else {
    const int nb = (H + 16 * kRT2 - 1) / (16 * kRT2);
    ffn_down_kernel<FMT, kNW, kRT2, MT><<<dim3((unsigned)(pl.tiles * nb)), kNW * 64, 0, stream>>>(
        h_hi, h_lo, n_slots, H, I, down, tiles, pl.n_experts, sorted_slot, nb, y_slots, nullptr);
  }
  return hipGetLastError();
}

// The range-managed FFN (Cascadia Sec. 3.3, Eq. 1) on the general kernels: u attenuated by
// u_scale, h rounded to binary16, outputs stored as binary16 in y16.
template <int FMT, int MT>
hipError_t ffn_range_mt(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
                        ProjDev down, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                        const TileEntry* tiles, float u_scale, uint16_t* y16, hipStream_t stream) {
  const int nb1 = (I + 16 * kRT1 - 1) / (16 * kRT1);
  ffn_gateup_kernel<FMT, kNW, kRT1, MT><<<dim3((unsigned)(pl.tiles * nb1)), kNW * 64, 0, stream>>>(
      (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb1, h_hi, h_lo, u_scale, 1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nb2 = (H + 16 * kRT2 - 1) / (16 * kRT2);
  ffn_down_kernel<FMT, kNW, kRT2, MT><<<dim3((unsigned)(pl.tiles * nb2)), kNW * 64, 0, stream>>>(
      h_hi, h_lo, T * k_total, H, I, down, tiles, pl.n_experts, sorted_slot, nb2, nullptr, y16);
  return hipGetLastError();
}
template <int FMT>
hipError_t ffn_range_fmt(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate,
                         ProjDev up, ProjDev down, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                         const TileEntry* tiles, float u_scale, uint16_t* y16, hipStream_t stream) {
  switch (pl.mt) {
    case 1: return ffn_range_mt<FMT, 1>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles, u_scale, y16, stream);
    case 2: return ffn_range_mt<FMT, 2>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles, u_scale, y16, stream);
    default: return ffn_range_mt<FMT, 4>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles, u_scale, y16, stream);
  }
}

// The tile kernels (planned only when ffn_plan_opts() gives kPlanBig for the call).
template <int FMT>
hipError_t gateup_tile(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
                       const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo, const TileEntry* tiles,
                       hipStream_t stream) {
  const int nb = (I + 16 * kTileRT * kNW - 1) / (16 * kTileRT * kNW), nbp = (nb + kXcds - 1) / kXcds * kXcds;
  ffn_gateup_tile_kernel<FMT, kNW, kTileRT, kTileMT><<<dim3((unsigned)(pl.tiles * nbp)), kNW * 64,
                                                 2 * kTileMT * 16 * kTileRow, stream>>>(
      (const uint16_t*)x, T, k_total, H, I, gate, up, tiles, pl.n_experts, sorted_slot, nb, nbp, h_hi, h_lo);
  return hipGetLastError();
}
template <int FMT>
hipError_t down_tile(const FfnPlan& pl, int T, int k_total, int H, int I, ProjDev down, const int32_t* sorted_slot,
                     float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo, const TileEntry* tiles,
                     hipStream_t stream) {
  const int nb = (H + 16 * 2 * kNW - 1) / (16 * 2 * kNW), nbp = (nb + kXcds - 1) / kXcds * kXcds;
  ffn_down_tile_kernel<FMT, kNW><<<dim3((unsigned)(pl.tiles * (kTileMT / kDnTileMT) * nbp)), kNW * 64,
                              2 * 2 * kDnTileMT * 16 * kTileRow, stream>>>(
      h_hi, h_lo, T * k_total, H, I, down, tiles, pl.n_experts, sorted_slot, nb, nbp, y_slots);
  return hipGetLastError();
}

template <int FMT>
hipError_t gateup_fmt(const FfnPlan& pl, const void* x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
                      const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo, const TileEntry* tiles,
                      hipStream_t stream) {
  switch (pl.mt) {
    case 1: return gateup_mt<FMT, 1>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
    case 2: return gateup_mt<FMT, 2>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
    default: return gateup_mt<FMT, 4>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  }
}

template <int FMT>
hipError_t down_fmt(const FfnPlan& pl, int T, int k_total, int H, int I, ProjDev down, const int32_t* sorted_slot,
                    float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo, const TileEntry* tiles,
                    hipStream_t stream) {
  switch (pl.mt) {
    case 1: return down_mt<FMT, 1>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
    case 2: return down_mt<FMT, 2>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
    default: return down_mt<FMT, 4>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  }
}

}  // namespace

hipError_t launch_ffn_range(const void* x, int T, int k_total, int fmt, int n_experts, int H, int I, ProjDev gate,
                            ProjDev up, ProjDev down, const int32_t* offsets, const int32_t* sorted_slot,
                            uint16_t* h_hi, uint16_t* h_lo, void* table, int att_log2, uint16_t* y16,
                            hipStream_t stream) {
  const FfnPlan pl = ffn_plan(T, k_total, n_experts, 0);
  hipError_t err = launch_ffn_plan(T, k_total, n_experts, 0, offsets, table, stream);
  if (err != hipSuccess) return err;
  const float u_scale = ldexpf(1.0f, -att_log2);
  const TileEntry* tiles = (const TileEntry*)table;
  if (fmt == MOE_W_FP16)
    return ffn_range_fmt<MOE_W_FP16>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles, u_scale,
                                     y16, stream);
  if (fmt == MOE_W_INT4_G32)
    return ffn_range_fmt<MOE_W_INT4_G32>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles,
                                         u_scale, y16, stream);
  if (fmt == MOE_W_NVFP4)
    return ffn_range_fmt<MOE_W_NVFP4>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles,
                                      u_scale, y16, stream);
  return ffn_range_fmt<MOE_W_MXFP4>(pl, x, T, k_total, H, I, gate, up, down, sorted_slot, h_hi, h_lo, tiles, u_scale,
                                    y16, stream);
}

int ffn_plan_opts(int fmt, int T, int k_total, int H, int I, const ProjDev& gate, const ProjDev& up,
                  const ProjDev& down) {
  const bool offs = (int64_t)T * H * 2 < INT32_MAX && (int64_t)T * k_total * I * 2 < INT32_MAX;
  const bool streams = stream_ok(gate, H, I) && stream_ok(up, H, I) && stream_ok(down, I, H) && offs;
  int opts = 0;
  if ((fmt == MOE_W_MXFP4 || fmt == MOE_W_FP16) && streams) opts |= kPlanBig;
  if (fmt == MOE_W_MXFP4 && streams && T <= kTinyT && I <= 128 * kTinyNC && I % 512 == 0 && H % (16 * kTinyNW) == 0 &&
      (down.sr & 15) == 0 && (down.se & 15) == 0 && ((uintptr_t)down.s & 15) == 0)
    opts |= kPlanTiny;
  return opts;
}

FfnPlan ffn_plan(int T, int k_total, int n_experts, int opts) {
  // Tokens per tile from the mean rows per active expert (known on the host without a sync).
  const int64_t rows = (int64_t)T * k_total;
  const int64_t active = rows < n_experts ? rows : n_experts;
  const double mean = (double)rows / (double)(active > 0 ? active : 1);
  FfnPlan p;
  p.n_experts = n_experts;
  p.tile = (opts & kPlanBig) && mean > 32.0;  // 16 * kTileMT-token tiles on the tile kernels
  p.tiny = !p.tile && (opts & kPlanTiny) && T <= kTinyT;
  p.mt = p.tile ? kTileMT : (mean <= 16.0 ? 1 : (mean <= 32.0 ? 2 : 4));
  p.rpt = p.tiny ? kTinyT : 16 * p.mt;
  p.tiles = (max_tiles(rows, n_experts, p.rpt) + kXcds - 1) / kXcds * kXcds;
  return p;
}

size_t ffn_table_bytes(int T, int k_total, int n_experts, int opts) {
  return (size_t)ffn_plan(T, k_total, n_experts, opts).tiles * sizeof(TileEntry);
}

hipError_t launch_ffn_tiles(const int32_t* offsets, int n_experts, int n_rows, int rows_per_tile, int64_t n_entries,
                            void* table, hipStream_t stream) {
  ffn_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, n_experts, n_rows, rows_per_tile, (int)n_entries,
                                           (TileEntry*)table);
  return hipGetLastError();
}

hipError_t launch_ffn_plan(int T, int k_total, int n_experts, int opts, const int32_t* offsets, void* table,
                           hipStream_t stream) {
  const FfnPlan pl = ffn_plan(T, k_total, n_experts, opts);
  ffn_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, n_experts, T * k_total, pl.rpt, (int)pl.tiles, (TileEntry*)table);
  return hipGetLastError();
}

hipError_t launch_ffn_gateup(const void* x, int T, int k_total, int fmt, int n_experts, int opts, int H, int I,
                             ProjDev gate, ProjDev up, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                             const void* table, hipStream_t stream) {
  const FfnPlan pl = ffn_plan(T, k_total, n_experts, opts);
  const TileEntry* tiles = (const TileEntry*)table;
  if (pl.tile) {
    if (fmt == MOE_W_FP16)
      return gateup_tile<MOE_W_FP16>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
    return gateup_tile<MOE_W_MXFP4>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  }
  if (fmt == MOE_W_FP16)
    return gateup_fmt<MOE_W_FP16>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  if (fmt == MOE_W_INT4_G32)
    return gateup_fmt<MOE_W_INT4_G32>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  if (fmt == MOE_W_NVFP4)
    return gateup_fmt<MOE_W_NVFP4>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
  return gateup_fmt<MOE_W_MXFP4>(pl, x, T, k_total, H, I, gate, up, sorted_slot, h_hi, h_lo, tiles, stream);
}

hipError_t launch_ffn_down(int T, int k_total, int fmt, int n_experts, int opts, int H, int I, ProjDev down,
                           const int32_t* sorted_slot, float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo,
                           const void* table, hipStream_t stream) {
  const FfnPlan pl = ffn_plan(T, k_total, n_experts, opts);
  const TileEntry* tiles = (const TileEntry*)table;
  if (pl.tile) {
    if (fmt == MOE_W_FP16)
      return down_tile<MOE_W_FP16>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
    return down_tile<MOE_W_MXFP4>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  }
  if (fmt == MOE_W_FP16)
    return down_fmt<MOE_W_FP16>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  if (fmt == MOE_W_INT4_G32)
    return down_fmt<MOE_W_INT4_G32>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  if (fmt == MOE_W_NVFP4)
    return down_fmt<MOE_W_NVFP4>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
  return down_fmt<MOE_W_MXFP4>(pl, T, k_total, H, I, down, sorted_slot, y_slots, h_hi, h_lo, tiles, stream);
}

}  // namespace moe
