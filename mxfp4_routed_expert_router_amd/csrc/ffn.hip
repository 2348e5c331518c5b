// Grouped SwiGLU expert FFN over the buckets (Cascadia, Sec. 3.1: gate/up projections, SwiGLU and
// down projection of the selected experts), with MXFP4 decode inside the reduction and FP32
// accumulation (FreeToken DeepSeek-V4-Flash post, "MXFP4 is not NVFP4": scales load once per
// 32-weight block and broadcast; no BF16 copy of an expert is ever materialised).
//
// Work unit.  A "tile" is up to 16*MT consecutive sorted rows (tokens) of one expert; tiles are
// numbered expert by expert, so an expert with n rows owns ceil(n / (16*MT)) tiles.  A workgroup
// takes one tile and one block of 16*RT weight rows and covers the full reduction dimension K:
// each of its NW waves reduces a contiguous share of K's 128-wide chunks, then the partial sums
// meet in LDS.  Weights are therefore read from HBM once per tile -- once per active expert when
// an expert has at most 16*MT tokens, which is the decode regime.
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

namespace moe {

namespace {

struct TileInfo {
  int e, r0, nr;  // expert, first sorted row, rows in this tile (0 => no tile)
};

// Tile j -> (expert, rows).  Wave 0 builds per-lane tile counts over the experts and a wave scan;
// the result goes through LDS to the whole workgroup.  Offsets are clamped so corrupt device data
// cannot produce rows outside [0, n_rows_max).
__device__ TileInfo find_tile(const int32_t* __restrict__ offsets, int n_experts, int n_rows_max, int rows_per_tile,
                              int j, int* s_info) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (n_experts + 63) / 64;
    const int eb = min(lane * per, n_experts), ee = min(eb + per, n_experts);
    int cnt = 0;
    for (int e = eb; e < ee; ++e) {
      int a = min(max(offsets[e], 0), n_rows_max), b = min(max(offsets[e + 1], 0), n_rows_max);
      int n = max(b - a, 0);
      cnt += (n + rows_per_tile - 1) / rows_per_tile;
    }
    const int incl = wave_incl_scan(cnt);
    const int excl = incl - cnt;
    const int total = __shfl(incl, 63, kWave);
    if (lane == 0 && j >= total) {
      s_info[0] = -1;
      s_info[1] = 0;
      s_info[2] = 0;
    }
    if (j >= excl && j < incl) {
      int acc = excl;
      for (int e = eb; e < ee; ++e) {
        int a = min(max(offsets[e], 0), n_rows_max), b = min(max(offsets[e + 1], 0), n_rows_max);
        int n = max(b - a, 0);
        int tiles = (n + rows_per_tile - 1) / rows_per_tile;
        if (j < acc + tiles) {
          const int r0 = a + (j - acc) * rows_per_tile;
          s_info[0] = e;
          s_info[1] = r0;
          s_info[2] = min(rows_per_tile, b - r0);
          break;
        }
        acc += tiles;
      }
    }
  }
  __syncthreads();
  TileInfo t;
  t.e = s_info[0];
  t.r0 = s_info[1];
  t.nr = t.e < 0 ? 0 : s_info[2];
  return t;
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

// Raw weight data of one lane for one chunk and one 16-row tile: the 16-byte MXFP4 block and its
// scale, or 4 x 16 bytes of fp16.
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

// Load lane's raw weights: row pointer `row` (already offset to expert and row), its scale row,
// k = this lane's block start; ok = row and block inside the matrix.
template <int FMT>
__device__ __forceinline__ RawW<FMT> load_w(const uint8_t* row, const uint8_t* srow, int k, bool ok) {
  RawW<FMT> r;
  if constexpr (FMT == MOE_W_MXFP4) {
    if (ok) {
      r.q = ld16(row + (k >> 1));
      r.e = srow[k >> 5];
    } else {
      r.q = u32x4{0, 0, 0, 0};
      r.e = 127;
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) r.q[s] = ok ? ld16(row + 2 * (k + 8 * s)) : u32x4{0, 0, 0, 0};
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ typename Op<FMT>::V decode_step(const RawW<FMT>& r, int s) {
  if constexpr (FMT == MOE_W_MXFP4) {
    return decode8_bf16(r.q[s], e8m0_to_f32(r.e));
  } else {
    return bitcast<f16x8>(r.q[s]);
  }
}

// ------------------------------------------------------------------------------------------------
// gate/up + SwiGLU:  h[r, n] = SiLU(sum_k Wg[e,n,k] x[t,k]) * (sum_k Wu[e,n,k] x[t,k])
// ------------------------------------------------------------------------------------------------
template <int FMT, int NW, int RT, int MT>
__global__ __launch_bounds__(NW * 64) void ffn_gateup_kernel(
    const uint16_t* __restrict__ x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int n_experts, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  typedef typename Op<FMT>::V V;
  __shared__ int s_info[4];
  __shared__ float s_red[NW][RT][2][256];
  const int n_slots = T * k_total;
  const int nblk = blockIdx.x % n_nblk;
  const int tile = blockIdx.x / n_nblk;
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
  if (ti.nr <= 0) return;  // uniform across the workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
  const uint8_t *grow[RT], *urow[RT], *gsrow[RT], *usrow[RT];
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

  RawW<FMT> wg[RT], wu[RT];
  if (c0 < c1) {
    const int k = c0 * 128 + 32 * lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wg[rt] = load_w<FMT>(grow[rt], gsrow[rt], k, row_ok[rt] && k < H);
      wu[rt] = load_w<FMT>(urow[rt], usrow[rt], k, row_ok[rt] && k < H);
    }
  }
  for (int c = c0; c < c1; ++c) {
    const int k = c * 128 + 32 * lq;
    const bool k_ok = k < H;
    // prefetch the next chunk's weights
    RawW<FMT> ng[RT], nu[RT];
    if (c + 1 < c1) {
      const int kn = k + 128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        ng[rt] = load_w<FMT>(grow[rt], gsrow[rt], kn, row_ok[rt] && kn < H);
        nu[rt] = load_w<FMT>(urow[rt], usrow[rt], kn, row_ok[rt] && kn < H);
      }
    }
    // activations: 4 x 16 bytes per token
    V xb[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xb[mt][s] = bitcast<V>((tok_ok[mt] && k_ok) ? ld16(xrow[mt] + k + 8 * s) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const V ag = decode_step<FMT>(wg[rt], s);
        const V au = decode_step<FMT>(wu[rt], s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          accg[mt][rt] = Op<FMT>::mfma(ag, xb[mt][s], accg[mt][rt]);
          accu[mt][rt] = Op<FMT>::mfma(au, xb[mt][s], accu[mt][rt]);
        }
      }
    }
    if (c + 1 < c1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        wg[rt] = ng[rt];
        wu[rt] = nu[rt];
      }
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
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < I && m < ti.nr) {
        const float h = (g / (1.0f + expf(-g))) * u;
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
template <int FMT, int NW, int RT, int MT>
__global__ __launch_bounds__(NW * 64) void ffn_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int n_slots, int H, int I, ProjDev down,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int n_experts, int n_nblk,
    float* __restrict__ y_slots) {
  typedef typename Op<FMT>::V V;
  __shared__ int s_info[4];
  __shared__ float s_red[NW][RT][256];
  const int nblk = blockIdx.x % n_nblk;
  const int tile = blockIdx.x / n_nblk;
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
  if (ti.nr <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
  const uint8_t *drow[RT], *dsrow[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + rt * 16 + l16;
    row_ok[rt] = n < H;
    const int nn = row_ok[rt] ? n : 0;
    drow[rt] = down.w + (int64_t)ti.e * down.we + (int64_t)nn * down.wr;
    dsrow[rt] = down.s ? down.s + (int64_t)ti.e * down.se + (int64_t)nn * down.sr : nullptr;
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
  if (c0 < c1) {
    const int k = c0 * 128 + 32 * lq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wd[rt] = load_w<FMT>(drow[rt], dsrow[rt], k, row_ok[rt] && k < I);
  }
  for (int c = c0; c < c1; ++c) {
    const int k = c * 128 + 32 * lq;
    const bool k_ok = k < I;
    RawW<FMT> nd[RT];
    if (c + 1 < c1) {
      const int kn = k + 128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) nd[rt] = load_w<FMT>(drow[rt], dsrow[rt], kn, row_ok[rt] && kn < I);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      V bh[MT], bl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bool ok = tok_ok[mt] && k_ok;
        bh[mt] = bitcast<V>(ok ? ld16(hrow_hi[mt] + k + 8 * s) : u32x4{0, 0, 0, 0});
        bl[mt] = bitcast<V>(ok ? ld16(hrow_lo[mt] + k + 8 * s) : u32x4{0, 0, 0, 0});
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const V a = decode_step<FMT>(wd[rt], s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][rt] = Op<FMT>::mfma(a, bh[mt], acc[mt][rt]);
          acc[mt][rt] = Op<FMT>::mfma(a, bl[mt], acc[mt][rt]);
        }
      }
    }
    if (c + 1 < c1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wd[rt] = nd[rt];
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
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < H && m < ti.nr) {
        const int s = sorted_slot[ti.r0 + m];
        if (s >= 0 && s < n_slots) y_slots[(int64_t)s * H + n] = v;
      }
    }
  }
}

// Upper bound of the number of tiles: A active experts hold at least one row each, so
// sum_e ceil(n_e / R) <= A + (rows - A) / R with A <= min(n_experts, rows).
int64_t max_tiles(int64_t rows, int n_experts, int rows_per_tile) {
  const int64_t a = rows < n_experts ? rows : n_experts;
  return a + (rows - a) / rows_per_tile;
}

template <int FMT, int MT>
hipError_t launch_ffn_mt(const void* x, int T, int k_total, int n_experts, int H, int I, ProjDev gate, ProjDev up,
                         ProjDev down, const int32_t* offsets, const int32_t* sorted_slot, float* y_slots,
                         uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream) {
  constexpr int NW = 4, RT1 = 2, RT2 = 4;
  const int n_slots = T * k_total;
  const int64_t tiles = max_tiles(n_slots, n_experts, 16 * MT);
  const int nb1 = (I + 16 * RT1 - 1) / (16 * RT1);
  const int nb2 = (H + 16 * RT2 - 1) / (16 * RT2);
  ffn_gateup_kernel<FMT, NW, RT1, MT><<<dim3((unsigned)(tiles * nb1)), NW * 64, 0, stream>>>(
      (const uint16_t*)x, T, k_total, H, I, gate, up, offsets, sorted_slot, n_experts, nb1, h_hi, h_lo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  ffn_down_kernel<FMT, NW, RT2, MT><<<dim3((unsigned)(tiles * nb2)), NW * 64, 0, stream>>>(
      h_hi, h_lo, n_slots, H, I, down, offsets, sorted_slot, n_experts, nb2, y_slots);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_ffn_fmt(const void* x, int T, int k_total, int n_experts, int H, int I, ProjDev gate, ProjDev up,
                          ProjDev down, const int32_t* offsets, const int32_t* sorted_slot, float* y_slots,
                          uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream) {
  // Tokens per tile from the mean rows per active expert (known on the host without a sync).
  const int64_t rows = (int64_t)T * k_total;
  const int64_t active = rows < n_experts ? rows : n_experts;
  const double mean = (double)rows / (double)(active > 0 ? active : 1);
  if (mean <= 16.0)
    return launch_ffn_mt<FMT, 1>(x, T, k_total, n_experts, H, I, gate, up, down, offsets, sorted_slot, y_slots, h_hi,
                                 h_lo, stream);
  if (mean <= 32.0)
    return launch_ffn_mt<FMT, 2>(x, T, k_total, n_experts, H, I, gate, up, down, offsets, sorted_slot, y_slots, h_hi,
                                 h_lo, stream);
  return launch_ffn_mt<FMT, 4>(x, T, k_total, n_experts, H, I, gate, up, down, offsets, sorted_slot, y_slots, h_hi,
                               h_lo, stream);
}

}  // namespace

hipError_t launch_expert_ffn(const void* x, int T, int k_total, int fmt, int n_experts, int H, int I, ProjDev gate,
                             ProjDev up, ProjDev down, const int32_t* offsets, const int32_t* sorted_slot,
                             float* y_slots, uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream) {
  if (fmt == MOE_W_FP16)
    return launch_ffn_fmt<MOE_W_FP16>(x, T, k_total, n_experts, H, I, gate, up, down, offsets, sorted_slot, y_slots,
                                      h_hi, h_lo, stream);
  return launch_ffn_fmt<MOE_W_MXFP4>(x, T, k_total, n_experts, H, I, gate, up, down, offsets, sorted_slot, y_slots,
                                     h_hi, h_lo, stream);
}

}  // namespace moe
