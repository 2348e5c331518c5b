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

// Work item of workgroup b.  Workgroups are dispatched round-robin over the 8 XCDs (b % 8), and
// each XCD has its own L2.  Tile t runs all of its n-blocks on XCD t % 8, consecutively, so the
// activation rows of an expert (and, in the down phase, its h rows written by the gate/up phase
// with the same mapping) are fetched into one L2 instead of eight.  The grid holds
// 8 * ceil(tiles / 8) * n_nblk workgroups.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_work(int b, int n_nblk, int& tile, int& nblk) {
  const int xcd = b % kXcds, slot = b / kXcds;
  tile = (slot / n_nblk) * kXcds + xcd;
  nblk = slot % n_nblk;
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
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
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
      wg[rt] = load_w<FMT>(grow[rt], gsrow[rt], k, row_ok[rt] && k < H);
      wu[rt] = load_w<FMT>(urow[rt], usrow[rt], k, row_ok[rt] && k < H);
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
        ng[rt] = load_w<FMT>(grow[rt], gsrow[rt], kn, row_ok[rt] && kn < H);
        nu[rt] = load_w<FMT>(urow[rt], usrow[rt], kn, row_ok[rt] && kn < H);
      }
      load_x(kn, nx);
    }
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
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
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
    for (int rt = 0; rt < RT; ++rt) wd[rt] = load_w<FMT>(drow[rt], dsrow[rt], k, row_ok[rt] && k < I);
    load_h(k, bh, bl);
  }
  for (int c = c0; c < c1; ++c) {
    const int k = c * 128 + 32 * lq;
    RawW<FMT> nd[RT];
    V nh[MT][4], nl[MT][4];
    if (c + 1 < c1) {
      const int kn = k + 128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) nd[rt] = load_w<FMT>(drow[rt], dsrow[rt], kn, row_ok[rt] && kn < I);
      load_h(kn, nh, nl);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const V a = decode_step<FMT>(wd[rt], s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][rt] = Op<FMT>::mfma(a, bh[mt][s], acc[mt][rt]);
          acc[mt][rt] = Op<FMT>::mfma(a, bl[mt][s], acc[mt][rt]);
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
      const int n = n0 + rt * 16 + row, m = mt * 16 + tok;
      if (n < H && m < ti.nr) {
        const int s = sorted_slot[ti.r0 + m];
        if (s >= 0 && s < n_slots) y_slots[(int64_t)s * H + n] = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Streaming variants for MXFP4 with 128-aligned K and 4-byte aligned scale rows (every workload
// shape): each wave keeps a private LDS ring of S chunks filled by direct global->LDS loads
// (global_load_lds_dwordx4 for codes, global_load_lds_dword for scales), so S-1 chunks of weights
// are in flight per wave without holding them in VGPRs.  The ring is private to its wave, so the
// loop has no barrier; completion is tracked with explicit vmcnt waits (loads return in issue
// order).  64 (matrix, row) pairs per workgroup row block: gate/up use 2 matrices x 32 rows,
// down 1 matrix x 64 rows, so one dword-load instruction fetches all scales of a chunk.
// ------------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Ring reads go through inline asm: the compiler cannot tell which in-flight DMA targets which
// stage and would otherwise wait for every outstanding load (vmcnt(0)) before each ring read.
// lds_sync ties the results to an explicit lgkmcnt wait so no use is scheduled before it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr)p; }
__device__ __forceinline__ u32x4 lds_read16(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ uint32_t lds_read8(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
template <int RT>
__device__ __forceinline__ void lds_sync(u32x4 (&q)[RT], uint32_t (&e)[RT]) {
  if constexpr (RT == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(q[0]), "+v"(q[1]), "+v"(e[0]), "+v"(e[1]));
  } else {
    static_assert(RT == 4, "lds_sync");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
  }
}

// Buffer resources (raw, stride 0) over one expert's matrix or one activation tensor.  Loads through
// them are MUBUF instructions: the compiler keeps exact vmcnt accounting for them (FLAT-encoded
// global_load_lds would make it treat the queue as unordered and drain it), and the descriptor's
// range bounds every access.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufferFlags);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, off, 0, 0, 0);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Per-wave LDS: a ring of S stages of NM*RT x 1 KB of codes, then a scale table holding, for each
// of the 64 (matrix, row) pairs of the workgroup, the scale bytes of the wave's whole K share
// (4 per chunk, as dwords).  The table is filled once per work item by dword DMAs whose
// consecutive lanes read consecutive dwords of one row, so an instruction touches a few cache
// lines instead of one line per row.
template <int NM, int RT>
struct Ring {
  static constexpr int kStage = NM * RT * 1024;
  static constexpr int kRows = NM * RT * 16;  // 64
  static_assert(kRows == 64, "one scale row per lane");
  static constexpr int kMaxChunksPerWave = 64;  // K share of a wave <= 8192
  static constexpr int bytes(int S, int cpw) { return S * kStage + kRows * cpw * 4; }
};

// Activation and h pointers are deliberately not __restrict__: their loads must stay in program
// order relative to the explicit vmcnt waits (an asm memory clobber does not fence restrict loads).
template <int NW, int MT, int S>
__global__ __launch_bounds__(NW * 64) void ffn_gateup_ring_kernel(
    const uint16_t* x, int T, int k_total, int H, int I, ProjDev gate, ProjDev up,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int n_experts, int n_nblk,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  constexpr int RT = 2, NM = 2;
  typedef Ring<NM, RT> R;
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_info[4];
  const int n_slots = T * k_total;
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
  if (ti.nr <= 0) return;
  // wave index in an SGPR: the K-share loop bounds are then wave-uniform (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;
  const int e = __builtin_amdgcn_readfirstlane(ti.e);

  // activation rows of this lane's tokens (padded lanes read the tile's first token)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)T * H * 2);
  uint32_t xoff[MT];
  {
    const int s_first = sorted_slot[ti.r0];
    const int t_first = (s_first >= 0 && s_first < n_slots) ? s_first / k_total : 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + l16;
      bool ok = m < ti.nr;
      const int sl = ok ? sorted_slot[ti.r0 + m] : -1;
      ok = ok && sl >= 0 && sl < n_slots;
      xoff[mt] = (uint32_t)(ok ? sl / k_total : t_first) * (uint32_t)H * 2u + 64u * lq;
    }
  }
  // this expert's gate and up matrices and scale grids
  const __amdgpu_buffer_rsrc_t wr[NM] = {make_rsrc(gate.w + (int64_t)e * gate.we, (int64_t)(I - 1) * gate.wr + H / 2),
                                         make_rsrc(up.w + (int64_t)e * up.we, (int64_t)(I - 1) * up.wr + H / 2)};
  const __amdgpu_buffer_rsrc_t sr[NM] = {make_rsrc(gate.s + (int64_t)e * gate.se, (int64_t)(I - 1) * gate.sr + H / 32),
                                         make_rsrc(up.s + (int64_t)e * up.se, (int64_t)(I - 1) * up.sr + H / 32)};
  uint32_t coff[NM][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min(n0 + rt * 16 + l16, I - 1);
    coff[0][rt] = (uint32_t)(n * gate.wr) + 16u * lq;
    coff[1][rt] = (uint32_t)(n * up.wr) + 16u * lq;
  }
  const int n_chunks = H >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);
  uint8_t* ring = lds + wave * R::bytes(S, cpw);
  uint8_t* stab = ring + S * R::kStage;  // [64 pairs][cpw dwords]; pair = matrix * 32 + row

  // scale table: dword f = pair * cpw + j holds blocks 4*(c0+j) .. +3 of that pair's row
  auto load_scales = [&]() {
    for (int f0 = 0; f0 < 64 * cpw; f0 += 64) {
      const int f = min(f0 + lane, 64 * cpw - 1);
      const int pair = f / cpw, j = f - pair * cpw;
      const int m = pair >> 5, n = min(n0 + (pair & 31), I - 1);
      const uint32_t off = (uint32_t)(n * (m == 0 ? gate.sr : up.sr)) + 4u * (c0 + j);
      // one descriptor per instruction: lanes of the other matrix are masked off by exec
      if (m == 0) dma4(sr[0], off, stab + f0 * 4);
      else dma4(sr[1], off, stab + f0 * 4);
    }
  };

  // Fill ring stage `stage` with chunk c.  Every step issues the same loads (past the end of the
  // wave's range it re-reads its last, L2-resident chunk into the free stage), so the vmcnt
  // bookkeeping is the same in every step.
  auto issue = [&](int stage, int c) {
    // the stage being refilled was read in an earlier step; its LDS reads have returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint8_t* st = ring + stage * R::kStage;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) dma16(wr[m], coff[m][rt] + 64u * c, st + (m * RT + rt) * 1024);
  };
  auto load_x = [&](int c, V (&dst)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[mt][s] = bitcast<V>(bld16(xr, xoff[mt] + 256u * c + 16u * s));
  };

  f32x4 accg[MT][RT], accu[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      accg[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // Per step: refill the stage freed by the previous step, wait for chunk c (its stage and the
  // activations loaded at the end of the previous step -- everything issued before this step's
  // DMAs), multiply, then load the next chunk's activations into the same registers.
  V xb[MT][4];
  if (c0 < c1) {
    load_scales();  // issued first: landed once the first chunk has
#pragma unroll
    for (int j = 0; j < S - 1; ++j) issue((c0 + j) % S, min(c0 + j, c1 - 1));
    load_x(c0, xb);
  }
  const uint32_t stab_a = lds_addr(stab);
  for (int c = c0; c < c1; ++c) {
    issue((c + S - 1) % S, min(c + S - 1, c1 - 1));
    wait_vmcnt<NM * RT>();
    const uint32_t st = lds_addr(ring + (c % S) * R::kStage);
    const uint32_t sc = stab_a + 4u * (c - c0) + lq;
    u32x4 qg[RT], qu[RT];
    uint32_t eg[RT], eu[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      qg[rt] = lds_read16(st + (0 * RT + rt) * 1024 + lane * 16);
      qu[rt] = lds_read16(st + (1 * RT + rt) * 1024 + lane * 16);
      eg[rt] = lds_read8(sc + 4u * cpw * (0 * 32 + rt * 16 + l16));
      eu[rt] = lds_read8(sc + 4u * cpw * (1 * 32 + rt * 16 + l16));
    }
    lds_sync<RT>(qg, eg);
    lds_sync<RT>(qu, eu);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float sg = e8m0_to_f32(eg[rt]), su = e8m0_to_f32(eu[rt]);
      // Padded rows (n >= I) and padded tokens read valid, finite data; an MFMA output element
      // depends only on its own row of A and column of B, so they only fill output rows and
      // columns that are never stored -- no zeroing is needed in the loop.
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const V ag = decode8_bf16(qg[rt][s], sg), au = decode8_bf16(qu[rt][s], su);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          accg[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, xb[mt][s], accg[mt][rt], 0, 0, 0);
          accu[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, xb[mt][s], accu[mt][rt], 0, 0, 0);
        }
      }
    }
    load_x(min(c + 1, c1 - 1), xb);
  }
  wait_vmcnt<0>();  // the last (re-read) DMAs have landed before the ring memory is reused

  // cross-wave reduction (reuses the ring memory once every wave has left its loop)
  float* red = reinterpret_cast<float*>(lds);  // [NW][RT][2][256]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    __syncthreads();
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

template <int NW, int MT, int S>
__global__ __launch_bounds__(NW * 64) void ffn_down_ring_kernel(
    const uint16_t* h_hi, const uint16_t* h_lo, int n_slots, int H, int I, ProjDev down,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int n_experts, int n_nblk,
    float* __restrict__ y_slots) {
  constexpr int RT = 4, NM = 1;
  typedef Ring<NM, RT> R;
  typedef bf16x8 V;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_info[4];
  int tile, nblk;
  xcd_work(blockIdx.x, n_nblk, tile, nblk);
  const TileInfo ti = find_tile(offsets, n_experts, n_slots, 16 * MT, tile, s_info);
  if (ti.nr <= 0) return;
  // wave index in an SGPR: the K-share loop bounds are then wave-uniform (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = nblk * 16 * RT;

  const int ex = __builtin_amdgcn_readfirstlane(ti.e);
  const __amdgpu_buffer_rsrc_t hr_hi = make_rsrc(h_hi, (int64_t)n_slots * I * 2);
  const __amdgpu_buffer_rsrc_t hr_lo = make_rsrc(h_lo, (int64_t)n_slots * I * 2);
  uint32_t hoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + l16;
    const int r = m < ti.nr ? ti.r0 + m : ti.r0;  // padded tokens read the tile's first row
    hoff[mt] = (uint32_t)r * (uint32_t)I * 2u + 64u * lq;
  }
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(down.w + (int64_t)ex * down.we, (int64_t)(H - 1) * down.wr + I / 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(down.s + (int64_t)ex * down.se, (int64_t)(H - 1) * down.sr + I / 32);
  uint32_t coff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) coff[rt] = (uint32_t)(min(n0 + rt * 16 + l16, H - 1) * down.wr) + 16u * lq;

  const int n_chunks = I >> 7;
  const int cpw = (n_chunks + NW - 1) / NW;
  const int c0 = wave * cpw, c1 = min(c0 + cpw, n_chunks);
  uint8_t* ring = lds + wave * R::bytes(S, cpw);
  uint8_t* stab = ring + S * R::kStage;  // [64 rows][cpw dwords]

  auto load_scales = [&]() {
    for (int f0 = 0; f0 < 64 * cpw; f0 += 64) {
      const int f = min(f0 + lane, 64 * cpw - 1);
      const int row = f / cpw, j = f - row * cpw;
      dma4(sr, (uint32_t)(min(n0 + row, H - 1) * down.sr) + 4u * (c0 + j), stab + f0 * 4);
    }
  };

  auto issue = [&](int stage, int c) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint8_t* st = ring + stage * R::kStage;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) dma16(wr, coff[rt] + 64u * c, st + rt * 1024);
  };
  auto load_h = [&](int c, V (&hi)[MT][4], V (&lo)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        hi[mt][s] = bitcast<V>(bld16(hr_hi, hoff[mt] + 256u * c + 16u * s));
        lo[mt][s] = bitcast<V>(bld16(hr_lo, hoff[mt] + 256u * c + 16u * s));
      }
  };

  f32x4 acc[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  V bh[MT][4], bl[MT][4];
  if (c0 < c1) {
    load_scales();
#pragma unroll
    for (int j = 0; j < S - 1; ++j) issue((c0 + j) % S, min(c0 + j, c1 - 1));
    load_h(c0, bh, bl);
  }
  const uint32_t stab_a = lds_addr(stab);
  for (int c = c0; c < c1; ++c) {
    issue((c + S - 1) % S, min(c + S - 1, c1 - 1));
    wait_vmcnt<RT>();
    const uint32_t st = lds_addr(ring + (c % S) * R::kStage);
    const uint32_t sc = stab_a + 4u * (c - c0) + lq;
    u32x4 q[RT];
    uint32_t e[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      q[rt] = lds_read16(st + rt * 1024 + lane * 16);
      e[rt] = lds_read8(sc + 4u * cpw * (rt * 16 + l16));
    }
    lds_sync<RT>(q, e);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float sc = e8m0_to_f32(e[rt]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const V a = decode8_bf16(q[rt][s], sc);  // padded rows / tokens: see the gate/up kernel
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[mt][s], acc[mt][rt], 0, 0, 0);
          acc[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[mt][s], acc[mt][rt], 0, 0, 0);
        }
      }
    }
    load_h(min(c + 1, c1 - 1), bh, bl);
  }
  wait_vmcnt<0>();

  float* red = reinterpret_cast<float*>(lds);  // [NW][RT][256]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    __syncthreads();
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

// Upper bound of the number of tiles: A active experts hold at least one row each, so
// sum_e ceil(n_e / R) <= A + (rows - A) / R with A <= min(n_experts, rows).
int64_t max_tiles(int64_t rows, int n_experts, int rows_per_tile) {
  const int64_t a = rows < n_experts ? rows : n_experts;
  return a + (rows - a) / rows_per_tile;
}

constexpr int kNW = 4, kRT1 = 2, kRT2 = 4;

// Tokens per tile from the mean rows per active expert (known on the host without a sync); both
// phases derive it from the same arguments, so they always agree on the tile numbering.
int pick_mt(int T, int k_total, int n_experts) {
  const int64_t rows = (int64_t)T * k_total;
  const int64_t active = rows < n_experts ? rows : n_experts;
  const double mean = (double)rows / (double)(active > 0 ? active : 1);
  return mean <= 16.0 ? 1 : (mean <= 32.0 ? 2 : 4);
}

constexpr int kRingStages = 3;

// Allows a kernel more than the default 64 KB of dynamic LDS (gfx950 has 160 KB per CU); done once
// per kernel and device.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  static int done_for_device[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (done_for_device[dev]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done_for_device[dev] = 1;
  return e;
}

inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
// The streaming kernels need whole 128-wide chunks and dword-aligned scale rows.
inline bool ring_ok(const ProjDev& p, int K) {
  return K % 128 == 0 && K <= 4 * 128 * Ring<1, 4>::kMaxChunksPerWave && al4(p.s) && p.se % 4 == 0 &&
         p.sr % 4 == 0;
}

template <int FMT, int MT>
hipError_t gateup_mt(const void* x, int T, int k_total, int n_experts, int H, int I, ProjDev gate, ProjDev up,
                     const int32_t* offsets, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                     hipStream_t stream) {
  const int64_t tiles = (max_tiles((int64_t)T * k_total, n_experts, 16 * MT) + kXcds - 1) / kXcds * kXcds;
  const int nb = (I + 16 * kRT1 - 1) / (16 * kRT1);
  const dim3 grid((unsigned)(tiles * nb));
  if (FMT == MOE_W_MXFP4 && ring_ok(gate, H) && ring_ok(up, H) && (int64_t)T * H * 2 < INT32_MAX &&
      (int64_t)I * gate.wr < INT32_MAX && (int64_t)I * up.wr < INT32_MAX) {
    const int cpw = (H / 128 + kNW - 1) / kNW;
    const size_t lds = (size_t)kNW * Ring<2, 2>::bytes(kRingStages, cpw);
    hipError_t e = allow_lds(ffn_gateup_ring_kernel<kNW, MT, kRingStages>, lds);
    if (e != hipSuccess) return e;
    ffn_gateup_ring_kernel<kNW, MT, kRingStages><<<grid, kNW * 64, lds, stream>>>(
        (const uint16_t*)x, T, k_total, H, I, gate, up, offsets, sorted_slot, n_experts, nb, h_hi, h_lo);
  } else {
    ffn_gateup_kernel<FMT, kNW, kRT1, MT><<<grid, kNW * 64, 0, stream>>>(
        (const uint16_t*)x, T, k_total, H, I, gate, up, offsets, sorted_slot, n_experts, nb, h_hi, h_lo);
  }
  return hipGetLastError();
}

template <int FMT, int MT>
hipError_t down_mt(int T, int k_total, int n_experts, int H, int I, ProjDev down, const int32_t* offsets,
                   const int32_t* sorted_slot, float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo,
                   hipStream_t stream) {
  const int n_slots = T * k_total;
  const int64_t tiles = (max_tiles(n_slots, n_experts, 16 * MT) + kXcds - 1) / kXcds * kXcds;
  const int nb = (H + 16 * kRT2 - 1) / (16 * kRT2);
  const dim3 grid((unsigned)(tiles * nb));
  if (FMT == MOE_W_MXFP4 && ring_ok(down, I) && (int64_t)n_slots * I * 2 < INT32_MAX &&
      (int64_t)H * down.wr < INT32_MAX) {
    const int cpw = (I / 128 + kNW - 1) / kNW;
    const size_t lds = (size_t)kNW * Ring<1, 4>::bytes(kRingStages, cpw);
    hipError_t e = allow_lds(ffn_down_ring_kernel<kNW, MT, kRingStages>, lds);
    if (e != hipSuccess) return e;
    ffn_down_ring_kernel<kNW, MT, kRingStages><<<grid, kNW * 64, lds, stream>>>(
        h_hi, h_lo, n_slots, H, I, down, offsets, sorted_slot, n_experts, nb, y_slots);
  } else {
    ffn_down_kernel<FMT, kNW, kRT2, MT><<<grid, kNW * 64, 0, stream>>>(h_hi, h_lo, n_slots, H, I, down, offsets,
                                                                      sorted_slot, n_experts, nb, y_slots);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t gateup_fmt(const void* x, int T, int k_total, int n_experts, int H, int I, ProjDev gate, ProjDev up,
                      const int32_t* offsets, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                      hipStream_t stream) {
  switch (pick_mt(T, k_total, n_experts)) {
    case 1: return gateup_mt<FMT, 1>(x, T, k_total, n_experts, H, I, gate, up, offsets, sorted_slot, h_hi, h_lo, stream);
    case 2: return gateup_mt<FMT, 2>(x, T, k_total, n_experts, H, I, gate, up, offsets, sorted_slot, h_hi, h_lo, stream);
    default: return gateup_mt<FMT, 4>(x, T, k_total, n_experts, H, I, gate, up, offsets, sorted_slot, h_hi, h_lo, stream);
  }
}

template <int FMT>
hipError_t down_fmt(int T, int k_total, int n_experts, int H, int I, ProjDev down, const int32_t* offsets,
                    const int32_t* sorted_slot, float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo,
                    hipStream_t stream) {
  switch (pick_mt(T, k_total, n_experts)) {
    case 1: return down_mt<FMT, 1>(T, k_total, n_experts, H, I, down, offsets, sorted_slot, y_slots, h_hi, h_lo, stream);
    case 2: return down_mt<FMT, 2>(T, k_total, n_experts, H, I, down, offsets, sorted_slot, y_slots, h_hi, h_lo, stream);
    default: return down_mt<FMT, 4>(T, k_total, n_experts, H, I, down, offsets, sorted_slot, y_slots, h_hi, h_lo, stream);
  }
}

}  // namespace

hipError_t launch_ffn_gateup(const void* x, int T, int k_total, int fmt, int n_experts, int H, int I, ProjDev gate,
                             ProjDev up, const int32_t* offsets, const int32_t* sorted_slot, uint16_t* h_hi,
                             uint16_t* h_lo, hipStream_t stream) {
  if (fmt == MOE_W_FP16)
    return gateup_fmt<MOE_W_FP16>(x, T, k_total, n_experts, H, I, gate, up, offsets, sorted_slot, h_hi, h_lo, stream);
  return gateup_fmt<MOE_W_MXFP4>(x, T, k_total, n_experts, H, I, gate, up, offsets, sorted_slot, h_hi, h_lo, stream);
}

hipError_t launch_ffn_down(int T, int k_total, int fmt, int n_experts, int H, int I, ProjDev down,
                           const int32_t* offsets, const int32_t* sorted_slot, float* y_slots, const uint16_t* h_hi,
                           const uint16_t* h_lo, hipStream_t stream) {
  if (fmt == MOE_W_FP16)
    return down_fmt<MOE_W_FP16>(T, k_total, n_experts, H, I, down, offsets, sorted_slot, y_slots, h_hi, h_lo, stream);
  return down_fmt<MOE_W_MXFP4>(T, k_total, n_experts, H, I, down, offsets, sorted_slot, y_slots, h_hi, h_lo, stream);
}

}  // namespace moe
