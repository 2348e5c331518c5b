// Tile schedule shared by the expert-FFN kernels, and the buffer-load helpers they use.
#pragma once
#include "common.hpp"

namespace moe {

struct TileInfo {
  int e, r0, nr;  // expert, first sorted row, rows in this tile (0 => no tile)
};

// Tile table, built once per expert-FFN call by ffn_tiles_kernel: entry t = (expert, first sorted
// row, rows) of tile t, tiles numbered expert by expert (an expert with n rows owns
// ceil(n / rows_per_tile) consecutive tiles); entries from the tile count up to the grid's bound
// hold rows = 0.  The gate/up and down phases read the same table.
struct TileEntry {
  int e, r0, nr, pad;
};

// Entry `tile`, checked against the launch: an entry naming an expert outside [0, n_experts), more
// than max_rows rows or rows outside [0, n_rows) (a table not built for this call) reads as empty,
// so the kernels never index outside their buffers.
__device__ __forceinline__ TileInfo get_tile(const TileEntry* __restrict__ table, int tile, int n_experts, int n_rows,
                                             int max_rows) {
  const TileEntry t = table[tile];
  TileInfo r;
  r.e = __builtin_amdgcn_readfirstlane(t.e);
  r.r0 = __builtin_amdgcn_readfirstlane(t.r0);
  r.nr = __builtin_amdgcn_readfirstlane(t.nr);
  if (r.e < 0 || r.e >= n_experts || r.r0 < 0 || r.nr > max_rows || r.r0 > n_rows - r.nr) r.nr = 0;
  return r;
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

// Work item of workgroup b in a grouped schedule: items are numbered tile-major (item = tile * n_nblk
// + nblk) and cut into chunks of `chunk` consecutive items, chunk c running on XCD c % 8.  With
// `chunk` = the workgroups one XCD holds at once, the workgroups of a chunk are dispatched together
// and stay in step, so that they share in that XCD's L2 the activation rows of their tiles (all
// n-blocks of a tile are in one chunk when n_nblk divides it) and the weight slices of the tiles of
// one expert -- instead of each n-block fetching every tile's activations into its own XCD.  The
// grid holds a multiple of 8 * chunk workgroups, which makes the map a permutation.
constexpr int kCusPerXcd = 32;
__device__ __forceinline__ int grouped_item(int b, int chunk) {
  const int xcd = b % kXcds, q = b / kXcds;
  return ((q / chunk) * kXcds + xcd) * chunk + q % chunk;
}

// The tile table built by one workgroup from bucket offsets held in LDS (off[e] = first sorted row
// of expert e, e < n_experts; `total` = valid rows), with the same entries as ffn_tiles_kernel:
// each expert's ceil(n_e / rows_per_tile) tiles in expert order, then empty entries up to
// n_entries.  scratch: (blockDim / 64 + 1) ints of LDS; ends with a barrier.
__device__ inline void tiles_from_offsets_block(const int* off, int total, int n_experts, int n_rows_max,
                                                int rows_per_tile, int n_entries, TileEntry* __restrict__ table,
                                                int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int per = (n_experts + blockDim.x - 1) / blockDim.x;  // consecutive experts per thread (<= 2)
  const int e0 = tid * per;
  int a[2] = {0, 0}, n[2] = {0, 0}, cnt[2] = {0, 0}, mine = 0;
  for (int i = 0; i < per && i < 2; ++i) {
    const int e = e0 + i;
    if (e < n_experts) {
      a[i] = min(max(off[e], 0), n_rows_max);
      const int b = min(max(e + 1 < n_experts ? off[e + 1] : total, 0), n_rows_max);
      n[i] = max(b - a[i], 0);
      cnt[i] = (n[i] + rows_per_tile - 1) / rows_per_tile;
      mine += cnt[i];
    }
  }
  const int incl = wave_incl_scan(mine);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int v = scratch[w];
      scratch[w] = run;
      run += v;
    }
    scratch[nwaves] = run;
  }
  __syncthreads();
  int first = scratch[wave] + incl - mine;
  for (int i = 0; i < per && i < 2; ++i) {
    for (int p = 0; p < cnt[i] && first + p < n_entries; ++p) {
      const int r0 = a[i] + p * rows_per_tile;
      table[first + p] = TileEntry{e0 + i, r0, min(rows_per_tile, a[i] + n[i] - r0), 0};
    }
    first += cnt[i];
  }
  for (int t = scratch[nwaves] + tid; t < n_entries; t += blockDim.x) table[t] = TileEntry{0, 0, 0, 0};
  __syncthreads();
}

// Upper bound of the number of tiles: A active experts hold at least one row each, so
// sum_e ceil(n_e / R) <= A + (rows - A) / R with A <= min(n_experts, rows).
inline int64_t max_tiles(int64_t rows, int n_experts, int rows_per_tile) {
  const int64_t a = rows < n_experts ? rows : n_experts;
  return a + (rows - a) / rows_per_tile;
}

// MUBUF buffer loads: a descriptor bounds every access, and a load past its range returns zeros
// without touching memory.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufferFlags);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// With a wave-uniform offset part in an SGPR (added to the per-lane offset).
// A 16-byte buffer load with the nontemporal hint (streamed data, read once): with whole 128-byte
// lines per instruction (8 lanes per row) it reads HBM about 10% faster than plain loads; with
// partial lines it is slower.
__device__ __forceinline__ u32x4 bld16nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ u32x4 bld16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ uint32_t bld4s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}

// A buffer offset past every descriptor range (ranges are < 2^31; offsets added to it stay < 2^32).
constexpr uint32_t kOutOfRange = 0x80000000u;

}  // namespace moe
