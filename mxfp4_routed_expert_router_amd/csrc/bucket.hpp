// Device-side pieces of the bucketing (stable counting sort of slots by expert), shared by the
// bucketing kernels and the router's fused route + bucket path.  See bucket.hip for the method.
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

constexpr int kBucketWaves = kBucketChunk / 64;

struct SlotRank {
  int key;   // expert id, or n_buckets for a dropped slot, or -1 past the end
  int rank;  // number of earlier slots in the chunk with the same key
};

// This thread's id in chunk `chunk` (read before ranking, so that a workgroup ranking several
// chunks issues all of their reads together), or -1 past the end.
__device__ __forceinline__ int chunk_id(const int32_t* __restrict__ ids, int n_slots, int chunk) {
  const int s = chunk * kBucketChunk + threadIdx.x;
  return s < n_slots ? ids[s] : -1;
}

// Rank of this thread's slot within its chunk, given its id from chunk_id.  wave_counts: LDS
// [kBucketWaves][n_buckets + 1].  Leaves wave_counts filled (per-wave counts of every key) and ends with
// a barrier.
__device__ inline SlotRank chunk_rank(int id, int n_slots, int n_buckets, int chunk, int* wave_counts) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int stride = n_buckets + 1;
  for (int i = tid; i < kBucketWaves * stride; i += kBucketChunk) wave_counts[i] = 0;
  const int s = chunk * kBucketChunk + tid;
  const bool in = s < n_slots;
  int key = -1;
  if (in) {
    key = id;
    if (key < 0 || key >= n_buckets) key = n_buckets;
  }
  uint64_t same = __ballot(in);
  const int nbits = 32 - __clz(n_buckets);  // bits to tell keys 0..n_buckets apart
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(in && bit);
    same &= bit ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_in_wave = __popcll(same & below);
  __syncthreads();  // zero-fill of wave_counts complete
  if (in && rank_in_wave == 0) wave_counts[wave * stride + key] = __popcll(same);
  __syncthreads();
  int before = 0;
  if (in)
    for (int w = 0; w < wave; ++w) before += wave_counts[w * stride + key];
  SlotRank r;
  r.key = in ? key : -1;
  r.rank = before + rank_in_wave;
  return r;
}

// Exclusive scan of vals[0..n) in LDS in place (n <= 4 * kBucketChunk); returns the total.
__device__ inline int block_exclusive_scan(int* vals, int n, int* scratch /* kBucketWaves + 1 ints */) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (n + kBucketChunk - 1) / kBucketChunk;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) local += vals[b0 + i];
  const int incl = wave_incl_scan(local);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kBucketWaves; ++w) {
      int v = scratch[w];
      scratch[w] = run;
      run += v;
    }
    scratch[kBucketWaves] = run;
  }
  __syncthreads();
  int run = scratch[wave] + incl - local;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) {
      int v = vals[b0 + i];
      vals[b0 + i] = run;
      run += v;
    }
  const int total = scratch[kBucketWaves];
  __syncthreads();
  return total;
}

// Up to kFusedChunks chunks in one workgroup: the chunks are ranked one after another (ranks and
// keys stay in registers, chunk histograms in LDS), then one scan and the scatter.  Saves the two
// extra launches of the multi-kernel path for decode-sized calls.
constexpr int kFusedChunks = 4;

// LDS ints the fused bucketing of one workgroup needs.
__host__ __device__ constexpr size_t bucket_fused_lds_ints(int n_buckets) {
  return (size_t)kBucketWaves * (n_buckets + 1) + (size_t)(kFusedChunks + 1) * n_buckets + kBucketWaves + 1;
}

// The whole bucketing of up to kFusedChunks chunks by one workgroup of kBucketChunk threads.
// lds: bucket_fused_lds_ints(n_buckets) ints.  On return (after a barrier) lds_base() holds the
// exclusive offsets of the buckets and the return value is the number of valid slots.
__device__ __forceinline__ int* fused_base(int* lds, int n_buckets) {
  return lds + kBucketWaves * (n_buckets + 1) + kFusedChunks * n_buckets;
}
__device__ inline int bucket_fused_block(const int32_t* __restrict__ ids, int n_slots, int n_buckets,
                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos, int* lds) {
  const int stride = n_buckets + 1;
  int* wave_counts = lds;                              // [kBucketWaves][n_buckets+1]
  int* table = wave_counts + kBucketWaves * stride;          // [kFusedChunks][n_buckets]: counts, then bases
  int* base = table + kFusedChunks * n_buckets;        // [n_buckets]
  int* scratch = base + n_buckets;                     // [kBucketWaves+1]
  const int tid = threadIdx.x;
  const int n_chunks = (n_slots + kBucketChunk - 1) / kBucketChunk;  // 1 .. kFusedChunks
  int id[kFusedChunks];
#pragma unroll
  for (int c = 0; c < kFusedChunks; ++c) id[c] = chunk_id(ids, n_slots, c);
  SlotRank r[kFusedChunks];
#pragma unroll
  for (int c = 0; c < kFusedChunks; ++c) {
    r[c].key = -1;
    r[c].rank = 0;
    if (c < n_chunks) {  // uniform
      r[c] = chunk_rank(id[c], n_slots, n_buckets, c, wave_counts);
      for (int b = tid; b < n_buckets; b += kBucketChunk) {
        int v = 0;
        for (int w = 0; w < kBucketWaves; ++w) v += wave_counts[w * stride + b];
        table[c * n_buckets + b] = v;
      }
      __syncthreads();  // the next chunk's ranking clears wave_counts
    }
  }
  for (int b = tid; b < n_buckets; b += kBucketChunk) {
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int v = table[c * n_buckets + b];
      table[c * n_buckets + b] = run;
      run += v;
    }
    base[b] = run;
    counts[b] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(base, n_buckets, scratch);
  for (int b = tid; b < n_buckets; b += kBucketChunk) offsets[b] = base[b];
  if (tid == 0) offsets[n_buckets] = total;
#pragma unroll
  for (int c = 0; c < kFusedChunks; ++c) {
    const int s = c * kBucketChunk + tid;
    if (r[c].key >= 0) {
      if (r[c].key < n_buckets) {
        const int pos = base[r[c].key] + table[c * n_buckets + r[c].key] + r[c].rank;
        sorted_slot[pos] = s;
        if (slot_pos) slot_pos[s] = pos;
      } else if (slot_pos) {
        slot_pos[s] = -1;
      }
    }
    if (s < n_slots && s >= total) sorted_slot[s] = -1;
  }
  return total;
}

// Calls of at most kSmallSlots slots, ids already in LDS: the bucketing and the tile table without
// histograms, with work that does not grow with the slot count.  Slot s (key k_s: its expert, or
// n_buckets when dropped) goes to position #{j : (k_j, j) < (k_s, s)}, the stable counting sort of
// the general path; the eight waves count over eight slots each and wave 0 adds the parts.  The
// keys in sorted order then give everything else: wave 0 walks the sorted positions (an expert's
// first row is where the key changes, a ballot finds the next such row, a DPP scan of the tile
// counts places each expert's tiles, in expert order as in tiles_from_offsets_block), and every
// bucket b takes offset = #{keys < b} and count = #{keys < b + 1} - offset by binary search.
// sids: the n_slots ids in LDS; tmp: kSmallLdsInts ints of LDS.  Workgroup of kBucketChunk threads.
constexpr int kSmallSlots = 64;
constexpr int kSmallLdsInts = kBucketWaves * kSmallSlots + kSmallSlots;
static_assert(kBucketWaves * 8 >= kSmallSlots, "eight slots per wave cover the small calls");
__device__ inline void bucket_small_block(const int* sids, int n_slots, int n_buckets, int32_t* __restrict__ counts,
                                          int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                                          int32_t* __restrict__ slot_pos, TileEntry* __restrict__ table,
                                          int rows_per_tile, int n_entries, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* part = tmp;                          // [kBucketWaves][64] partial positions
  int* sk = tmp + kBucketWaves * kSmallSlots;  // [64] keys in sorted order
  auto key = [&](int j) {
    const int id = sids[j];
    return (id < 0 || id >= n_buckets) ? n_buckets : id;
  };
  if (8 * wave < n_slots) {  // uniform
    const int ks = lane < n_slots ? key(lane) : n_buckets;
    int r = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * wave + jj;
      if (j < n_slots) {  // uniform
        const int kj = key(j);
        r += (kj < ks) | ((kj == ks) & (j < lane));
      }
    }
    part[wave * kSmallSlots + lane] = r;
  }
  __syncthreads();
  if (wave == 0) {
    const bool in = lane < n_slots;
    const int ks = in ? key(lane) : n_buckets;
    int pos = 0;
#pragma unroll
    for (int w = 0; w < kBucketWaves; ++w)
      if (8 * w < n_slots) pos += part[w * kSmallSlots + lane];  // uniform condition
    const bool valid = in && ks < n_buckets;
    const int total = __popcll(__ballot(valid));
    if (valid) {
      sorted_slot[pos] = lane;
      if (slot_pos) slot_pos[lane] = pos;
    } else if (in && slot_pos) {
      slot_pos[lane] = -1;
    }
    if (lane >= total && in) sorted_slot[lane] = -1;
    if (lane == 0) offsets[n_buckets] = total;
    if (in) sk[pos] = ks;  // pos runs over 0 .. n_slots - 1, dropped slots after the valid ones
    if (table) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bool row = lane < total;  // sorted position `lane` holds a valid row
      const int kp = row ? sk[lane] : 0;
      const bool first = row && (lane == 0 || sk[lane - 1] != kp);
      const uint64_t fm = __ballot(first);
      const uint64_t later = lane == 63 ? 0ull : fm & (~0ull << (lane + 1));
      const int next = later ? __builtin_ctzll(later) : total;
      const int cnt = next - lane;  // rows of expert kp (at its first row)
      const int ntl = first ? (cnt + rows_per_tile - 1) / rows_per_tile : 0;
      const int incl = (int)wave_incl_scan_dpp((uint32_t)ntl);
      const int all_tiles = __builtin_amdgcn_readlane(incl, 63);
      for (int q = 0; q < ntl && incl - ntl + q < n_entries; ++q)
        table[incl - ntl + q] = TileEntry{kp, lane + q * rows_per_tile, min(rows_per_tile, cnt - q * rows_per_tile), 0};
      for (int t = all_tiles + lane; t < n_entries; t += 64) table[t] = TileEntry{0, 0, 0, 0};
    }
  }
  __syncthreads();  // sk complete
  for (int b = tid; b < n_buckets; b += blockDim.x) {
    int lo = 0, hi = 0;  // #{keys < b}, #{keys < b + 1}
#pragma unroll
    for (int step = kSmallSlots; step > 0; step >>= 1) {
      if (lo + step <= n_slots && sk[lo + step - 1] < b) lo += step;
      if (hi + step <= n_slots && sk[hi + step - 1] <= b) hi += step;
    }
    counts[b] = hi - lo;
    offsets[b] = lo;
  }
}

}  // namespace moe

