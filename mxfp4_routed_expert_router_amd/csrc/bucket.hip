// Bucketing: group the T*k slots by expert with a stable counting sort (Cascadia, Sec. 3.1: the
// fused path executes only the selected experts' work).
//
// Slots are processed in chunks of 512 (8 waves).  Within a wave, lanes holding the same expert
// id find each other with one ballot per id bit (an emulated match-any); the lane's rank among
// equal ids in lower lanes is a popcount.  Per-wave counts in LDS give the rank among equal ids in
// earlier waves of the chunk.  A chunk histogram plus a scan over chunks and buckets turns ranks
// into global positions.  No atomics are used, so the permutation is the unique stable one and is
// identical on every run.
//   up to 4 chunks : bucket_fused_kernel does rank + scan + scatter in one workgroup;
//   more chunks    : bucket_rank_kernel -> bucket_scan_kernel -> bucket_scatter_kernel.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
constexpr int kWaves = kBucketChunk / 64;

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
// [kWaves][n_buckets + 1].  Leaves wave_counts filled (per-wave counts of every key) and ends with
// a barrier.
__device__ SlotRank chunk_rank(int id, int n_slots, int n_buckets, int chunk, int* wave_counts) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int stride = n_buckets + 1;
  for (int i = tid; i < kWaves * stride; i += kBucketChunk) wave_counts[i] = 0;
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
__device__ int block_exclusive_scan(int* vals, int n, int* scratch /* kWaves + 1 ints */) {
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
    for (int w = 0; w < kWaves; ++w) {
      int v = scratch[w];
      scratch[w] = run;
      run += v;
    }
    scratch[kWaves] = run;
  }
  __syncthreads();
  int run = scratch[wave] + incl - local;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) {
      int v = vals[b0 + i];
      vals[b0 + i] = run;
      run += v;
    }
  const int total = scratch[kWaves];
  __syncthreads();
  return total;
}

// Up to kFusedChunks chunks in one workgroup: the chunks are ranked one after another (ranks and
// keys stay in registers, chunk histograms in LDS), then one scan and the scatter.  Saves the two
// extra launches of the multi-kernel path for decode-sized calls.
constexpr int kFusedChunks = 4;

__global__ __launch_bounds__(kBucketChunk) void bucket_fused_kernel(const int32_t* __restrict__ ids, int n_slots,
                                                                     int n_buckets, int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_slot,
                                                                     int32_t* __restrict__ slot_pos) {
  extern __shared__ int lds[];
  const int stride = n_buckets + 1;
  int* wave_counts = lds;                              // [kWaves][n_buckets+1]
  int* table = wave_counts + kWaves * stride;          // [kFusedChunks][n_buckets]: counts, then bases
  int* base = table + kFusedChunks * n_buckets;        // [n_buckets]
  int* scratch = base + n_buckets;                     // [kWaves+1]
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
        for (int w = 0; w < kWaves; ++w) v += wave_counts[w * stride + b];
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
}

// ws layout: rank [n_slots] | chunk table [n_chunks][n_buckets] (counts, then bases in place)
__global__ __launch_bounds__(kBucketChunk) void bucket_rank_kernel(const int32_t* __restrict__ ids, int n_slots,
                                                                    int n_buckets, int32_t* __restrict__ rank,
                                                                    int32_t* __restrict__ table) {
  extern __shared__ int lds[];
  const int chunk = blockIdx.x;
  SlotRank r = chunk_rank(chunk_id(ids, n_slots, chunk), n_slots, n_buckets, chunk, lds);
  const int s = chunk * kBucketChunk + threadIdx.x;
  if (s < n_slots) rank[s] = r.rank;
  for (int b = threadIdx.x; b < n_buckets; b += kBucketChunk) {
    int c = 0;
    for (int w = 0; w < kWaves; ++w) c += lds[w * (n_buckets + 1) + b];
    table[(int64_t)chunk * n_buckets + b] = c;
  }
}

__global__ __launch_bounds__(kBucketChunk) void bucket_scan_kernel(int n_chunks, int n_buckets,
                                                                    int32_t* __restrict__ table,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets) {
  extern __shared__ int lds[];
  int* tot = lds;                  // [n_buckets]
  int* scratch = lds + n_buckets;  // [kWaves+1]
  for (int b = threadIdx.x; b < n_buckets; b += kBucketChunk) {
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      int v = table[(int64_t)c * n_buckets + b];
      table[(int64_t)c * n_buckets + b] = run;
      run += v;
    }
    tot[b] = run;
    counts[b] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(tot, n_buckets, scratch);
  for (int b = threadIdx.x; b < n_buckets; b += kBucketChunk) offsets[b] = tot[b];
  if (threadIdx.x == 0) offsets[n_buckets] = total;
}

__global__ __launch_bounds__(kBucketChunk) void bucket_scatter_kernel(const int32_t* __restrict__ ids, int n_slots,
                                                                       int n_buckets, const int32_t* __restrict__ rank,
                                                                       const int32_t* __restrict__ table,
                                                                       const int32_t* __restrict__ offsets,
                                                                       int32_t* __restrict__ sorted_slot,
                                                                       int32_t* __restrict__ slot_pos) {
  const int s = blockIdx.x * kBucketChunk + threadIdx.x;
  if (s >= n_slots) return;
  const int chunk = blockIdx.x;
  int key = ids[s];
  const int total = offsets[n_buckets];
  if (key >= 0 && key < n_buckets) {
    const int pos = offsets[key] + table[(int64_t)chunk * n_buckets + key] + rank[s];
    sorted_slot[pos] = s;
    if (slot_pos) slot_pos[s] = pos;
  } else if (slot_pos) {
    slot_pos[s] = -1;
  }
  if (s >= total) sorted_slot[s] = -1;
}
}  // namespace

hipError_t launch_bucket(const int32_t* ids, int n_slots, int n_buckets, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_slot, int32_t* slot_pos, int32_t* ws, hipStream_t stream) {
  const int n_chunks = (n_slots + kBucketChunk - 1) / kBucketChunk;
  const size_t rank_lds = sizeof(int) * (size_t)kWaves * (n_buckets + 1);
  if (n_chunks <= kFusedChunks) {
    const size_t lds = rank_lds + sizeof(int) * ((size_t)(kFusedChunks + 1) * n_buckets + kWaves + 1);
    bucket_fused_kernel<<<1, kBucketChunk, lds, stream>>>(ids, n_slots, n_buckets, counts, offsets, sorted_slot,
                                                          slot_pos);
    return hipGetLastError();
  }
  int32_t* rank = ws;
  int32_t* table = ws + n_slots;
  bucket_rank_kernel<<<n_chunks, kBucketChunk, rank_lds, stream>>>(ids, n_slots, n_buckets, rank, table);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  bucket_scan_kernel<<<1, kBucketChunk, sizeof(int) * ((size_t)n_buckets + kWaves + 1), stream>>>(
      n_chunks, n_buckets, table, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  bucket_scatter_kernel<<<n_chunks, kBucketChunk, 0, stream>>>(ids, n_slots, n_buckets, rank, table, offsets,
                                                               sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
