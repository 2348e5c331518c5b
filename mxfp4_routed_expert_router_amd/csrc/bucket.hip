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
#include "bucket.hpp"
#include "tiles.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(kBucketChunk) void bucket_fused_kernel(const int32_t* __restrict__ ids, int n_slots,
                                                                     int n_buckets, int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_slot,
                                                                     int32_t* __restrict__ slot_pos) {
  extern __shared__ int lds[];
  bucket_fused_block(ids, n_slots, n_buckets, counts, offsets, sorted_slot, slot_pos, lds);
}

// bucket_fused_kernel followed, in the same workgroup, by the expert FFN's tile table built from the
// offsets it leaves in LDS (saves the plan launch).
__global__ __launch_bounds__(kBucketChunk) void bucket_fused_plan_kernel(
    const int32_t* __restrict__ ids, int n_slots, int n_buckets, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos,
    TileEntry* __restrict__ table, int rows_per_tile, int n_entries) {
  extern __shared__ int lds[];
  const int total = bucket_fused_block(ids, n_slots, n_buckets, counts, offsets, sorted_slot, slot_pos, lds);
  tiles_from_offsets_block(fused_base(lds, n_buckets), total, n_buckets, n_slots, rows_per_tile, n_entries, table,
                           lds);
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
    for (int w = 0; w < kBucketWaves; ++w) c += lds[w * (n_buckets + 1) + b];
    table[(int64_t)chunk * n_buckets + b] = c;
  }
}

__global__ __launch_bounds__(kBucketChunk) void bucket_scan_kernel(int n_chunks, int n_buckets,
                                                                    int32_t* __restrict__ table,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets) {
  extern __shared__ int lds[];
  int* tot = lds;                  // [n_buckets]
  int* scratch = lds + n_buckets;  // [kBucketWaves+1]
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
  const size_t rank_lds = sizeof(int) * (size_t)kBucketWaves * (n_buckets + 1);
  if (n_chunks <= kFusedChunks) {
    const size_t lds = sizeof(int) * bucket_fused_lds_ints(n_buckets);
    bucket_fused_kernel<<<1, kBucketChunk, lds, stream>>>(ids, n_slots, n_buckets, counts, offsets, sorted_slot,
                                                          slot_pos);
    return hipGetLastError();
  }
  int32_t* rank = ws;
  int32_t* table = ws + n_slots;
  bucket_rank_kernel<<<n_chunks, kBucketChunk, rank_lds, stream>>>(ids, n_slots, n_buckets, rank, table);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  bucket_scan_kernel<<<1, kBucketChunk, sizeof(int) * ((size_t)n_buckets + kBucketWaves + 1), stream>>>(
      n_chunks, n_buckets, table, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  bucket_scatter_kernel<<<n_chunks, kBucketChunk, 0, stream>>>(ids, n_slots, n_buckets, rank, table, offsets,
                                                               sorted_slot, slot_pos);
  return hipGetLastError();
}

static_assert(2 * kBucketChunk >= MOE_MAX_EXPERTS, "tiles_from_offsets_block covers two experts per thread");
bool bucket_plans_inline(int n_slots) { return (n_slots + kBucketChunk - 1) / kBucketChunk <= kFusedChunks; }

hipError_t launch_bucket_plan(const int32_t* ids, int n_slots, int n_buckets, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_slot, int32_t* slot_pos, int32_t* ws, void* table, int rows_per_tile,
                              int64_t n_entries, hipStream_t stream) {
  if (!bucket_plans_inline(n_slots))
    return launch_bucket(ids, n_slots, n_buckets, counts, offsets, sorted_slot, slot_pos, ws, stream);
  const size_t lds = sizeof(int) * bucket_fused_lds_ints(n_buckets);
  bucket_fused_plan_kernel<<<1, kBucketChunk, lds, stream>>>(ids, n_slots, n_buckets, counts, offsets, sorted_slot,
                                                             slot_pos, (TileEntry*)table, rows_per_tile,
                                                             (int)n_entries);
  return hipGetLastError();
}

}  // namespace moe
