// Host-side launchers of the gfx950 kernels (one per kernel family), called by the C ABI after it
// has validated every argument.  Each returns the launch status (hipGetLastError after enqueue).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---- router ----
int route_splits(int T, int H, int E);
// sigmoid: Cascadia's sigmoid router (bias on the selection only, weights routed_scale * s / sum s,
// shared slots shared_weight) instead of softmax -> top-k -> renormalise.
hipError_t launch_route(const void* x, int x_fp16, int T, int H, const float* w_router, const float* bias,
                        int E, int top_k, int n_shared, int32_t* ids, float* weights, float* probs,
                        float* partial, int splits, hipStream_t stream, bool sigmoid = false,
                        float routed_scale = 1.0f, float shared_weight = 1.0f);

// Router, bucketing and (table != NULL) the expert FFN's tile table in two launches (logits, then
// one workgroup that selects, buckets and plans), for the small calls route_bucket_fusable()
// accepts (at most 8 tokens).
bool route_bucket_fusable(int T, int k_total, int n_buckets);
hipError_t launch_route_bucket(const void* x, int x_fp16, int T, int H, const float* w_router, const float* bias,
                               int E, int top_k, int n_shared, int32_t* ids, float* weights, float* probs,
                               float* partial, int splits, int n_buckets, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slot, int32_t* slot_pos, void* table, int rows_per_tile,
                               int64_t n_entries, hipStream_t stream);

// ---- fixed row shapes: zero routing weights and invalid ids on rows past the device row count ----
hipError_t launch_pad_rows(const int32_t* n_rows, int T_shape, int k_total, int32_t* ids, float* weights,
                           hipStream_t stream);

// ---- streaming-read probe (a measurement utility) ----
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);

// ---- bucketing ----
constexpr int kBucketChunk = 512;
hipError_t launch_bucket(const int32_t* ids, int n_slots, int n_buckets, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_slot, int32_t* slot_pos, int32_t* ws, hipStream_t stream);
// Whether launch_bucket_plan builds the tile table inside the bucketing launch (one workgroup holds
// all of the slots); otherwise the caller runs the plan launch after it.
bool bucket_plans_inline(int n_slots);
// launch_bucket, and for bucket_plans_inline(n_slots) the expert FFN's tile table (n_entries
// entries of rows_per_tile rows, the entries of ffn_tiles_kernel) from the offsets it just built.
hipError_t launch_bucket_plan(const int32_t* ids, int n_slots, int n_buckets, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_slot, int32_t* slot_pos, int32_t* ws, void* table, int rows_per_tile,
                              int64_t n_entries, hipStream_t stream);

// ---- expert FFN ----
struct ProjDev {
  const uint8_t* w;
  const uint8_t* s;
  int64_t we, wr, se, sr;
  const uint8_t* z;  // INT4 group-32 zero points
  int64_t ze, zr;
  const float* ts;   // NVFP4 tensor scales [n_experts]
};
// Tile plan of one expert-FFN call: 16*mt sorted rows per tile, `tiles` entries in the tile table
// (an upper bound, padded to a multiple of the XCD count).
struct FfnPlan {
  int mt;   // token tiles of 16 per MFMA column block (the kernels' MT)
  int rpt;  // sorted rows (tokens) per tile: 16 * mt, or kTinyT for the tiny down kernel
  int64_t tiles;
  int n_experts;
  bool tile;  // the tile kernels (MXFP4, many rows per expert)
  bool tiny;  // the tiny down kernel (at most kTinyT tokens)
};
constexpr int kTinyT = 4;  // tokens of a call the tiny down kernel takes (at most kTinyT rows per tile)
// Kernel choices that depend on the weights description, as flags for ffn_plan: kPlanBig -- calls
// with many rows per expert may use the 128-token tile kernels (MXFP4 or FP16, whole 128-wide
// chunks, aligned scale rows, 32-bit offsets); kPlanTiny -- calls of at most kTinyT tokens may use
// the tiny down kernel (MXFP4, I a multiple of 512 up to 2048, H a multiple of 64, 16-byte
// aligned scale rows).  The
// FFN entry points and the workspace query must agree, so they all derive the flags from the same
// weights description.
constexpr int kPlanBig = 1, kPlanTiny = 2;
int ffn_plan_opts(int fmt, int T, int k_total, int H, int I, const ProjDev& gate, const ProjDev& up,
                  const ProjDev& down);
FfnPlan ffn_plan(int T, int k_total, int n_experts, int opts);
size_t ffn_table_bytes(int T, int k_total, int n_experts, int opts);
// The tile table of `rows_per_tile`-row tiles for the bucket offsets (entries up to n_entries).
hipError_t launch_ffn_tiles(const int32_t* offsets, int n_experts, int n_rows, int rows_per_tile, int64_t n_entries,
                            void* table, hipStream_t stream);
// The plan builds the tile table in `table`; the gate/up phase reads it and writes h; the down
// phase reads both.
hipError_t launch_ffn_plan(int T, int k_total, int n_experts, int opts, const int32_t* offsets, void* table,
                           hipStream_t stream);
hipError_t launch_ffn_gateup(const void* x, int T, int k_total, int fmt, int n_experts, int opts, int H, int I,
                             ProjDev gate, ProjDev up, const int32_t* sorted_slot, uint16_t* h_hi, uint16_t* h_lo,
                             const void* table, hipStream_t stream);
hipError_t launch_ffn_down(int T, int k_total, int fmt, int n_experts, int opts, int H, int I, ProjDev down,
                           const int32_t* sorted_slot, float* y_slots, const uint16_t* h_hi, const uint16_t* h_lo,
                           const void* table, hipStream_t stream);

// The range-managed FFN (Cascadia Sec. 3.3, Eq. 1): builds its own tile table (non-tile plan) in
// `table`, runs the general kernels with u attenuated by 2^-att_log2 and h rounded to binary16,
// and writes binary16 outputs to y16.
hipError_t launch_ffn_range(const void* x, int T, int k_total, int fmt, int n_experts, int H, int I, ProjDev gate,
                            ProjDev up, ProjDev down, const int32_t* offsets, const int32_t* sorted_slot,
                            uint16_t* h_hi, uint16_t* h_lo, void* table, int att_log2, uint16_t* y16,
                            hipStream_t stream);

// ---- expert FFN, MX mode (MXFP4 weights x MX-quantised activations on scaled MFMAs) ----
int mx_bits(int fmt);                                  // 8, 6 or 4 bits per code; 0 for an unknown format
int64_t mx_tiles(int T, int k_total, int n_experts);   // tile-table entries of an MX call
struct MxFfnArgs {
  int fmt;                                   // moe_mx_format
  const void* x;                             // [T][H] bf16
  int T, k_total, n_experts, H, I;
  ProjDev gate, up, down;
  const int32_t* offsets;
  const int32_t* sorted_slot;
  float* y_slots;
  uint8_t *xq, *xs;                          // x codes [T][H/32 blocks], scales [T][H/32]
  uint8_t *hq, *hs;                          // h codes [T*k_total][I/32 blocks], scales
  void* table;                               // tile table
};
// Quantises a contiguous [n_rows][K] bf16/fp16 matrix into packed codes + E8M0 scales.
hipError_t launch_mx_quantize(const void* x, bool x_fp16, int64_t n_rows, int K, int fmt, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);
// x quantisation, tile table, gate/up (writes h codes), down (writes y_slots).
hipError_t launch_ffn_mx(const MxFfnArgs& a, hipStream_t stream);

// ---- combine ----
hipError_t launch_combine(const float* y_slots, const float* weights, int T, int k_total, int H, float* y,
                          hipStream_t stream);
hipError_t launch_combine_restore(const uint16_t* y16, const float* weights, int T, int k_total, int H, int att_log2,
                                  float* y, hipStream_t stream);

// ---- decode primitive ----
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int n_rows, int K, int64_t code_stride,
                          int64_t scale_stride, uint16_t* out, hipStream_t stream);

}  // namespace moe
