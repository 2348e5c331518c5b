// The C ABI (include/moe.h): synchronous host-side validation, then asynchronous launches on the
// caller's stream.  Nothing here allocates, synchronises or reads device memory.
#include <limits.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "launch.hpp"

namespace {

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
inline bool known_format(int f) {
  return f == MOE_W_MXFP4 || f == MOE_W_FP16 || f == MOE_W_INT4_G32 || f == MOE_W_NVFP4;
}

// Checks of one projection; K is its reduction dimension.
moe_status check_proj(const moe_proj& p, moe_w_format fmt, int n_experts, int N, int K) {
  if (!p.w) return MOE_ERR_NULL;
  if (fmt == MOE_W_INT4_G32 || fmt == MOE_W_NVFP4) {
    // 16 code bytes are one INT4 group or two NVFP4 blocks: a base or stride off that grid starts
    // inside one, and the group and block scales are sliced with the codes
    if (!p.scales || (fmt == MOE_W_INT4_G32 && !p.zeros) || (fmt == MOE_W_NVFP4 && !p.tensor_scale))
      return MOE_ERR_NULL;
    if (K % 32 != 0) return MOE_ERR_BLOCK;
    const int64_t srow = fmt == MOE_W_INT4_G32 ? 2 * (K / 32) : K / 16;
    if (p.w_row_stride < K / 2 || p.s_row_stride < srow || p.w_expert_stride < 0 || p.s_expert_stride < 0)
      return MOE_ERR_SHAPE;
    if (fmt == MOE_W_INT4_G32 && (p.z_row_stride < (K / 32 + 1) / 2 || p.z_expert_stride < 0)) return MOE_ERR_SHAPE;
    if (!al16(p.w) || p.w_row_stride % 16 != 0 || p.w_expert_stride % 16 != 0) return MOE_ERR_BLOCK;
    if (fmt == MOE_W_NVFP4 && !al4(p.tensor_scale)) return MOE_ERR_ALIGN;
    (void)n_experts;
    (void)N;
    return MOE_OK;
  }
  if (fmt == MOE_W_MXFP4) {
    if (!p.scales) return MOE_ERR_NULL;
    if (K % 32 != 0) return MOE_ERR_BLOCK;
    if (p.w_row_stride < K / 2 || p.s_row_stride < K / 32 || p.w_expert_stride < 0 || p.s_expert_stride < 0)
      return MOE_ERR_SHAPE;
  } else {
    if (p.scales) return MOE_ERR_DTYPE;
    if (K % 32 != 0) return MOE_ERR_SHAPE;
    if (p.w_row_stride < 2 * (int64_t)K || p.w_expert_stride < 0) return MOE_ERR_SHAPE;
  }
  // A 16-byte step of packed MXFP4 codes is exactly one 32-value block, so a base or stride off that
  // grid starts a slice inside a block (FreeToken DeepSeek-V4-Flash post, "Why it would not run":
  // such partitions are refused).  For FP16 weights the same rule is only the 128-bit load alignment.
  if (!al16(p.w) || p.w_row_stride % 16 != 0 || p.w_expert_stride % 16 != 0)
    return fmt == MOE_W_MXFP4 ? MOE_ERR_BLOCK : MOE_ERR_ALIGN;
  (void)n_experts;
  (void)N;
  return MOE_OK;
}

moe::ProjDev dev(const moe_proj& p);
// The FFN's kernel-choice flags, derived from the weights description alone (see ffn_plan_opts).
int plan_opts(const moe_expert_weights* W, int T, int k_total) {
  return moe::ffn_plan_opts(W->fmt, T, k_total, W->hidden, W->inter, dev(W->gate), dev(W->up), dev(W->down));
}

moe::ProjDev dev(const moe_proj& p) {
  moe::ProjDev d;
  d.w = (const uint8_t*)p.w;
  d.s = p.scales;
  d.we = p.w_expert_stride;
  d.wr = p.w_row_stride;
  d.se = p.s_expert_stride;
  d.sr = p.s_row_stride;
  d.z = p.zeros;
  d.ze = p.z_expert_stride;
  d.zr = p.z_row_stride;
  d.ts = p.tensor_scale;
  return d;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid size or shape";
    case MOE_ERR_BLOCK: return "MXFP4 dimension or slice cuts a 32-value block";
    case MOE_ERR_ALIGN: return "pointer or stride not aligned";
    case MOE_ERR_DTYPE: return "unsupported dtype or format combination";
    case MOE_ERR_TOPK: return "invalid top_k";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "kernel launch failed";
  }
  return "unknown status";
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

// ---------------------------------------------------------------------------------------------
size_t moe_route_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  const int s = moe::route_splits(T, H, E);
  return round_up(sizeof(float) * (size_t)s * (size_t)T * (size_t)E, 256);
}

moe_status moe_route(const void* x, moe_act_dtype x_dtype, int T, int H, const float* w_router,
                     const float* logit_bias, int E, int top_k, int n_shared, int32_t* ids, float* weights,
                     float* probs, void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS || n_shared < 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16) return MOE_ERR_DTYPE;
  if (top_k < 1 || top_k > E || top_k + n_shared > MOE_MAX_SLOTS_PER_TOKEN) return MOE_ERR_TOPK;
  if (!x || !w_router || !ids || !weights) return MOE_ERR_NULL;
  if ((int64_t)T * (top_k + n_shared) > INT_MAX || (int64_t)T * E > INT_MAX) return MOE_ERR_SHAPE;
  if (!al16(x) || !al4(w_router) || !al4(ids) || !al4(weights) || (probs && !al4(probs)) ||
      (logit_bias && !al4(logit_bias)))
    return MOE_ERR_ALIGN;
  const size_t need = moe_route_workspace_bytes(T, H, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_route(x, x_dtype == MOE_ACT_FP16, T, H, w_router, logit_bias, E, top_k, n_shared,
                                      ids, weights, probs, (float*)workspace, moe::route_splits(T, H, E),
                                      (hipStream_t)stream));
}

moe_status moe_route_sigmoid(const void* x, moe_act_dtype x_dtype, int T, int H, const float* w_router,
                             const float* selection_bias, int E, int top_k, int n_shared, float routed_scale,
                             float shared_weight, int32_t* ids, float* weights, float* scores, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS || n_shared < 0) return MOE_ERR_SHAPE;
  if (!(routed_scale - routed_scale == 0.0f) || !(shared_weight - shared_weight == 0.0f)) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16) return MOE_ERR_DTYPE;
  if (top_k < 1 || top_k > E || top_k + n_shared > MOE_MAX_SLOTS_PER_TOKEN) return MOE_ERR_TOPK;
  if (!x || !w_router || !ids || !weights) return MOE_ERR_NULL;
  if ((int64_t)T * (top_k + n_shared) > INT_MAX || (int64_t)T * E > INT_MAX) return MOE_ERR_SHAPE;
  if (!al16(x) || !al4(w_router) || !al4(ids) || !al4(weights) || (scores && !al4(scores)) ||
      (selection_bias && !al4(selection_bias)))
    return MOE_ERR_ALIGN;
  const size_t need = moe_route_workspace_bytes(T, H, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_route(x, x_dtype == MOE_ACT_FP16, T, H, w_router, selection_bias, E, top_k,
                                      n_shared, ids, weights, scores, (float*)workspace,
                                      moe::route_splits(T, H, E), (hipStream_t)stream, true, routed_scale,
                                      shared_weight));
}

// ---------------------------------------------------------------------------------------------
int moe_row_shape(int T, const int* shapes, int n_shapes) {
  if (T < 0 || !shapes || n_shapes < 1) return -1;
  int best = -1;
  for (int i = 0; i < n_shapes; ++i)
    if (shapes[i] >= T && shapes[i] > 0 && (best < 0 || shapes[i] < best)) best = shapes[i];
  return best;
}

moe_status moe_pad_rows(const int32_t* n_rows, int T_shape, int k_total, int32_t* ids, float* weights,
                        void* stream) {
  if (T_shape == 0) return MOE_OK;
  if (T_shape < 0 || k_total < 1 || k_total > MOE_MAX_SLOTS_PER_TOKEN || (int64_t)T_shape * k_total > INT_MAX)
    return MOE_ERR_SHAPE;
  if (!n_rows || !ids || !weights) return MOE_ERR_NULL;
  if (!al4(n_rows) || !al4(ids) || !al4(weights)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_pad_rows(n_rows, T_shape, k_total, ids, weights, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
size_t moe_bucket_workspace_bytes(int n_slots, int n_buckets) {
  if (n_slots <= moe::kBucketChunk || n_buckets <= 0) return 0;
  const size_t chunks = (size_t)(n_slots + moe::kBucketChunk - 1) / moe::kBucketChunk;
  return round_up(sizeof(int32_t) * ((size_t)n_slots + chunks * (size_t)n_buckets), 256);
}

moe_status moe_bucket(const int32_t* ids, int n_slots, int n_buckets, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_slot, int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (n_slots == 0) return MOE_OK;
  if (n_slots < 0 || n_buckets < 1 || n_buckets > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (!ids || !counts || !offsets || !sorted_slot) return MOE_ERR_NULL;
  if (!al4(ids) || !al4(counts) || !al4(offsets) || !al4(sorted_slot) || (slot_pos && !al4(slot_pos)))
    return MOE_ERR_ALIGN;
  const size_t need = moe_bucket_workspace_bytes(n_slots, n_buckets);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_bucket(ids, n_slots, n_buckets, counts, offsets, sorted_slot, slot_pos,
                                       (int32_t*)workspace, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
size_t moe_expert_ffn_workspace_bytes(int T, int k_total, const moe_expert_weights* W) {
  if (!W || T <= 0 || k_total <= 0 || W->inter <= 0 || W->n_experts <= 0) return 0;
  // h as a high plane and a low plane of 16-bit values, one row of `inter` per sorted slot,
  // then the tile table shared by the two phases
  const size_t plane = round_up(sizeof(uint16_t) * (size_t)T * (size_t)k_total * (size_t)W->inter, 256);
  return 2 * plane + round_up(moe::ffn_table_bytes(T, k_total, W->n_experts, plan_opts(W, T, k_total)), 256);
}

}  // extern "C"

namespace {

// Validation shared by moe_expert_ffn and its two phases.  On success h_hi / h_lo point into the
// workspace.
moe_status check_ffn(const void* x, moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                     const int32_t* offsets, const int32_t* sorted_slot, const float* y_slots, bool need_x,
                     bool need_y, void* workspace, size_t workspace_bytes, uint16_t** h_hi, uint16_t** h_lo,
                     void** table) {
  if (!W) return MOE_ERR_NULL;
  if (T < 0 || k_total < 1 || k_total > MOE_MAX_SLOTS_PER_TOKEN) return MOE_ERR_SHAPE;
  if (!known_format(W->fmt)) return MOE_ERR_DTYPE;
  if (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16) return MOE_ERR_DTYPE;
  if (W->n_experts < 1 || W->n_experts > MOE_MAX_EXPERTS || W->hidden < 1 || W->inter < 1) return MOE_ERR_SHAPE;
  if ((int64_t)T * k_total > INT_MAX) return MOE_ERR_SHAPE;
  if ((W->fmt != MOE_W_FP16) != (x_dtype == MOE_ACT_BF16)) return MOE_ERR_DTYPE;
  if ((need_x && !x) || !offsets || !sorted_slot || (need_y && !y_slots)) return MOE_ERR_NULL;
  const int H = W->hidden, I = W->inter;
  moe_status st;
  if (need_x) {
    if ((st = check_proj(W->gate, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
    if ((st = check_proj(W->up, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
  }
  if (need_y) {
    if ((st = check_proj(W->down, W->fmt, W->n_experts, H, I)) != MOE_OK) return st;
  }
  if ((need_x && !al16(x)) || (need_y && !al16(y_slots)) || !al4(offsets) || !al4(sorted_slot))
    return MOE_ERR_ALIGN;
  const size_t need = moe_expert_ffn_workspace_bytes(T, k_total, W);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  const size_t plane = round_up(sizeof(uint16_t) * (size_t)T * (size_t)k_total * (size_t)W->inter, 256);
  *h_hi = (uint16_t*)workspace;
  *h_lo = (uint16_t*)((uint8_t*)workspace + plane);
  *table = (uint8_t*)workspace + 2 * plane;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn_plan(moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                               const int32_t* offsets, void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  uint16_t *h_hi, *h_lo;
  void* table;
  // a non-null stand-in for sorted_slot: the plan reads only offsets
  moe_status st = check_ffn(nullptr, x_dtype, T, k_total, W, offsets, offsets, nullptr, false, false, workspace,
                            workspace_bytes, &h_hi, &h_lo, &table);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_plan(T, k_total, W->n_experts, plan_opts(W, T, k_total), offsets, table,
                                         (hipStream_t)stream));
}

moe_status moe_expert_ffn_gateup(const void* x, moe_act_dtype x_dtype, int T, int k_total,
                                 const moe_expert_weights* W, const int32_t* offsets, const int32_t* sorted_slot,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  uint16_t *h_hi, *h_lo;
  void* table;
  moe_status st = check_ffn(x, x_dtype, T, k_total, W, offsets, sorted_slot, nullptr, true, false, workspace,
                            workspace_bytes, &h_hi, &h_lo, &table);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_gateup(x, T, k_total, W->fmt, W->n_experts, plan_opts(W, T, k_total), W->hidden,
                                           W->inter, dev(W->gate),
                                           dev(W->up), sorted_slot, h_hi, h_lo, table, (hipStream_t)stream));
}

moe_status moe_expert_ffn_down(moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                               const int32_t* offsets, const int32_t* sorted_slot, float* y_slots, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  uint16_t *h_hi, *h_lo;
  void* table;
  moe_status st = check_ffn(nullptr, x_dtype, T, k_total, W, offsets, sorted_slot, y_slots, false, true, workspace,
                            workspace_bytes, &h_hi, &h_lo, &table);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_down(T, k_total, W->fmt, W->n_experts, plan_opts(W, T, k_total), W->hidden,
                                         W->inter, dev(W->down),
                                         sorted_slot, y_slots, h_hi, h_lo, table, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const void* x, moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                          const int32_t* offsets, const int32_t* sorted_slot, float* y_slots, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  uint16_t *h_hi, *h_lo;
  void* table;
  moe_status st = check_ffn(x, x_dtype, T, k_total, W, offsets, sorted_slot, y_slots, true, true, workspace,
                            workspace_bytes, &h_hi, &h_lo, &table);
  if (st != MOE_OK) return st;
  const int H = W->hidden, I = W->inter;
  const int opts = plan_opts(W, T, k_total);
  hipError_t err = moe::launch_ffn_plan(T, k_total, W->n_experts, opts, offsets, table, (hipStream_t)stream);
  if (err != hipSuccess) return MOE_ERR_HIP;
  err = moe::launch_ffn_gateup(x, T, k_total, W->fmt, W->n_experts, opts, H, I, dev(W->gate), dev(W->up), sorted_slot,
                               h_hi, h_lo, table, (hipStream_t)stream);
  if (err != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_ffn_down(T, k_total, W->fmt, W->n_experts, opts, H, I, dev(W->down), sorted_slot, y_slots,
                                         h_hi, h_lo, table, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
// Range-managed FP16 path (Cascadia Sec. 3.3, Eq. 1)
size_t moe_expert_ffn_f16_workspace_bytes(int T, int k_total, const moe_expert_weights* W) {
  if (!W || T <= 0 || k_total <= 0 || W->inter <= 0 || W->n_experts <= 0) return 0;
  const size_t plane = round_up(sizeof(uint16_t) * (size_t)T * (size_t)k_total * (size_t)W->inter, 256);
  return 2 * plane + round_up(moe::ffn_table_bytes(T, k_total, W->n_experts, false), 256);
}

moe_status moe_expert_ffn_f16(const void* x, moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                              int attenuation_log2, const int32_t* offsets, const int32_t* sorted_slot,
                              uint16_t* y_slots, void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  if (!W) return MOE_ERR_NULL;
  if (T < 0 || k_total < 1 || k_total > MOE_MAX_SLOTS_PER_TOKEN || (int64_t)T * k_total > INT_MAX) return MOE_ERR_SHAPE;
  if (attenuation_log2 < 0 || attenuation_log2 > MOE_MAX_ATTENUATION_LOG2) return MOE_ERR_SHAPE;
  if (!known_format(W->fmt)) return MOE_ERR_DTYPE;
  if (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16) return MOE_ERR_DTYPE;
  if ((W->fmt != MOE_W_FP16) != (x_dtype == MOE_ACT_BF16)) return MOE_ERR_DTYPE;
  if (W->n_experts < 1 || W->n_experts > MOE_MAX_EXPERTS || W->hidden < 1 || W->inter < 1) return MOE_ERR_SHAPE;
  if (!x || !offsets || !sorted_slot || !y_slots) return MOE_ERR_NULL;
  const int H = W->hidden, I = W->inter;
  moe_status st;
  if ((st = check_proj(W->gate, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
  if ((st = check_proj(W->up, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
  if ((st = check_proj(W->down, W->fmt, W->n_experts, H, I)) != MOE_OK) return st;
  if (!al16(x) || !al4(offsets) || !al4(sorted_slot) || ((uintptr_t)y_slots & 1u)) return MOE_ERR_ALIGN;
  const size_t need = moe_expert_ffn_f16_workspace_bytes(T, k_total, W);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  const size_t plane = round_up(sizeof(uint16_t) * (size_t)T * (size_t)k_total * (size_t)I, 256);
  uint8_t* ws = (uint8_t*)workspace;
  return hip_status(moe::launch_ffn_range(x, T, k_total, W->fmt, W->n_experts, H, I, dev(W->gate), dev(W->up),
                                          dev(W->down), offsets, sorted_slot, (uint16_t*)ws, (uint16_t*)(ws + plane),
                                          ws + 2 * plane, attenuation_log2, y_slots, (hipStream_t)stream));
}

moe_status moe_combine_restore(const uint16_t* y_slots, const float* weights, int T, int k_total, int H,
                               int attenuation_log2, float* y, void* stream) {
  if (T == 0) return MOE_OK;
  if (T < 0 || k_total < 1 || H < 1 || H % 4 != 0) return MOE_ERR_SHAPE;
  if (attenuation_log2 < 0 || attenuation_log2 > MOE_MAX_ATTENUATION_LOG2) return MOE_ERR_SHAPE;
  if (!y_slots || !weights || !y) return MOE_ERR_NULL;
  if (((uintptr_t)y_slots & 7u) || !al16(y) || !al4(weights)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine_restore(y_slots, weights, T, k_total, H, attenuation_log2, y,
                                                (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// moe_expert_ffn_static: moe_expert_ffn with its workspace (h planes and tile table) in a fixed
// device array instead of a caller buffer.  In host code `scratch` only names a host-side stand-in;
// the array's device address comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_FFN_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first call there).
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn_static(const void* x, moe_act_dtype x_dtype, int T, int k_total,
                                 const moe_expert_weights* W, const int32_t* offsets, const int32_t* sorted_slot,
                                 float* y_slots, void* stream) {
  if (T == 0) return MOE_OK;
  if (!W) return MOE_ERR_NULL;
  if (T < 0 || k_total < 1 || k_total > MOE_MAX_SLOTS_PER_TOKEN || (int64_t)T * k_total > INT_MAX)
    return MOE_ERR_SHAPE;
  const size_t need = moe_expert_ffn_workspace_bytes(T, k_total, W);
  if (need > MOE_FFN_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  // Every byte the kernels read from the workspace is written earlier in the same call (the plan
  // writes all tile-table entries, gate/up every h row that down reads), so nothing is cleared.
  return moe_expert_ffn(x, x_dtype, T, k_total, W, offsets, sorted_slot, y_slots, ws, MOE_FFN_STATIC_SCRATCH_BYTES,
                        stream);
}

// ---------------------------------------------------------------------------------------------
// MX mode
size_t moe_mx_row_bytes(moe_mx_format fmt, int K) {
  const int bits = moe::mx_bits(fmt);
  if (bits == 0 || K < 1 || K % 32 != 0) return 0;
  return (size_t)(K / 32) * 4 * (size_t)bits;
}

moe_status moe_mx_quantize(const void* x, moe_act_dtype x_dtype, int n_rows, int K, moe_mx_format fmt,
                           uint8_t* codes, uint8_t* scales, void* stream) {
  if (n_rows == 0) return MOE_OK;
  if (n_rows < 0 || K < 1) return MOE_ERR_SHAPE;
  if (K % 32 != 0) return MOE_ERR_BLOCK;
  if (moe::mx_bits(fmt) == 0 || (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16)) return MOE_ERR_DTYPE;
  if (!x || !codes || !scales) return MOE_ERR_NULL;
  if (!al16(x) || !al16(codes)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_mx_quantize(x, x_dtype == MOE_ACT_FP16, n_rows, K, fmt, codes, scales,
                                            (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Workspace of an MX call: x codes, x scales, h codes, h scales, tile table (each 256-aligned).
struct MxWs {
  size_t xq, xs, hq, hs, table, total;
};
MxWs mx_ws(int T, int k_total, const moe_expert_weights* W, moe_mx_format fmt) {
  MxWs w{};
  const size_t n_slots = (size_t)T * (size_t)k_total;
  w.xq = 0;
  w.xs = w.xq + round_up((size_t)T * moe_mx_row_bytes(fmt, W->hidden), 256);
  w.hq = w.xs + round_up((size_t)T * (size_t)(W->hidden / 32), 256);
  w.hs = w.hq + round_up(n_slots * moe_mx_row_bytes(fmt, W->inter), 256);
  w.table = w.hs + round_up(n_slots * (size_t)(W->inter / 32), 256);
  w.total = w.table + round_up((size_t)moe::mx_tiles(T, k_total, W->n_experts) * 16, 256);
  return w;
}

// The MX kernels address weight rows, scale rows and activation rows with 32-bit buffer offsets.
bool mx_offsets_ok(const moe_proj& p, int N) {
  return (int64_t)N * p.w_row_stride < INT32_MAX && (int64_t)N * p.s_row_stride < INT32_MAX;
}

}  // namespace

extern "C" {

size_t moe_expert_ffn_mx_workspace_bytes(int T, int k_total, const moe_expert_weights* W, moe_mx_format fmt) {
  if (!W || T <= 0 || k_total <= 0 || W->hidden <= 0 || W->inter <= 0 || W->n_experts <= 0 ||
      moe::mx_bits(fmt) == 0 || W->hidden % 32 != 0 || W->inter % 32 != 0)
    return 0;
  return mx_ws(T, k_total, W, fmt).total;
}

moe_status moe_expert_ffn_mx_workspace_layout(int T, int k_total, const moe_expert_weights* W, moe_mx_format fmt,
                                              size_t* offsets) {
  if (!W || !offsets) return MOE_ERR_NULL;
  if (moe::mx_bits(fmt) == 0) return MOE_ERR_DTYPE;
  if (T <= 0 || k_total <= 0 || W->hidden <= 0 || W->inter <= 0 || W->n_experts <= 0 || W->hidden % 32 != 0 ||
      W->inter % 32 != 0)
    return MOE_ERR_SHAPE;
  const MxWs w = mx_ws(T, k_total, W, fmt);
  offsets[0] = w.xq;
  offsets[1] = w.xs;
  offsets[2] = w.hq;
  offsets[3] = w.hs;
  return MOE_OK;
}

moe_status moe_expert_ffn_mx(const void* x, moe_act_dtype x_dtype, int T, int k_total, const moe_expert_weights* W,
                             moe_mx_format fmt, const int32_t* offsets, const int32_t* sorted_slot, float* y_slots,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  if (!W) return MOE_ERR_NULL;
  if (T < 0 || k_total < 1 || k_total > MOE_MAX_SLOTS_PER_TOKEN) return MOE_ERR_SHAPE;
  if (W->fmt != MOE_W_MXFP4 || x_dtype != MOE_ACT_BF16 || moe::mx_bits(fmt) == 0) return MOE_ERR_DTYPE;
  if (W->n_experts < 1 || W->n_experts > MOE_MAX_EXPERTS || W->hidden < 1 || W->inter < 1) return MOE_ERR_SHAPE;
  if ((int64_t)T * k_total > INT_MAX) return MOE_ERR_SHAPE;
  if (!x || !offsets || !sorted_slot || !y_slots) return MOE_ERR_NULL;
  const int H = W->hidden, I = W->inter;
  moe_status st;
  if ((st = check_proj(W->gate, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
  if ((st = check_proj(W->up, W->fmt, W->n_experts, I, H)) != MOE_OK) return st;
  if ((st = check_proj(W->down, W->fmt, W->n_experts, H, I)) != MOE_OK) return st;
  if (H % 256 != 0 || I % 256 != 0) return MOE_ERR_SHAPE;
  const moe_proj* ps[3] = {&W->gate, &W->up, &W->down};
  for (const moe_proj* p : ps)
    if (((uintptr_t)p->scales & 7u) != 0 || p->s_row_stride % 8 != 0 || p->s_expert_stride % 8 != 0)
      return MOE_ERR_ALIGN;
  if (!mx_offsets_ok(W->gate, I) || !mx_offsets_ok(W->up, I) || !mx_offsets_ok(W->down, H)) return MOE_ERR_SHAPE;
  const int64_t n_slots = (int64_t)T * k_total;
  if ((int64_t)T * (int64_t)moe_mx_row_bytes(fmt, H) >= INT32_MAX ||
      n_slots * (int64_t)moe_mx_row_bytes(fmt, I) >= INT32_MAX)
    return MOE_ERR_SHAPE;
  if (!al16(x) || !al16(y_slots) || !al4(offsets) || !al4(sorted_slot)) return MOE_ERR_ALIGN;
  const MxWs w = mx_ws(T, k_total, W, fmt);
  if (!workspace || workspace_bytes < w.total) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  uint8_t* ws = (uint8_t*)workspace;
  moe::MxFfnArgs a;
  a.fmt = fmt;
  a.x = x;
  a.T = T;
  a.k_total = k_total;
  a.n_experts = W->n_experts;
  a.H = H;
  a.I = I;
  a.gate = dev(W->gate);
  a.up = dev(W->up);
  a.down = dev(W->down);
  a.offsets = offsets;
  a.sorted_slot = sorted_slot;
  a.y_slots = y_slots;
  a.xq = ws + w.xq;
  a.xs = ws + w.xs;
  a.hq = ws + w.hq;
  a.hs = ws + w.hs;
  a.table = ws + w.table;
  return hip_status(moe::launch_ffn_mx(a, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
moe_status moe_combine(const float* y_slots, const float* weights, int T, int k_total, int H, float* y,
                       void* stream) {
  if (T == 0) return MOE_OK;
  if (T < 0 || k_total < 1 || H < 1 || H % 4 != 0) return MOE_ERR_SHAPE;
  if (!y_slots || !weights || !y) return MOE_ERR_NULL;
  if (!al16(y_slots) || !al16(y) || !al4(weights)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(y_slots, weights, T, k_total, H, y, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
moe_status moe_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int n_rows, int K, int64_t code_row_stride,
                             int64_t scale_row_stride, uint16_t* out, void* stream) {
  if (n_rows == 0) return MOE_OK;
  if (n_rows < 0 || K < 1) return MOE_ERR_SHAPE;
  if (K % 32 != 0) return MOE_ERR_BLOCK;
  if (!codes || !scales || !out) return MOE_ERR_NULL;
  if (code_row_stride < K / 2 || scale_row_stride < K / 32) return MOE_ERR_SHAPE;
  if (!al16(codes) || code_row_stride % 16 != 0) return MOE_ERR_BLOCK;  // a row would start mid-block
  if (!al16(out)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_dequant(codes, scales, n_rows, K, code_row_stride, scale_row_stride, out,
                                        (hipStream_t)stream));
}

moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!buf || !sink) return MOE_ERR_NULL;
  if (!al16(buf) || bytes % 16 != 0) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_stream_read(buf, (uint64_t)bytes, sink, (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

// ---------------------------------------------------------------------------------------------
// moe_route_bucket.  Workspace: router partial sums | bucketing workspace.
size_t moe_route_bucket_workspace_bytes(int T, int H, int E, int top_k, int n_shared) {
  if (T <= 0 || H <= 0 || E <= 0 || top_k < 1 || n_shared < 0) return 0;
  const int64_t n_slots = (int64_t)T * (top_k + n_shared);
  if (n_slots > INT_MAX) return 0;
  return moe_route_workspace_bytes(T, H, E) + round_up(moe_bucket_workspace_bytes((int)n_slots, E + n_shared), 256);
}

moe_status moe_route_bucket(const void* x, moe_act_dtype x_dtype, int T, int H, const float* w_router,
                            const float* logit_bias, int E, int top_k, int n_shared, int32_t* ids, float* weights,
                            float* probs, int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                            const moe_expert_weights* W, void* ffn_workspace, size_t ffn_workspace_bytes,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (T == 0) return MOE_OK;
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS || n_shared < 0 || E + n_shared > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (x_dtype != MOE_ACT_BF16 && x_dtype != MOE_ACT_FP16) return MOE_ERR_DTYPE;
  if (top_k < 1 || top_k > E || top_k + n_shared > MOE_MAX_SLOTS_PER_TOKEN) return MOE_ERR_TOPK;
  const int k_total = top_k + n_shared, n_buckets = E + n_shared;
  if ((int64_t)T * k_total > INT_MAX || (int64_t)T * E > INT_MAX) return MOE_ERR_SHAPE;
  if (!x || !w_router || !ids || !weights || !counts || !offsets || !sorted_slot) return MOE_ERR_NULL;
  if (!al16(x) || !al4(w_router) || !al4(ids) || !al4(weights) || (probs && !al4(probs)) ||
      (logit_bias && !al4(logit_bias)) || !al4(counts) || !al4(offsets) || !al4(sorted_slot) ||
      (slot_pos && !al4(slot_pos)))
    return MOE_ERR_ALIGN;
  void* table = nullptr;
  moe::FfnPlan pl{};
  if (W) {  // the tile table goes where moe_expert_ffn_plan would write it
    if (W->n_experts != n_buckets) return MOE_ERR_SHAPE;
    uint16_t *h_hi, *h_lo;
    const moe_act_dtype xdt = W->fmt == MOE_W_FP16 ? MOE_ACT_FP16 : MOE_ACT_BF16;
    const moe_status st = check_ffn(nullptr, xdt, T, k_total, W, offsets, offsets, nullptr, false, false,
                                    ffn_workspace, ffn_workspace_bytes, &h_hi, &h_lo, &table);
    if (st != MOE_OK) return st;
    pl = moe::ffn_plan(T, k_total, W->n_experts, plan_opts(W, T, k_total));
  }
  const size_t need = moe_route_bucket_workspace_bytes(T, H, E, top_k, n_shared);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  uint8_t* ws = (uint8_t*)workspace;
  float* partial = (float*)ws;
  const size_t rws = moe_route_workspace_bytes(T, H, E);
  int32_t* bws = (int32_t*)(ws + rws);
  const int splits = moe::route_splits(T, H, E);
  hipStream_t st = (hipStream_t)stream;
  if (moe::route_bucket_fusable(T, k_total, n_buckets))
    return hip_status(moe::launch_route_bucket(x, x_dtype == MOE_ACT_FP16, T, H, w_router, logit_bias, E, top_k,
                                               n_shared, ids, weights, probs, partial, splits, n_buckets, counts,
                                               offsets, sorted_slot, slot_pos, table, pl.rpt, pl.tiles, st));
  hipError_t err = moe::launch_route(x, x_dtype == MOE_ACT_FP16, T, H, w_router, logit_bias, E, top_k, n_shared, ids,
                                     weights, probs, partial, splits, st);
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (!W) {
    err = moe::launch_bucket(ids, T * k_total, n_buckets, counts, offsets, sorted_slot, slot_pos, bws, st);
    return err != hipSuccess ? MOE_ERR_HIP : MOE_OK;
  }
  err = moe::launch_bucket_plan(ids, T * k_total, n_buckets, counts, offsets, sorted_slot, slot_pos, bws, table,
                                pl.rpt, pl.tiles, st);
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (moe::bucket_plans_inline(T * k_total)) return MOE_OK;
  return hip_status(moe::launch_ffn_plan(T, k_total, W->n_experts, plan_opts(W, T, k_total), offsets, table, st));
}

}  // extern "C"
