// moe_api.hip - the extern "C" entry points of libmoe_mxfp4: argument
// validation (before anything is enqueued), the gfx950 check, then the
// kernel launchers.  No call allocates, frees or synchronizes.
#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

moe_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev < kMaxDevices) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return MOE_OK;
    if (st == 2) return MOE_ERR_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Device scratch of moe_decode_layer_mxfp4_noalloc: one copy per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address; it uses the per-device pointer hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up once per device (with
// that device current) and kept.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

bool rows_fit(int32_t T, int32_t k) { return T >= 0 && k >= 1 && (int64_t)T * k <= INT32_MAX / 2; }

bool weights_ok(const moe_mxfp4_weights* w) {
  if (!w) return false;
  if (!w->gate_q || !w->gate_s || !w->up_q || !w->up_s || !w->down_q || !w->down_s) return false;
  if (!aligned16(w->gate_q) || !aligned16(w->up_q) || !aligned16(w->down_q)) return false;
  if (((uintptr_t)w->gate_s & 3) || ((uintptr_t)w->up_s & 3) || ((uintptr_t)w->down_s & 3)) return false;
  if (w->expert_stride <= 0 || (w->expert_stride & 15) != 0) return false;
  if (w->num_experts < 1 || w->num_experts > MOE_MAX_EXPERTS) return false;
  if (w->hidden < 32 || w->hidden > MOE_MAX_DIM || (w->hidden & 31) != 0) return false;
  if (w->inter < 32 || w->inter > MOE_MAX_DIM || (w->inter & 31) != 0) return false;
  return true;
}

bool decode_args_ok(const float* logits, const uint16_t* x, int32_t k, const moe_mxfp4_weights* w,
                    const int32_t* topk_ids, const float* topk_weights, const int32_t* expert_offsets,
                    const int32_t* sorted_rows, const int32_t* row_pos, const int32_t* active, const float* y_rows,
                    const float* out) {
  if (!logits || !x || !topk_ids || !topk_weights || !expert_offsets || !sorted_rows || !row_pos || !active ||
      !y_rows || !out)
    return false;
  if (!aligned16(x) || !aligned16(y_rows) || !aligned16(out)) return false;
  return weights_ok(w) && k >= 1 && k <= MOE_MAX_TOPK && k <= w->num_experts;
}

moe_status decode_layer_launch(const float* logits, const uint16_t* x, int32_t k, const moe_mxfp4_weights* w,
                               int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                               int32_t* sorted_rows, int32_t* row_pos, int32_t* active, float* y_rows, float* out,
                               void* ws, hipStream_t s) {
  const int E = w->num_experts;
  if (moe::route_ffn_combine_one_ok(E, k, *w))
    return from_hip(moe::launch_route_ffn_combine_one(logits, k, x, nullptr, 0.0f, nullptr, *w, topk_ids,
                                                      topk_weights, expert_offsets, sorted_rows, row_pos, active,
                                                      y_rows, out, ws, s));
  hipError_t err;
  if (E <= 2048) {
    err = moe::launch_route_group_one(logits, E, k, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos,
                                      active, s);
  } else {
    err = moe::launch_route_topk(logits, 1, E, k, topk_ids, topk_weights, s);
    if (err == hipSuccess)
      err = moe::launch_group_rows(topk_ids, 1, k, E, expert_offsets, sorted_rows, row_pos, active, nullptr, s);
  }
  if (err != hipSuccess) return MOE_ERR_HIP;
  return from_hip(moe::launch_expert_ffn_combine(x, 1, k, *w, expert_offsets, sorted_rows, active, topk_weights,
                                                 row_pos, y_rows, out, ws, s));
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null or misaligned pointer, or size out of range";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE: the current HIP device is not gfx950";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace_bytes below moe_workspace_bytes()";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "MOE_ERR_SCRATCH_TOO_SMALL: the shape needs more than the library's static scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown moe_status";
}

size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  if (H < 32 || H > MOE_MAX_DIM || (H & 31) || I < 32 || I > MOE_MAX_DIM || (I & 31)) return 0;
  const size_t g = moe::group_rows_workspace(T, k, E);
  const size_t f = moe::expert_ffn_workspace(T, k, E, H, I);
  const size_t b = g > f ? g : f;
  return b < 256 ? 256 : b;
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                          float* topk_weights, moe_stream_t stream) {
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E || !rows_fit(T, k))
    return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_weights, (hipStream_t)stream));
}

moe_status moe_group_rows(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
                          int32_t* sorted_rows, int32_t* row_pos, int32_t* active, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream) {
  if (!expert_offsets || !active) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !sorted_rows || !row_pos)) return MOE_ERR_INVALID_ARG;
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::group_rows_workspace(T, k, E);
  if (need > 0 && (!workspace || !aligned16(workspace))) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_group_rows(topk_ids, T, k, E, expert_offsets, sorted_rows, row_pos, active,
                                         workspace, (hipStream_t)stream));
}

moe_status moe_expert_ffn_mxfp4(const uint16_t* x, int32_t T, int32_t k, const moe_mxfp4_weights* w,
                                const int32_t* expert_offsets, const int32_t* sorted_rows, const int32_t* active,
                                float* y_rows, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  if (!expert_offsets || !active || !workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !sorted_rows || !y_rows)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y_rows)) return MOE_ERR_INVALID_ARG;
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || !weights_ok(w)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe::expert_ffn_workspace(T, k, w->num_experts, w->hidden, w->inter))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_expert_ffn(x, T, k, *w, expert_offsets, sorted_rows, active, y_rows, workspace,
                                         (hipStream_t)stream));
}

moe_status moe_combine(const float* y_rows, const float* topk_weights, const int32_t* row_pos, int32_t T,
                       int32_t k, int32_t H, float* out, moe_stream_t stream) {
  if (T > 0 && (!y_rows || !topk_weights || !row_pos || !out)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_rows) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || H < 1 || H > MOE_MAX_DIM) return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_combine(y_rows, topk_weights, row_pos, T, k, H, out, (hipStream_t)stream));
}

moe_status moe_rms_rescale_bf16(const float* y, int32_t T, int32_t H, float eps, uint16_t* x_next,
                                moe_stream_t stream) {
  if ((T > 0 && (!y || !x_next)) || T < 0 || H < 32 || H > MOE_MAX_DIM || (H & 31) != 0 || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)y & 15) != 0 || ((uintptr_t)x_next & 7) != 0) return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_rms_rescale(y, T, H, eps, x_next, (hipStream_t)stream));
}

moe_status moe_route_group_one(const float* logits, int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                               int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos, int32_t* active,
                               moe_stream_t stream) {
  if (!logits || !topk_ids || !topk_weights || !expert_offsets || !sorted_rows || !row_pos || !active)
    return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  const hipStream_t s = (hipStream_t)stream;
  if (E <= 2048)
    return from_hip(moe::launch_route_group_one(logits, E, k, topk_ids, topk_weights, expert_offsets, sorted_rows,
                                                row_pos, active, s));
  hipError_t err = moe::launch_route_topk(logits, 1, E, k, topk_ids, topk_weights, s);
  if (err == hipSuccess)  // k rows: the grouping needs no workspace
    err = moe::launch_group_rows(topk_ids, 1, k, E, expert_offsets, sorted_rows, row_pos, active, nullptr, s);
  return from_hip(err);
}

moe_status moe_combine_rms_bf16(const float* y_rows, const float* topk_weights, const int32_t* row_pos, int32_t T,
                                int32_t k, int32_t H, float eps, float* out, uint16_t* x_next, moe_stream_t stream) {
  if (T > 0 && (!y_rows || !topk_weights || !row_pos || !out || !x_next)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_rows) || !aligned16(out) || ((uintptr_t)x_next & 7) != 0) return MOE_ERR_INVALID_ARG;
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || H < 32 || H > MOE_MAX_DIM || (H & 31) != 0 || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_combine_rms(y_rows, topk_weights, row_pos, T, k, H, eps, out, x_next,
                                          (hipStream_t)stream));
}

moe_status moe_expert_ffn_combine_mxfp4(const uint16_t* x, int32_t T, int32_t k, const moe_mxfp4_weights* w,
                                        const int32_t* expert_offsets, const int32_t* sorted_rows,
                                        const int32_t* active, const float* topk_weights, const int32_t* row_pos,
                                        float* y_rows, float* out, void* workspace, size_t workspace_bytes,
                                        moe_stream_t stream) {
  if (!expert_offsets || !active || !workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !sorted_rows || !y_rows || !topk_weights || !row_pos || !out)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y_rows) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (!rows_fit(T, k) || k > MOE_MAX_TOPK || !weights_ok(w)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe::expert_ffn_workspace(T, k, w->num_experts, w->hidden, w->inter))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_expert_ffn_combine(x, T, k, *w, expert_offsets, sorted_rows, active, topk_weights,
                                                 row_pos, y_rows, out, workspace, (hipStream_t)stream));
}

moe_status moe_decode_layer_mxfp4(const float* logits, const uint16_t* x, int32_t k, const moe_mxfp4_weights* w,
                                  int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                                  int32_t* sorted_rows, int32_t* row_pos, int32_t* active, float* y_rows, float* out,
                                  void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  if (!decode_args_ok(logits, x, k, w, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos, active, y_rows,
                      out))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe::expert_ffn_workspace(1, k, w->num_experts, w->hidden, w->inter))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return decode_layer_launch(logits, x, k, w, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos, active,
                             y_rows, out, workspace, (hipStream_t)stream);
}

moe_status moe_decode_layer_mxfp4_noalloc(const float* logits, const uint16_t* x, int32_t k,
                                          const moe_mxfp4_weights* w, int32_t* topk_ids, float* topk_weights,
                                          int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos,
                                          int32_t* active, float* y_rows, float* out, moe_stream_t stream) {
  if (!decode_args_ok(logits, x, k, w, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos, active, y_rows,
                      out))
    return MOE_ERR_INVALID_ARG;
  if (moe::expert_ffn_workspace(1, k, w->num_experts, w->hidden, w->inter) > MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_SCRATCH_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  void* ws = nullptr;
  const moe_status sp = scratch_ptr(&ws);
  if (sp != MOE_OK) return sp;
  return decode_layer_launch(logits, x, k, w, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos, active,
                             y_rows, out, ws, (hipStream_t)stream);
}

moe_status moe_decode_layer_rms_mxfp4(const float* logits, const float* y_prev, float eps, uint16_t* x_next,
                                      int32_t k, const moe_mxfp4_weights* w, int32_t* topk_ids,
                                      float* topk_weights, int32_t* expert_offsets, int32_t* sorted_rows,
                                      int32_t* row_pos, int32_t* active, float* y_rows, float* out, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream) {
  if (!y_prev || !x_next || !aligned16(y_prev) || !aligned16(x_next) || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (!weights_ok(w)) return MOE_ERR_INVALID_ARG;
  const int E = w->num_experts;
  if (k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_ERR_INVALID_ARG;
  if (!moe::route_ffn_combine_one_ok(E, k, *w)) {
    // the rescale, then the layer as moe_decode_layer_mxfp4 runs it
    if (!logits || !topk_ids || !topk_weights || !expert_offsets || !sorted_rows || !row_pos || !active ||
        !y_rows || !out || !workspace)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(y_rows) || !aligned16(out) || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < moe::expert_ffn_workspace(1, k, E, w->hidden, w->inter)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    const moe_status d = check_device();
    if (d != MOE_OK) return d;
    if (moe::launch_rms_rescale(y_prev, 1, w->hidden, eps, x_next, (hipStream_t)stream) != hipSuccess)
      return MOE_ERR_HIP;
    return moe_decode_layer_mxfp4(logits, x_next, k, w, topk_ids, topk_weights, expert_offsets, sorted_rows, row_pos,
                                  active, y_rows, out, workspace, workspace_bytes, stream);
  }
  if (!logits || !topk_ids || !topk_weights || !expert_offsets || !sorted_rows || !row_pos || !active || !y_rows ||
      !out || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_rows) || !aligned16(out) || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe::expert_ffn_workspace(1, k, E, w->hidden, w->inter)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_route_ffn_combine_one(logits, k, nullptr, y_prev, eps, x_next, *w, topk_ids,
                                                    topk_weights, expert_offsets, sorted_rows, row_pos, active,
                                                    y_rows, out, workspace, (hipStream_t)stream));
}

moe_status moe_router_logits(const uint16_t* x_bf16, int32_t T, int32_t H, const float* w_router, int32_t E,
                             float* logits, moe_stream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || H < 32 || H > MOE_MAX_DIM || (H & 31) != 0)
    return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x_bf16 || !w_router || !logits)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x_bf16) || !aligned16(w_router) || ((uintptr_t)logits & 3) != 0))
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_INVALID_ARG;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(moe::launch_router_logits(x_bf16, T, H, w_router, E, logits, (hipStream_t)stream));
}

}  // extern "C"
