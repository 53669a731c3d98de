// C ABI of the decode-attention library: host validation, device checks and
// dispatch to the kernel launchers. Declarations and the contract of every
// entry point are in include/decode_attn.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/decode_attn_trace.h"
#include "launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kGlobalMaxBatch = 256;    // per-call prefix table held in LDS (model domain B <= 256)
constexpr int kGlobalMaxSplits = 1 << 16;

struct DeviceInfo {
  std::atomic<int> state{0};  // 0 unknown, 1 gfx950, -1 unsupported
  int num_cus = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Current device if it is a gfx950, else a status. Only called after the
// host-side argument checks.
da_status current_device(int* dev_out, int* num_cus) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return DA_ERR_NO_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DA_ERR_NO_DEVICE;
  DeviceInfo& di = g_dev[dev];
  if (di.state.load(std::memory_order_acquire) == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (di.state.load(std::memory_order_relaxed) == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DA_ERR_NO_DEVICE;
      const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      di.num_cus = prop.multiProcessorCount;
      di.state.store(ok ? 1 : -1, std::memory_order_release);
    }
  }
  if (di.state.load(std::memory_order_acquire) != 1) return DA_ERR_NO_DEVICE;
  *dev_out = dev;
  *num_cus = di.num_cus;
  return DA_OK;
}

da_status check_common(const da_shape* s) {
  if (!s) return DA_ERR_INVALID_ARG;
  if (s->batch <= 0 || s->num_kv_heads <= 0 || s->group <= 0 || s->head_dim <= 0 ||
      s->max_pages_per_seq <= 0 || s->num_pages <= 0 || s->page_size <= 0 || s->num_splits < 0)
    return DA_ERR_INVALID_ARG;
  if (s->kv_dtype != DA_DTYPE_F32 && s->kv_dtype != DA_DTYPE_BF16) return DA_ERR_INVALID_ARG;
  if (s->out_dtype != DA_DTYPE_F32 && s->out_dtype != DA_DTYPE_BF16) return DA_ERR_INVALID_ARG;
  if ((long long)s->max_pages_per_seq * s->page_size > (1LL << 30)) return DA_ERR_INVALID_ARG;
  if (s->page_size != da::kPageSizeAbi) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

// The calls whose only output is fp32 (multi-query, appends).
da_status check_f32_out(const da_shape* s) {
  da_status st = check_common(s);
  if (st != DA_OK) return st;
  return s->out_dtype == DA_DTYPE_F32 ? DA_OK : DA_ERR_UNSUPPORTED;
}

da_status check_global_shape(const da_shape* s) {
  da_status st = check_common(s);
  if (st != DA_OK) return st;
  if (s->num_kv_heads != 1 || s->group != 16 || s->head_dim != 512) return DA_ERR_UNSUPPORTED;
  if (s->batch > kGlobalMaxBatch || s->num_splits > kGlobalMaxSplits) return DA_ERR_UNSUPPORTED;
  // the split's page prefix is 32-bit: at most 2^30 cached pages per call
  if ((long long)s->batch * s->max_pages_per_seq > (1LL << 30)) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

da_status decode_sliding(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t window, const float* gate, void* out,
                         const da_shape* shape, void* stream) {
  da_status st = check_common(shape);
  if (st != DA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return DA_ERR_INVALID_ARG;
  if (window < 0) return DA_ERR_INVALID_ARG;
  if (shape->group != 2 || shape->head_dim != 256) return DA_ERR_UNSUPPORTED;
  // waves per (sequence, KV head): 0 (the default, 4), or 1, 2, 4 or 8 (8
  // with bf16 caches only)
  const int ns = shape->num_splits;
  if (ns != 0 && ns != 1 && ns != 2 && ns != 4 && ns != 8) return DA_ERR_UNSUPPORTED;
  if (ns == 8 && shape->kv_dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  if ((long long)shape->batch * shape->num_kv_heads > 0x7FFFFFFFLL) return DA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  return da::launch_sliding(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, *shape,
                            (hipStream_t)stream);
}

da_status decode_global(const void* q, const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const float* gate, void* out, const da_shape* shape, void* workspace,
                        size_t workspace_bytes, void* stream, const float* w_k = nullptr,
                        unsigned long long* trace = nullptr) {
  da_status st = check_global_shape(shape);
  if (st != DA_OK) return st;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return DA_ERR_INVALID_ARG;
  // the pre-norm cache and the timeline are built for bf16 only
  if ((w_k || trace) && shape->kv_dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  const int splits = da::global_num_splits(*shape, cus);
  const size_t need = da::global_workspace_bytes(*shape, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DA_ERR_WORKSPACE;
  return da::launch_global(q, kv_cache, block_table, seq_lens, gate, w_k, out, *shape, splits, workspace,
                           (hipStream_t)stream, trace);
}

constexpr int kMaxQueries = 1 << 18;  // the model's position domain

// Shapes the multi-query kernels are built for: sliding (any Hkv, G 2, D 256)
// or global (Hkv 1, G 16, D 512), bf16 caches.
da_status check_multiquery_shape(const da_shape* s, bool sliding, int32_t max_queries) {
  da_status st = check_f32_out(s);
  if (st != DA_OK) return st;
  if (max_queries <= 0) return DA_ERR_INVALID_ARG;
  if (max_queries > kMaxQueries) return DA_ERR_UNSUPPORTED;
  if (s->kv_dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  if (sliding ? (s->group != 2 || s->head_dim != 256) : (s->num_kv_heads != 1 || s->group != 16 || s->head_dim != 512))
    return DA_ERR_UNSUPPORTED;
  if ((long long)s->batch * s->num_kv_heads > 65535 || s->num_splits > 65535) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

da_status multiquery(bool sliding, const void* q, const int32_t* q_start, int32_t max_queries, const void* k_cache,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens, int32_t window,
                     void* out, const da_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  da_status st = check_multiquery_shape(shape, sliding, max_queries);
  if (st != DA_OK) return st;
  if (!q || !q_start || !k_cache || !v_cache || !block_table || !seq_lens || !out) return DA_ERR_INVALID_ARG;
  if (window < 0) return DA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  const da::mq_plan plan = da::multiquery_plan(*shape, max_queries, window, cus);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return DA_ERR_WORKSPACE;
  return da::launch_multiquery(q, q_start, max_queries, k_cache, v_cache, block_table, seq_lens, window, out,
                               *shape, plan, workspace, (hipStream_t)stream);
}

}  // namespace

extern "C" {

da_status attn_multiquery_sliding(const void* q, const int32_t* q_start, int32_t max_queries,
                                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t window, void* out, const da_shape* shape,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return multiquery(true, q, q_start, max_queries, k_cache, v_cache, block_table, seq_lens, window, out, shape,
                    workspace, workspace_bytes, stream);
}

da_status attn_multiquery_global(const void* q, const int32_t* q_start, int32_t max_queries,
                                 const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                                 void* out, const da_shape* shape, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return multiquery(false, q, q_start, max_queries, kv_cache, kv_cache, block_table, seq_lens, 0, out, shape,
                    workspace, workspace_bytes, stream);
}

da_status attn_multiquery_workspace_bytes(const da_shape* shape, int32_t max_queries, int32_t window,
                                          size_t* bytes) {
  if (!bytes) return DA_ERR_INVALID_ARG;
  const bool sliding = shape && shape->head_dim == 256;
  da_status st = check_multiquery_shape(shape, sliding, max_queries);
  if (st != DA_OK) return st;
  if (window < 0) return DA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  *bytes = da::multiquery_plan(*shape, max_queries, window, cus).ws_bytes;
  return DA_OK;
}

da_status attn_decode_sliding(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t window,
                              void* out, const da_shape* shape, void* stream) {
  return decode_sliding(q, k_cache, v_cache, block_table, seq_lens, window, nullptr, out, shape, stream);
}

da_status attn_decode_sliding_gated(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, int32_t window,
                                    const float* gate, void* out, const da_shape* shape, void* stream) {
  if (!gate) return DA_ERR_INVALID_ARG;
  return decode_sliding(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, shape, stream);
}

da_status attn_decode_global_workspace_bytes(const da_shape* shape, size_t* bytes) {
  if (!bytes) return DA_ERR_INVALID_ARG;
  da_status st = check_global_shape(shape);
  if (st != DA_OK) return st;
  int dev = 0, cus = 0;
  if (shape->num_splits == 0) {
    st = current_device(&dev, &cus);
    if (st != DA_OK) return st;
  }
  *bytes = da::global_workspace_bytes(*shape, da::global_num_splits(*shape, cus));
  return DA_OK;
}

da_status attn_decode_global(const void* q, const void* kv_cache, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, const da_shape* shape,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_global(q, kv_cache, block_table, seq_lens, nullptr, out, shape, workspace, workspace_bytes,
                       stream);
}

da_status attn_decode_global_traced(const void* q, const void* kv_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, void* out, const da_shape* shape, void* workspace,
                                    size_t workspace_bytes, uint64_t* trace, void* stream) {
  if (!trace) return DA_ERR_INVALID_ARG;
  return decode_global(q, kv_cache, block_table, seq_lens, nullptr, out, shape, workspace, workspace_bytes, stream,
                       nullptr, reinterpret_cast<unsigned long long*>(trace));
}

da_status attn_decode_global_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, void* out, const da_shape* shape, void* stream) {
  da_status st = check_global_shape(shape);
  if (st != DA_OK) return st;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return DA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  int max_splits = 0;
  st = da::global_scratch(dev, &scratch, &scratch_bytes, &max_splits);
  if (st != DA_OK) return st;
  // the default split (one workgroup per compute unit) is capped at what the
  // scratch array holds; an explicit split beyond it is refused
  const int splits = shape->num_splits > 0 ? shape->num_splits : (cus < max_splits ? cus : max_splits);
  if (splits > max_splits) return DA_ERR_WORKSPACE;
  if (da::global_workspace_bytes(*shape, splits) > scratch_bytes) return DA_ERR_WORKSPACE;
  return da::launch_global(q, kv_cache, block_table, seq_lens, nullptr, nullptr, out, *shape, splits, scratch,
                           (hipStream_t)stream);
}

da_status attn_decode_global_prenorm(const void* q, const void* x_cache, const float* w_k,
                                     const int32_t* block_table, const int32_t* seq_lens, void* out,
                                     const da_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  if (!w_k) return DA_ERR_INVALID_ARG;
  return decode_global(q, x_cache, block_table, seq_lens, nullptr, out, shape, workspace, workspace_bytes, stream,
                       w_k);
}

da_status attn_decode_global_gated(const void* q, const void* kv_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, const float* gate, void* out, const da_shape* shape,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate) return DA_ERR_INVALID_ARG;
  return decode_global(q, kv_cache, block_table, seq_lens, gate, out, shape, workspace, workspace_bytes, stream);
}

da_status attn_kv_append_sliding(const float* q_raw, const float* k_raw, const float* v_raw, const float* w_q,
                                 const float* w_k, const int32_t* block_table, const int32_t* positions,
                                 void* k_cache, void* v_cache, void* q_out, const da_shape* shape, void* stream) {
  da_status st = check_f32_out(shape);
  if (st != DA_OK) return st;
  if (!q_raw || !k_raw || !v_raw || !w_q || !w_k || !block_table || !positions || !k_cache || !v_cache ||
      !q_out)
    return DA_ERR_INVALID_ARG;
  if (shape->head_dim != 256) return DA_ERR_UNSUPPORTED;
  if ((long long)shape->batch * shape->num_kv_heads * (shape->group + 2) > 0x7FFFFFFFLL) return DA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  return da::launch_append_sliding(q_raw, k_raw, v_raw, w_q, w_k, block_table, positions, k_cache, v_cache, q_out,
                                   *shape, (hipStream_t)stream);
}

da_status attn_kv_append_global(const float* q_raw, const float* kv_raw, const float* w_q, const float* w_k,
                                const int32_t* block_table, const int32_t* positions, void* kv_cache, void* q_out,
                                const da_shape* shape, void* stream) {
  da_status st = check_f32_out(shape);
  if (st != DA_OK) return st;
  if (!q_raw || !kv_raw || !w_q || !w_k || !block_table || !positions || !kv_cache || !q_out)
    return DA_ERR_INVALID_ARG;
  if (shape->head_dim != 512) return DA_ERR_UNSUPPORTED;
  if ((long long)shape->batch * shape->num_kv_heads * (shape->group + 1) > 0x7FFFFFFFLL) return DA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  return da::launch_append_global(q_raw, kv_raw, w_q, w_k, block_table, positions, kv_cache, q_out, *shape,
                                  (hipStream_t)stream);
}

da_status attn_kv_append_global_prenorm(const float* q_raw, const float* x_raw, const float* w_q,
                                        const int32_t* block_table, const int32_t* positions, void* x_cache,
                                        void* q_out, const da_shape* shape, void* stream) {
  da_status st = check_f32_out(shape);
  if (st != DA_OK) return st;
  if (!q_raw || !x_raw || !w_q || !block_table || !positions || !x_cache || !q_out) return DA_ERR_INVALID_ARG;
  if (shape->head_dim != 512 || shape->kv_dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  if ((long long)shape->batch * shape->num_kv_heads * (shape->group + 1) > 0x7FFFFFFFLL) return DA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != DA_OK) return st;
  return da::launch_append_global_prenorm(q_raw, x_raw, w_q, block_table, positions, x_cache, q_out, *shape,
                                          (hipStream_t)stream);
}

const char* attn_status_string(da_status status) {
  switch (status) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID_ARG: return "invalid argument";
    case DA_ERR_UNSUPPORTED: return "unsupported shape, dtype or page size";
    case DA_ERR_WORKSPACE: return "workspace missing or too small";
    case DA_ERR_NO_DEVICE: return "no gfx950 HIP device is current";
    case DA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
