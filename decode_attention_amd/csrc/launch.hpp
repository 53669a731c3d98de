// Internal launcher interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes the arguments already passed host validation.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/decode_attn.h"

namespace da {

constexpr int kPageSizeAbi = 16;  // tokens per page the kernels are built for

// gate: fp32 [B][Hq][D] for the sigmoidGate epilogue, or null.
da_status launch_sliding(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t window, const float* gate,
                         void* out, const da_shape& s, hipStream_t stream);

// Number of workgroups the global kernel divides the batch's pages among.
int global_num_splits(const da_shape& s, int num_cus);
size_t global_workspace_bytes(const da_shape& s, int num_splits);

// Device address (on device `dev`, which must be current) and size of the
// library's own scratch array for the allocation-free global call, and the
// largest split it holds.
da_status global_scratch(int dev, void** ptr, size_t* bytes, int* max_splits);

// w_k: null for the K=V cache; the k-norm weight [512] for the pre-norm cache.
// trace: null, or [num_splits][4] uint64 per-workgroup timeline entries.
da_status launch_global(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, const float* gate, const float* w_k, void* out,
                        const da_shape& s, int num_splits, void* workspace, hipStream_t stream,
                        unsigned long long* trace = nullptr);

// Decode-step norm + RoPE of the new tokens and their append to the caches.
da_status launch_append_sliding(const float* q_raw, const float* k_raw, const float* v_raw, const float* w_q,
                                const float* w_k, const int32_t* block_table, const int32_t* positions,
                                void* k_cache, void* v_cache, void* q_out, const da_shape& s, hipStream_t stream);
da_status launch_append_global(const float* q_raw, const float* kv_raw, const float* w_q, const float* w_k,
                               const int32_t* block_table, const int32_t* positions, void* kv_cache, void* q_out,
                               const da_shape& s, hipStream_t stream);
// The same for the pre-norm cache of the global layers: q as above, the new
// token's projection stored unnormalised and unrotated.
da_status launch_append_global_prenorm(const float* q_raw, const float* x_raw, const float* w_q,
                                       const int32_t* block_table, const int32_t* positions, void* x_cache,
                                       void* q_out, const da_shape& s, hipStream_t stream);

// Several queries per sequence at its last positions (row f2).
// Work layout: a fixed number of pieces per unit (sequence, KV head, row
// block), or a layout made on the device from the units' page counts over
// `grid` workgroups: pieces per unit (sliding layers) or equal shares of all
// units' steps laid end to end (global layers).
struct mq_plan {
  int nblk;         // row blocks per sequence
  int units;        // batch * num_kv_heads * nblk
  int balanced;     // 1: pieces per unit; 2: contiguous shares
  int nsplit;       // fixed split: pieces per unit (1: none)
  int grid;         // balanced: workgroups of the main kernel
  int rows;         // rows per block: 128, or 256 (sliding layers, long chunks)
  size_t ws_bytes;  // workspace the call needs
};
mq_plan multiquery_plan(const da_shape& s, int max_queries, int window, int num_cus);
da_status launch_multiquery(const void* q, const int32_t* q_start, int max_queries, const void* k_cache,
                            const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                            int window, void* out, const da_shape& s, const mq_plan& p, void* workspace,
                            hipStream_t stream);

}  // namespace da
