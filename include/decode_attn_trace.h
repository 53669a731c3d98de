/*
 * decode_attn_trace.h - measurement support exported by libdecode_attn.so:
 * the global decode call with a per-workgroup timeline. It is not part of
 * the attention path; it runs the same kernels as attn_decode_global and, in
 * addition, has every workgroup of the decode kernel record when it started
 * and finished, which compute die (XCC) it ran on and how many pages and
 * segments it walked. The timeline shows where the call's time goes: the
 * start-up before the first page arrives, the spread of workgroup end times
 * (the tail) and the merge after them.
 */
#ifndef DECODE_ATTN_TRACE_H
#define DECODE_ATTN_TRACE_H

#include <stdint.h>

#include "decode_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* attn_decode_global (same arguments, results and errors) that also writes,
 * for every workgroup w of the decode kernel (w < number of splits: the
 * shape's num_splits, or one per compute unit when it is 0), four uint64
 * entries at trace[4w .. 4w+3]:
 *   [0] start, [1] end: the device's 100 MHz real-time counter (10 ns
 *       ticks; only differences mean anything);
 *   [2] bits 0..3: XCC id; bits 8..: segments the workgroup finished;
 *   [3] bits 0..31: pages in its range; bits 32..63: the HW_ID register of
 *       its first wave (CU, SIMD, shader engine).
 * trace: device memory of at least 32 * splits bytes, caller-owned. A NULL
 * trace is an invalid argument. Built for bf16 caches only (an fp32 cache
 * returns DA_ERR_UNSUPPORTED).
 */
da_status attn_decode_global_traced(const void* q, const void* kv_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, void* out, const da_shape* shape,
                                    void* workspace, size_t workspace_bytes, uint64_t* trace,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_TRACE_H */
