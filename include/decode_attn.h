/*
 * decode_attn.h - C ABI of a paged decode-attention library for AMD MI355X
 * (gfx950, CDNA4).
 *
 * What is computed (pages: Op Specs of google/gemma-4-12B, Attention.lean, and
 * the gemma-4-12b Model Spec, "Compute-graph nodes" attn.core rows):
 *
 *   for every sequence b and query head h = c*G + g (KV head c = h / G):
 *     o[b,h,:] = sum over visible positions l of
 *                softmax_l( 1 * <q[b,h,:], k[b,l,c,:]> ) * v[b,l,c,:]
 *
 *   - attn_decode_sliding: slidingDecodeGQA. The query sits at the last
 *     position L-1 of the L = seq_lens[b] cached tokens and sees the keys with
 *     L-1-window < l <= L-1 (the window predicate of slidingGQA with
 *     p = L-1), i.e. exactly min(L, window) keys. Separate k and v caches.
 *   - attn_decode_global: decodeGQA. Every cached position is visible, and
 *     values equal keys ("values = keys" on the global layers), so one cache
 *     is read as both k and v. Long sequences are split over workgroups and
 *     the per-split results are merged with their log-sum-exp values inside
 *     the call.
 *
 *   The softmax scale is fixed at 1 (this model normalises q and k per head
 *   instead of scaling the logits), so it is not an argument. A sequence
 *   with no visible key (L = 0, or window = 0) gets an all-zero output row.
 *
 * Paged KV layout (page = 16 tokens, the model's page size):
 *   block_table : int32 [batch][max_pages_per_seq], row-major. Entry j of row
 *                 b is the physical page that holds tokens 16j .. 16j+15 of
 *                 sequence b. Only the entries a call needs are read:
 *                 sliding reads j in [max(0,L-window)/16, (L-1)/16], global
 *                 reads j in [0, (L-1)/16]. Other entries may hold anything.
 *   sliding caches (k_cache, v_cache): row-major [num_pages][Hkv][16][D];
 *                 token t of sequence b, KV head c, coordinate d is element
 *                 [block_table[b][t/16]][c][t%16][d].
 *   global cache (kv_cache): tiled [num_pages][Hkv][D/x][16][x], where
 *                 x = 16 bytes / element size (8 for bf16, 4 for fp32); the
 *                 same element is [block_table[b][t/16]][c][d/x][t%16][d%x].
 *                 Each 16-byte chunk holds x consecutive coordinates of one
 *                 token; chunks are ordered by coordinate group, then token.
 *   Slots and pages outside the visible positions are never read; they may
 *   hold any bits, NaN included.
 *
 *   q   : [batch][Hkv*G][D], same dtype as the caches.
 *   out : [batch][Hkv*G][D], fp32.
 *
 * Conventions:
 *   - Every pointer argument except `shape` and `stream` is a device pointer
 *     owned by the caller. The library reads q, the caches, block_table and
 *     seq_lens, writes out (and the workspace), and keeps no pointer after
 *     the call returns.
 *   - Calls are asynchronous: they validate on the host, enqueue kernels on
 *     `stream` (a hipStream_t; NULL = the device's null stream) and return.
 *     Results are valid after the stream is synchronised. Calls hold no
 *     global state and may be made from several host threads.
 *   - Host-side validation happens before any HIP call; a non-zero status
 *     means nothing was enqueued.
 *   - Preconditions the library cannot check without a device sync (the
 *     caller's responsibility): 0 <= seq_lens[b] <= 16*max_pages_per_seq,
 *     every block-table entry a call reads is in [0, num_pages), and out does
 *     not overlap any input. Violating them is undefined behaviour.
 *   - The workspace of attn_decode_global must not be shared by two calls
 *     that may run concurrently.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t da_status;

#define DA_OK 0
#define DA_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, bad window ... */
#define DA_ERR_UNSUPPORTED (-2) /* valid but not built: other (Hkv, G, D), dtype, page size */
#define DA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define DA_ERR_NO_DEVICE (-4)   /* no HIP device, or the current device is not gfx950 */
#define DA_ERR_LAUNCH (-5)      /* a HIP launch reported an error */

#define DA_DTYPE_F32 0
#define DA_DTYPE_BF16 1

/* Problem description. Host memory, read during the call only. */
typedef struct da_shape {
  int32_t batch;             /* B >= 1 sequences */
  int32_t num_kv_heads;      /* Hkv */
  int32_t group;             /* G query heads per KV head (Hq = Hkv*G) */
  int32_t head_dim;          /* D */
  int32_t page_size;         /* tokens per page; must be 16 */
  int32_t max_pages_per_seq; /* P_max >= 1: length of a block-table row */
  int32_t num_pages;         /* physical pages in the cache pool, >= 1 */
  int32_t kv_dtype;          /* DA_DTYPE_F32 or DA_DTYPE_BF16 (q, k, v) */
  int32_t out_dtype;         /* DA_DTYPE_F32, or DA_DTYPE_BF16 for the decode
                                calls (sliding, global, gated, pre-norm,
                                no-alloc): each output element rounded to
                                nearest even once; the multi-query calls and
                                the appends take DA_DTYPE_F32 only */
  int32_t num_splits;        /* attn_decode_global: number of workgroups the
                                cached pages of the whole batch are divided
                                among (0 = one per compute unit).
                                attn_decode_sliding: number of waves each
                                (sequence, KV head) window is divided among,
                                page by page, their states merged in LDS:
                                0 (the default, 4), 1, 2, 4 or 8 (8 with bf16
                                caches only) */
} da_shape;

/*
 * slidingDecodeGQA over paged k/v caches (Gemma-4-12B sliding layers:
 * Hkv = 8, G = 2, D = 256, window 1024).
 *   Built shapes: (Hkv, G, D) with G = 2, D = 256, any Hkv >= 1;
 *   kv dtypes fp32 and bf16; out fp32 or bf16 (shape->out_dtype).
 *   window >= 0 (0 gives zeros). seq_lens: int32 [batch].
 *   shape->num_splits: 0, 1, 2, 4 or 8 (waves per sequence and KV head,
 *   above; 8 with bf16 caches only); other values return
 *   DA_ERR_UNSUPPORTED. The results of
 *   different wave counts agree to fp32 rounding.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_NO_DEVICE or
 * DA_ERR_LAUNCH.
 */
da_status attn_decode_sliding(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t window, void* out, const da_shape* shape, void* stream);

/*
 * Bytes of device workspace attn_decode_global needs for `shape` on the
 * current device: a 16 KiB header (the batch's page prefix table) and, for
 * each of 2*num_splits partial-result slots, Hq*(D+2) fp32 values. 0 when
 * the call would use a single workgroup (nothing to merge). num_splits = 0
 * asks for the default, one workgroup per compute unit of the current
 * device. Writes the size to *bytes.
 */
da_status attn_decode_global_workspace_bytes(const da_shape* shape, size_t* bytes);

/*
 * decodeGQA over a paged K=V cache (Gemma-4-12B global layers: Hkv = 1,
 * G = 16, D = 512, values equal keys).
 *   Built shapes: Hkv = 1, G = 16, D = 512; kv dtype bf16 or fp32 (q in the
 *   same dtype; fp32 caches run a kernel whose scores are summed in fp64 and
 *   whose weights and PV products are fp32, for results within 1e-5); out
 *   fp32 or bf16 (shape->out_dtype; the split pieces are merged in fp32 and
 *   rounded once);
 *   batch <= 256 (larger batches return DA_ERR_UNSUPPORTED; split them into
 *   calls of at most 256 sequences); num_splits <= 65536;
 *   batch * max_pages_per_seq <= 2^30.
 *   Work split: the cached pages of the batch, laid end to end, are cut
 *   into contiguous ranges, one per workgroup (num_splits of them, or one
 *   per compute unit when num_splits = 0), of equal weight, where a page
 *   weighs 1 and the start of each non-empty sequence 8 more (a range that
 *   opens a sequence stages its q and writes its partial result); the
 *   output is reproducible bit for bit for a given split.
 *   workspace: device memory of at least attn_decode_global_workspace_bytes
 *   (may be NULL when that size is 0). Its contents need no initialisation
 *   and are meaningless after the call.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE,
 * DA_ERR_NO_DEVICE or DA_ERR_LAUNCH.
 */
da_status attn_decode_global(const void* q, const void* kv_cache, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, const da_shape* shape,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_global without a caller-provided workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The partial results live in a
 * scratch array the library holds in device memory (16.9 MB per device, for
 * at most 256 workgroups); the call allocates nothing.
 *   Arguments, shapes and results as for attn_decode_global. num_splits = 0
 *   uses one workgroup per compute unit, at most 256; an explicit num_splits
 *   above 256 returns DA_ERR_WORKSPACE.
 *   Every call on a device uses that device's one scratch array: calls that
 *   may overlap on one device (different streams without ordering) race and
 *   give undefined results. Calls ordered on a stream are safe; nothing in
 *   the array needs clearing between calls.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE,
 * DA_ERR_NO_DEVICE or DA_ERR_LAUNCH (also when the scratch array's device
 * address cannot be resolved).
 */
da_status attn_decode_global_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, void* out, const da_shape* shape,
                                     void* stream);

/*
 * Global decode from the shared pre-norm projection (pages: gemma-4-12b Model
 * Spec, compute-graph nodes attn.qk_norm, attn.v_norm, attn.rope of the
 * global layers; Op Specs Norm.lean rmsnorm / rmsnormUnit and Rope.lean rope).
 * The cache holds, per token, the 512-wide kv projection x before its norms;
 * the call derives, for every cached position l,
 *   k[l] = rope(pos l, rmsnorm(1e-6, x[l], w_k))   (theta 1e6, rot = denom =
 *          512, the first 64 frequencies active: pairs (d, d + 256), d < 64)
 *   v[l] = rmsnormUnit(1e-6, x[l])
 * and computes decodeGQA(q, k, v) as attn_decode_global does, reading each
 * page once. q is the already normed and rotated query.
 *
 *   x_cache : bf16 [num_pages][1][64][16][8]: coordinate d of token t is
 *             element [block_table[b][t/16]][0][32*(B%2) + 4*(B/2) + (d%32)/8]
 *             [t%16][d%8] with B = d/32 (each 32-coordinate block B in half
 *             B%2, so the pair (d, d + 256) shares a chunk slot of one half).
 *   w_k     : fp32 [512] device array, the k-norm weight.
 *   shape->kv_dtype must be BF16 (DA_ERR_UNSUPPORTED otherwise). Everything
 *   else (shape limits, workspace, out, NaN in unread storage) as for
 *   attn_decode_global; the workspace size is the same.
 */
da_status attn_decode_global_prenorm(const void* q, const void* x_cache, const float* w_k,
                                     const int32_t* block_table, const int32_t* seq_lens, void* out,
                                     const da_shape* shape, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * attn_decode_sliding and attn_decode_global followed by the output gate of
 * gated attention, o * sigmoid(gate) elementwise (pages: Op Specs of
 * google/gemma-4-12B, Attention.lean sigmoidGate; Op Specs overview, "Scalar
 * functions", sigmoid(x) = 1 / (1 + exp(-x))), applied where each output row
 * is written. gate: fp32 device array [batch][Hkv*G][D], the layout of out;
 * it must not overlap out. A NULL gate is an invalid argument. Everything
 * else as for the ungated calls.
 */
da_status attn_decode_sliding_gated(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t window, const float* gate, void* out,
                                    const da_shape* shape, void* stream);
da_status attn_decode_global_gated(const void* q, const void* kv_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, const float* gate, void* out,
                                   const da_shape* shape, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Decode-step preparation of the new token of every sequence on a sliding
 * layer (pages: Op Specs of google/gemma-4-12B, Norm.lean rmsnorm and
 * rmsnormUnit, Rope.lean rope; gemma-4-12b Model Spec, attn.qk_norm,
 * attn.v_norm and attn.rope rows of the sliding layers):
 *   q = rope(rmsnorm(q_raw) * w_q),  k = rope(rmsnorm(k_raw) * w_k),
 *   v = rmsnormUnit(v_raw),
 * per head, eps 1e-6, rope with theta 10^4 on all 256 coordinates (pairs
 * (i, i + 128), all 128 frequencies) at position positions[b]. q is written
 * to q_out; k and v are stored in slot positions[b] % 16 of page
 * block_table[b][positions[b] / 16] of k_cache and v_cache (row-major pages,
 * as attn_decode_sliding reads them). The token at position p is the
 * (p+1)-th cached token: call attn_decode_sliding afterwards with
 * seq_lens[b] = positions[b] + 1.
 *   q_raw [batch][Hkv*G][256], k_raw and v_raw [batch][Hkv][256], w_q and
 *   w_k [256]: fp32. q_out [batch][Hkv*G][256] and the caches: kv_dtype
 *   (bf16 values are rounded to nearest even). positions: int32 [batch].
 *   Sequences with positions[b] outside [0, 16*max_pages_per_seq) are left
 *   untouched (no q_out row, no cache write).
 *   Built shapes: head_dim 256, any Hkv and G. The block-table entry read must
 *   be a page of the pool; no other cache element is written.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_NO_DEVICE or
 * DA_ERR_LAUNCH.
 */
da_status attn_kv_append_sliding(const float* q_raw, const float* k_raw, const float* v_raw,
                                 const float* w_q, const float* w_k, const int32_t* block_table,
                                 const int32_t* positions, void* k_cache, void* v_cache, void* q_out,
                                 const da_shape* shape, void* stream);

/*
 * The same for a global layer (gemma-4-12b Model Spec, attn.qk_norm and
 * attn.rope rows of the global layers): one 512-wide projection kv_raw per
 * sequence and KV head is both k and v; q = rope(rmsnorm(q_raw) * w_q) and
 * k = rope(rmsnorm(kv_raw) * w_k) with theta 10^6 and only the first 64 of
 * the 256 frequencies active (pairs (i, i + 256), i < 64, rotated; the rest
 * unchanged). k is stored in the tiled K=V cache that attn_decode_global
 * reads as both keys and values.
 *   q_raw [batch][Hkv*G][512], kv_raw [batch][Hkv][512], w_q and w_k [512]:
 *   fp32. Built shapes: head_dim 512. Other conventions as above.
 */
da_status attn_kv_append_global(const float* q_raw, const float* kv_raw, const float* w_q,
                                const float* w_k, const int32_t* block_table, const int32_t* positions,
                                void* kv_cache, void* q_out, const da_shape* shape, void* stream);

/*
 * The decode-step append for the pre-norm cache of the global layers (the
 * cache attn_decode_global_prenorm reads): q as in attn_kv_append_global
 * (rmsnorm with w_q, then RoPE, theta 10^6, 64 active frequencies; Op Specs
 * Norm.lean and Rope.lean, Model Spec attn.qk_norm and attn.rope), and the
 * new token's shared projection x stored as it comes, rounded to bf16, in
 * slot positions[b] % 16 of page block_table[b][positions[b] / 16] of
 * x_cache [P][Hkv][64][16][8] (coordinate d of 32-wide block B = d / 32 in
 * chunk 32 (B % 2) + 4 (B / 2) + (d / 8) % 4, element d % 8). The k-norm
 * weight and the rotation of k are applied by the decode.
 *
 *   q_raw : fp32 [batch][Hkv*G][512];  x_raw : fp32 [batch][Hkv][512];
 *   w_q   : fp32 [512];  x_cache : bf16 pre-norm pages;  q_out : bf16
 *   [batch][Hkv*G][512]. shape: head_dim 512, kv_dtype BF16. Positions,
 *   block table, ownership, errors and asynchrony as for
 *   attn_kv_append_global.
 */
da_status attn_kv_append_global_prenorm(const float* q_raw, const float* x_raw, const float* w_q,
                                        const int32_t* block_table, const int32_t* positions, void* x_cache,
                                        void* q_out, const da_shape* shape, void* stream);

/*
 * Several queries per sequence (chunked prefill, speculative verification):
 * causalGQA and slidingGQA of the Op Specs (Attention.lean) with consecutive
 * query positions. Sequence b holds L = seq_lens[b] cached tokens, the last
 * S_b = q_start[b+1] - q_start[b] of which are its queries' own (written to
 * the cache before the call, e.g. by attn_kv_append_*); query s of sequence b
 * (q row q_start[b] + s) sits at position p = L - S_b + s and sees the keys
 * l <= p, and on sliding layers only those with p - window < l. A query with
 * p < 0 (S_b > L), or that sees no key, gets an all-zero output row.
 *
 *   q       : [T][Hkv*G][D] bf16, T = q_start[batch]; the rows of sequence b
 *             are q_start[b] .. q_start[b+1]-1.
 *   q_start : int32 [batch + 1] device array, q_start[0] = 0, non-decreasing.
 *   max_queries : host int, >= every S_b (sizes the grid; rows of a sequence
 *             past max_queries are not written). 1 .. 2^18.
 *   caches, block_table, seq_lens : as for the decode calls (sliding:
 *             k_cache, v_cache row-major; global: kv_cache tiled, read as
 *             both k and v). The block-table entries read are those of the
 *             positions some query sees.
 *   out     : [T][Hkv*G][D] fp32. q and out must not be NULL, also when
 *             T = 0 (a call without query rows reads and writes nothing).
 *   workspace : device buffer of at least attn_multiquery_workspace_bytes()
 *             bytes for the same shape, max_queries and window (0 bytes when
 *             the call needs none; may then be NULL). It holds per-piece
 *             partial results when a block's keys are split over several
 *             workgroups; no initialisation needed. Calls that share a
 *             workspace must be ordered (same stream).
 *
 * Built shapes: sliding (Hkv any, G = 2, D = 256), global (Hkv = 1, G = 16,
 * D = 512); bf16 caches only; batch * Hkv <= 65535. shape->num_splits > 0
 * forces the number of pieces per block (tests); 0 chooses it.
 */
da_status attn_multiquery_sliding(const void* q, const int32_t* q_start, int32_t max_queries,
                                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t window, void* out,
                                  const da_shape* shape, void* workspace, size_t workspace_bytes,
                                  void* stream);
da_status attn_multiquery_global(const void* q, const int32_t* q_start, int32_t max_queries,
                                 const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, void* out, const da_shape* shape,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* Workspace size of the multi-query call for this shape (head_dim 256:
 * sliding, 512: global), max_queries and window (ignored for global). Needs a
 * current gfx950 device (the split depends on its compute-unit count). */
da_status attn_multiquery_workspace_bytes(const da_shape* shape, int32_t max_queries, int32_t window,
                                          size_t* bytes);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(da_status status);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
