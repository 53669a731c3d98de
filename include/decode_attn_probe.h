/*
 * decode_attn_probe.h - HBM read probe that ships beside the attention
 * library (libdecode_attn_probe.so). It is measurement support, not part of
 * the attention path: it reads whole KV-sized pages with the same access
 * pattern as the decode kernels (16 KB pages in block-table order, 16-byte
 * non-temporal loads) and computes nothing, so its time gives the read
 * bandwidth that pattern can reach on the device the kernels run on.
 */
#ifndef DECODE_ATTN_PROBE_H
#define DECODE_ATTN_PROBE_H

#include <stdint.h>

#include "decode_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads pages page_ids[0 .. num_pages) of `base`, each 16384 bytes, page p
 * at base + 16384 * page_ids[p]. The list is split into `workgroups`
 * contiguous, equal ranges (one per workgroup of 256 threads) that each
 * keep four pages of loads in flight.
 *
 *   base       : device pointer, 16-byte aligned, caller-owned; only read.
 *   page_ids   : device int32 [num_pages]; every entry must lie inside the
 *                caller's buffer (not checked: that needs a device sync).
 *   num_pages  : >= 0 (0 enqueues nothing).
 *   workgroups : 1 .. 65535.
 *   sink       : device uint32 [1]; written only when the xor of everything
 *                read equals a fixed constant (keeps the loads from being
 *                removed); its contents carry no meaning.
 *   stream     : hipStream_t; NULL = the null stream. Asynchronous.
 *
 * Returns DA_OK, DA_ERR_INVALID_ARG (a null pointer or a size out of range;
 * nothing enqueued) or DA_ERR_LAUNCH.
 */
da_status da_probe_read_pages(const void* base, const int32_t* page_ids, int32_t num_pages,
                              int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_PROBE_H */
