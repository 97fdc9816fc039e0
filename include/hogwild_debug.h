/*
 * hogwild_debug.h -- host-only introspection of the Hogwild! decode library, for tests.
 *
 * Apart from the profiling hooks and the streaming-read probe at the end, these calls touch
 * no GPU and enqueue nothing, so the host logic (slot assignment, page
 * allocation, view resolution, validation) can be checked bit-exactly on a machine without
 * a GPU. Same status codes and validation rules as hogwild.h.
 */
#ifndef HOGWILD_DEBUG_H
#define HOGWILD_DEBUG_H

#include "hogwild.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The host half of hw_append_kv without the kernel: validates, takes pages from the free
 * list and advances the blocks' lengths exactly as hw_append_kv would, WITHOUT writing any
 * K/V (the pool slots keep whatever they held). Writes the copy plan to runs[cap][5]:
 * {input row of the first token, page id, first token slot in the page, token count,
 * local position of the first token}; one run never crosses a page. *n_runs gets the
 * count even when it exceeds cap (then nothing is mutated and HW_ERR_INVALID_ARG is
 * returned). Blocks cited by the pages' append step: summary s8, s9. */
hw_status hw_debug_reserve(hw_ctx *ctx, int32_t layer, int32_t n_blocks, const int32_t *block_ids,
                           const int32_t *n_tokens, int32_t *runs, int32_t cap, int32_t *n_runs);

/* The view resolution hw_concurrent_decode would upload for `layer` (summary s5 step 3,
 * s9: each block's start in each worker's view -> the query rotation per (worker, block)).
 *   segs[cap_segs]                 block id of each segment of the union of the views, in
 *                                  order of first appearance (worker 0's view first)
 *   delta[cap_segs][n_workers]     q_pos(w) - offset(w, block), or -1 if w does not see it
 *   groups[cap_groups][4]          {page, 32-token group within the page, segment, valid
 *                                  tokens 1..32} of every token group of every segment
 *   *n_splits                      KV partitions per head a decode would use now
 * Counts are written even when they exceed the caps (then the arrays are left untouched and
 * HW_ERR_INVALID_ARG is returned). Validation failures return HW_ERR_STALE_VIEW. */
hw_status hw_debug_resolve(hw_ctx *ctx, int32_t layer, int32_t *segs, int32_t *delta,
                           int32_t cap_segs, int32_t *n_segs, int32_t *groups,
                           int32_t cap_groups, int32_t *n_groups, int32_t *n_splits);

/* The partition of a group list into KV partitions that hw_concurrent_decode uses (host
 * only, no context). block_first[n_groups]: 1 where a group starts a new block of the union
 * (group 0 always counts as one). A partition costs 1 per group plus alpha per block it
 * touches; bounds[n_splits + 1] receives cuts 0 = bounds[0] <= ... <= bounds[n_splits] =
 * n_groups (partition p = groups [bounds[p], bounds[p + 1]); trailing ones may be empty)
 * whose largest partition cost is minimal up to one group's cost. Decodes use alpha 0 for
 * up to 32 rows per workgroup and a measured per-block weight for the cooperative kernels
 * (33..64 bf16 rows), with at most 255 partitions (beyond that, uniform cuts
 * p * n_groups / n_splits). Errors: HW_ERR_INVALID_ARG (n_groups < 0, n_splits < 1,
 * alpha < 0 or NaN, NULL arrays); hw_last_error(NULL) then explains. */
hw_status hw_debug_partition(const uint8_t *block_first, int32_t n_groups, int32_t n_splits,
                             double alpha, int32_t *bounds);

/* ---- profiling hooks (these two do call HIP) ---------------------------------------------
 * With capacity > 0, each following hw_concurrent_decode has its concurrent_decode kernel
 * (not the split merge that follows it) record a start and a stop HIP event with its own
 * dispatch, for up to `capacity` calls; capacity 0 stops recording and frees the events.
 * Errors: HW_ERR_HIP. */
hw_status hw_debug_kernel_events(hw_ctx *ctx, int32_t capacity);

/* Wait for the recorded events and write, per recorded call i < cap, decode_ms[i]: the
 * duration of that call's concurrent_decode kernel. *n receives the number of recorded
 * calls; recording then restarts at zero. */
hw_status hw_debug_kernel_elapsed(hw_ctx *ctx, float *decode_ms, int32_t cap, int32_t *n);

/* Measurement aid, independent of any context: n_blocks workgroups of 256 threads read the
 * `bytes` bytes at `src` (device, 16-byte aligned, bytes a positive multiple of 16) once,
 * each workgroup a contiguous 1/n_blocks of them, with 16-byte streaming loads, four in
 * flight per thread. Nothing is written unless an impossible checksum turns up (then one
 * float per workgroup goes to sink[n_blocks], device); the read bandwidth it achieves is the
 * streaming ceiling the decode kernel is compared with. Enqueued on `stream`. elapsed_ms:
 * NULL, or it receives the kernel's duration from start/stop events recorded by the
 * kernel's own dispatch, and the call then waits for the kernel.
 * Errors: HW_ERR_INVALID_ARG (pointers, alignment, sizes, n_blocks outside 1..65535),
 * HW_ERR_HIP; hw_last_error(NULL) then explains, on the calling thread. */
hw_status hw_debug_stream_read(const void *src, size_t bytes, float *sink, int32_t n_blocks,
                               void *stream, float *elapsed_ms);

#ifdef __cplusplus
}
#endif

#endif /* HOGWILD_DEBUG_H */
