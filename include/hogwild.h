/*
 * hogwild.h -- C ABI of the Hogwild! concurrent-attention decode step on MI355X (gfx950).
 *
 * N workers decode together over ONE shared, paged KV cache. Each worker sees the cache's
 * blocks in its own view order; each block's keys are stored once, RoPE-rotated at
 * block-local positions 0..len-1, and a worker rotates its QUERY by each block's offset
 * instead of re-encoding the keys.
 *   [Hogwild! Inference paper summary, gentlecold.top] s5 "RoPE position rearrangement"
 *     (concatenation identity; procedure: store each block once, local positions from 0,
 *     per-worker block offsets, several rotations of the current query, per-block attention
 *     aggregated in one softmax); s6 (combined layout); s8 (step order: append, build views,
 *     attend); s9 (a block holds every layer's K/V at local positions; the view is computed
 *     at attention time; a Flash-Decoding style kernel balanced by KV entries followed by a
 *     reduction of partial results).
 *   [ocdem.com article on Hogwild! Inference] s2.1 (neighbour blocks in ascending worker
 *     ID), s2.2 (rotate q by the block offset; rotation is an isometry).
 *
 * Conventions fixed here (the pages leave them open):
 *   RoPE   pairs (j, j + d/2) rotated by pos * theta^(-2j/d). For stored keys, the fp32
 *          cos/sin of every position p < max_position is computed once on the host in fp64
 *          with libm cos/sin of (double)p * pow(theta, -(2.0*j)/d), rounded once to fp32.
 *   Query  q[w][h] is fp32 and unrotated. Row (w, h) reads KV head h / (Hq / Hkv).
 *          Score = (R(delta) q) . k_stored * softmax_scale, delta = q_pos - block offset.
 *          The decode kernel forms delta * theta_j / (2 pi) in fp64, reduces it to a fraction
 *          of a turn and takes the hardware's fp32 sine and cosine of that fraction.
 *          The rotated query and the softmax probabilities enter the matrix cores as bf16
 *          operands for bf16 pools (fp32 for fp32 pools); accumulation is fp32.
 *   Output out[w][h][:] fp32 and lse[w][h] = ln(sum_t exp(score_t)) fp32.
 *
 * Threading and streams: a context is not thread-safe. Use ONE stream per context for
 * hw_append_kv and hw_concurrent_decode; ordering between appends, decodes and page reuse
 * relies on that stream's order. Device faults surface at the caller's next synchronisation.
 *
 * Graph capture (HIP stream capture, e.g. torch.cuda.graph): a decode launches kernels only,
 * except when the views' device tables must be uploaded first (views set since the last
 * upload, or lengths of the views' blocks changed by appends or resets): then it copies
 * from pinned staging, which capture cannot hold, so during a capture it returns
 * HW_ERR_INVALID_ARG and enqueues nothing. Capture decodes after an eager decode with the
 * same views and lengths has uploaded the tables. Replays read the tables in the workspace
 * and are valid until the next upload (the next eager decode after the views or lengths
 * change); the split partials in the workspace are shared by every decode of the context,
 * so replays and eager work on the context must stay ordered on one stream. hw_append_kv
 * captures as kernels, but the host advances the blocks' lengths at capture time, not at
 * replay, so a captured append is replayed into the same slots: for steps that grow the
 * cache, capture under a step plan (hw_plan_steps below), whose appends and decodes take
 * their positions from device-side counters. No call records a memset node. hw_set_views
 * is host-only (nothing to order on a stream, hence no stream argument): it takes effect at
 * the next decode's upload.
 *
 * Errors: every call returns hw_status. Arguments and state are validated before anything
 * is mutated or enqueued: on any error other than HW_ERR_HIP nothing was enqueued and the
 * context is unchanged. HW_ERR_HIP reports a failed HIP call (a launch or a copy); the
 * context's host state is rolled back where the call mutated it. hw_last_error() explains
 * the last failure. Nothing throws or aborts across this ABI.
 */
#ifndef HOGWILD_H
#define HOGWILD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hw_ctx hw_ctx; /* opaque: host metadata and pinned staging only */

typedef enum {
  HW_OK = 0,
  HW_ERR_INVALID_ARG = 1,  /* bad pointer, id, size, dtype or configuration */
  HW_ERR_OUT_OF_PAGES = 2, /* the pool has too few free pages for an append */
  HW_ERR_STALE_VIEW = 3,   /* a view overlaps, repeats a block, or has a key after its query */
  HW_ERR_WORKSPACE = 4,    /* no workspace set, or too small */
  HW_ERR_HIP = 5           /* a HIP runtime call failed */
} hw_status;

typedef enum { HW_BF16 = 0, HW_F32 = 1 } hw_dtype;

typedef struct {
  int32_t n_layers;     /* layers whose K/V the pools hold */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t page_size;    /* tokens per page: a multiple of 32 */
  int32_t n_pages;      /* pages in the pool; page p names the same slots in every layer */
  int32_t max_blocks;   /* block ids are 0 .. max_blocks-1 */
  int32_t max_workers;  /* most workers any view set may have */
  int32_t max_position; /* every local position and every query offset delta must be below */
  int32_t max_splits;   /* most KV partitions per head a decode may use; 0 => 256 */
  int32_t max_query_tokens; /* most query tokens per worker of hw_concurrent_decode_tokens; 0 => 1 */
  hw_dtype kv_dtype;    /* element type of both pools */
  uint32_t page_seed;   /* 0: free pages handed out in ascending order; else shuffled (below) */
  double rope_theta;    /* RoPE base, > 1 */
  float softmax_scale;  /* 0 => 1/sqrt(head_dim) */
  /* Device pools, allocated and owned by the caller, each
   *   n_layers * n_pages * n_kv_heads * page_size * head_dim elements of kv_dtype,
   * 256-byte aligned. Within (layer, page, kv head) the page holds page_size/32 token
   * groups of 32 * head_dim elements; token t of the page is group t/32, u = t%32:
   *   K element (u, i) at (((i/32)*2 + (u/4)%2)*4 + (i%32)/8)*16*8 + (4*(u/8) + u%4)*8 + i%8
   *   V element (u, i) at (((i/16)*4 + u/8)*16 + i%16)*8 + u%8
   * so that every 64-lane, 16-byte-per-lane load of the decode kernel reads 1 KiB of
   * contiguous memory straight into the matrix-core operand layout. K holds rotated keys,
   * V raw values. The decode reads whole 32-token groups; the slots of a group that no token
   * occupies are masked out (their scores dropped, their values zeroed before use), so the
   * pools need no initialisation and may hold any bits, NaN included. */
  void *k_pool;
  void *v_pool;
} hw_config;

/* Create a context for cfg (copied). No device memory is allocated: the caller gives a
 * workspace with hw_set_workspace before the first append or decode. When page_seed != 0
 * the free list is a Fisher-Yates shuffle of page ids 0..n_pages-1: for i = n_pages-1 down
 * to 1, swap entries i and j = splitmix64() % (i + 1), where splitmix64 is Steele, Lea and
 * Flood's generator (state += 0x9E3779B97F4A7C15; z = state; z = (z ^ (z >> 30)) *
 * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB; return z ^ (z >> 31))
 * seeded with state = page_seed; pages are then handed out from entry 0 upward.
 * Errors: HW_ERR_INVALID_ARG for a bad configuration (out is then set to NULL). */
hw_status hw_create(const hw_config *cfg, hw_ctx **out);

/* Free the context's host memory and pinned staging. The caller must have synchronised the
 * stream it used. NULL is a no-op. */
hw_status hw_destroy(hw_ctx *ctx);

/* Text of the last error on ctx ("" if none); owned by ctx, valid until its next call.
 * With ctx == NULL: the last error of a failed context-free call (hw_create, or the
 * streaming-read probe of hogwild_debug.h) on this thread. */
const char *hw_last_error(const hw_ctx *ctx);

/* Bytes of device workspace the context needs: the fp32 cos/sin table
 * [max_position][head_dim/2][2], the per-decode tables (token groups and per-(block,
 * worker) query offsets) and the split partials. */
size_t hw_workspace_bytes(const hw_ctx *ctx);

/* Hand the context a device workspace of at least hw_workspace_bytes() bytes (256-byte
 * aligned, caller-owned, must outlive every call that uses it). Computes the cos/sin table
 * on the host and copies it synchronously, and allocates the context's pinned staging ring
 * for table uploads; this is setup, not a step: no later call allocates memory.
 * Errors: HW_ERR_WORKSPACE if too small or misaligned, HW_ERR_HIP on a copy or allocation
 * failure. */
hw_status hw_set_workspace(hw_ctx *ctx, void *dev, size_t bytes);

/* Append n_tokens[i] tokens to block block_ids[i] of one layer, for i < n_blocks
 * (summary s8: every worker appends its new token before views are built; s5 steps 1-2
 * and s9: stored once, at block-local positions). Block ids are caller-chosen; a block
 * comes into being with its first append and every block id may appear once per call.
 * k, v: device [sum n_tokens][n_kv_heads][head_dim] of kv_dtype, raw (unrotated), rows in
 * the order of block_ids. Token j of block b gets local position len(b, layer) + j; its key
 * is written as bf16_rne / fp32 of (a*c - b*s, b*c + a*s) with fp32 products and sums (no
 * fused multiply-add) and the table's cos/sin of that position; its value is copied.
 * Pages are shared by all layers of a block: a new page is taken from the free list when
 * the block's length in ANY layer first needs it. The call is all-or-nothing.
 * Errors: HW_ERR_INVALID_ARG (ids, counts, pointers, layer), HW_ERR_OUT_OF_PAGES,
 * HW_ERR_WORKSPACE, HW_ERR_INVALID_ARG if a position would reach max_position. */
hw_status hw_append_kv(hw_ctx *ctx, int32_t layer, int32_t n_blocks, const int32_t *block_ids,
                       const int32_t *n_tokens, const void *k, const void *v, void *stream);

/* Record the views of n_workers workers (host-only; nothing is enqueued). Worker w's view
 * is view_len[w] block ids, taken in order from view_blocks (summary s4/s6: common history,
 * other workers' current blocks in ascending worker ID, own block last; any order and any
 * subset of blocks is accepted). view_offsets: NULL, or one start position per listed
 * block (gaps allowed, overlaps rejected at decode time). q_pos: NULL, or one query
 * position per worker. Missing offsets default to the running sum of the blocks' lengths
 * and a missing q_pos to the last position of the view, both evaluated at decode time from
 * that layer's lengths. The arrays are copied.
 * Errors: HW_ERR_INVALID_ARG (counts, ids, repeated block in a view, negative values). */
hw_status hw_set_views(hw_ctx *ctx, int32_t n_workers, const int32_t *view_len,
                       const int32_t *view_blocks, const int64_t *view_offsets,
                       const int64_t *q_pos);

/* One decode step of one layer (summary s5 step 4-5, s9): for every worker w and query head
 * h, attention of q[w][h] over every token of w's view, computed as split-K partials over
 * the union of the views' blocks, balanced by KV entries, merged by log-sum-exp.
 * q: device fp32 [n_workers][n_q_heads][head_dim]; out: device fp32, same shape;
 * lse: device fp32 [n_workers][n_q_heads] or NULL. A worker whose view holds no token gets
 * out = 0 and lse = -inf. The views' device tables are uploaded (pinned staging, async copy
 * on stream) only when the views or the lengths of their blocks changed since the last
 * upload, so layers with equal lengths share one upload.
 * Errors: HW_ERR_INVALID_ARG, HW_ERR_WORKSPACE, HW_ERR_STALE_VIEW (no views set, more
 * workers than max_workers, overlapping blocks, a key position above the worker's q_pos, or
 * a delta at or above max_position), HW_ERR_HIP. */
hw_status hw_concurrent_decode(hw_ctx *ctx, int32_t layer, const float *q, float *out,
                               float *lse, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): hw_concurrent_decode with the split partials kept in a
 * static device array of the library (16 MiB per GPU, held until the process ends) instead
 * of the workspace. Same arguments, kernels and results as hw_concurrent_decode; it calls no
 * hipMalloc, hipFree or other routine that allocates device or pinned memory (the pinned
 * staging ring and the array's address are set up by hw_set_workspace). Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one GPU, from any context or stream, race.
 * Errors: as hw_concurrent_decode; HW_ERR_WORKSPACE when the partials of the partition count
 * the decode would use (partitions x n_kv_heads x n_workers x (n_q_heads / n_kv_heads) x
 * (head_dim + 1) fp32) do not fit 16 MiB: force fewer with hw_set_split. */
hw_status hw_concurrent_decode_noalloc(hw_ctx *ctx, int32_t layer, const float *q, float *out,
                                       float *lse, void *stream);

/* Several query tokens per worker in one pass (summary s8 step 4: a worker that starts a
 * fresh block first inserts a paragraph header, whose tokens are appended and attended
 * together). q: device fp32 [n_workers][n_new][n_q_heads][head_dim], raw. Token t of worker
 * w sits at position q_pos(w) - (n_new - 1 - t), q_pos(w) being the position
 * hw_concurrent_decode uses (the last token), and attends to the keys of w's view at or
 * before its own position: causal, so a block's keys after the token (this step's later
 * tokens of the worker's own block) are left out. out: device fp32, same shape as q; lse:
 * device fp32 [n_workers][n_new][n_q_heads] or NULL. A token with no key at or before it
 * gets out = 0 and lse = -inf. n_new = 1 computes what hw_concurrent_decode computes.
 * Errors: as hw_concurrent_decode; HW_ERR_INVALID_ARG when n_new < 1 or n_new >
 * max_query_tokens; HW_ERR_STALE_VIEW when a worker's first token would sit below 0. */
hw_status hw_concurrent_decode_tokens(hw_ctx *ctx, int32_t layer, int32_t n_new, const float *q,
                                      float *out, float *lse, void *stream);

/* ---- Step plans: a whole decode step, appends included, with no host work inside --------
 * The pages' step (summary s8) is: every worker appends its token, the views are rebuilt,
 * attention runs. Between two steps of one paragraph the views keep their blocks and only
 * the lengths grow, so with default offsets every quantity a decode reads is affine in the
 * number of steps taken: each block's length, each group's token count and each (worker,
 * block) query offset (the sum of the lengths from that block to the end of the worker's
 * view, minus one). A step plan resolves the views once for a window of n_steps steps and
 * keeps, per layer, a device-side count of the planned steps done; the append and the
 * decode kernels derive the step's positions, group sizes and offsets from it, and the
 * decode's last kernel advances it.
 * A step (per layer: hw_append_step, then hw_concurrent_decode) then performs no host-side
 * resolution, no staging wait and no copy: it can be captured once as a HIP graph and
 * replayed for each step of the window.
 *
 * hw_plan_steps: block_ids[i] grows by tokens_per_step[i] tokens per step in every layer,
 * for i < n_blocks (each id once; any other block of the views stays as it is). Needs
 * bf16 pools, views set with default offsets and query positions (hw_set_views with NULL
 * view_offsets and q_pos), and every block of the views and of the plan at the same length
 * in every layer. Takes the pages of the whole window from the free list now, resolves the
 * views' tables for the window (the groups the blocks will have at its end; a group's token
 * count is clamped to 0..32 at each step), chooses the partitions as a decode would (or as
 * hw_set_split forces), uploads the tables, zeroes the step counters and waits for the
 * upload on `stream`. While a plan is active, hw_append_kv, hw_set_views, hw_reset_block,
 * hw_set_workspace and hw_debug_reserve return HW_ERR_INVALID_ARG, decodes read the plan's
 * tables, hw_concurrent_decode_tokens takes n_new = 1 only, and hw_block_info reports the
 * lengths the blocks had when the plan began.
 * Errors: HW_ERR_INVALID_ARG (a plan already active, fp32 pools, explicit offsets or q_pos,
 * ids, counts, lengths that differ between layers, a block that would reach max_position;
 * more than 64 planned blocks, 1024 tokens per step or 512 pages written in the window),
 * HW_ERR_STALE_VIEW (no views, or a view that would reach max_position within the window),
 * HW_ERR_OUT_OF_PAGES, HW_ERR_WORKSPACE, HW_ERR_HIP; on any error nothing changed. Not
 * capturable (it uploads and waits). */
hw_status hw_plan_steps(hw_ctx *ctx, int32_t n_steps, int32_t n_blocks, const int32_t *block_ids,
                        const int32_t *tokens_per_step, void *stream);

/* One planned step's append for one layer (summary s8: append before attention; s5 steps
 * 1-2: stored once, RoPE'd at block-local positions). k, v: device [rows][n_kv_heads]
 * [head_dim] bf16, raw, 16-byte aligned, rows = sum of tokens_per_step, in the plan's
 * block order. Planned
 * block i's tokens go to local positions base_i + s * tokens_per_step[i] + j, s being the
 * number of planned steps this layer has completed, written as hw_append_kv writes them
 * (one workgroup per token). The layer's next hw_concurrent_decode attends over them and,
 * after its kernels have read the count, advances it (with the split merge, or a one-thread
 * kernel when the decode needs no merge): a layer's planned step is hw_append_step then
 * hw_concurrent_decode, and a decode without an append before it sees the count as it is.
 * An append past the window's n_steps writes nothing and is reported by hw_plan_end.
 * Capturable: enqueues one kernel and reads nothing from the host.
 * Errors: HW_ERR_INVALID_ARG (no plan, layer, NULL or misaligned k/v, or a second append of
 * the layer before its decode), HW_ERR_HIP. */
hw_status hw_append_step(hw_ctx *ctx, int32_t layer, const void *k, const void *v, void *stream);

/* One planned step of one layer with its append fused into the decode (summary s8: the
 * step's tokens are appended, then attended): the same results, pool bytes and counts as
 * hw_append_step(layer, k, v) followed by hw_concurrent_decode(layer, q, out, lse), in one
 * decode launch (plus the split merge) instead of two. Each (KV head, token group) is read by
 * one wave of the decode; the wave whose groups the step's tokens fall in writes those tokens
 * for its KV head before reading them, so no other synchronisation is needed. k, v as for
 * hw_append_step; q, out, lse as for hw_concurrent_decode. Capturable (no host work).
 * Errors: as hw_append_step and hw_concurrent_decode; HW_ERR_INVALID_ARG when the plan has a
 * growing block that no view holds, or more query rows per KV head than one decode
 * workgroup takes (64 for bf16): use the two calls then. A step past the window writes
 * nothing and is reported by hw_plan_end. */
hw_status hw_decode_step(hw_ctx *ctx, int32_t layer, const void *k, const void *v, const float *q,
                         float *out, float *lse, void *stream);

/* End the active plan: waits for `stream`, reads the device's per-layer counts of planned
 * steps back (a layer appended but not yet decoded counts its append), sets every planned
 * block's length in each layer to base + count * tokens_per_step, and returns the pages
 * the blocks did not fill to the free list. Views
 * and tables are then as without a plan (the next decode uploads fresh tables).
 * Errors: HW_ERR_INVALID_ARG if no plan is active, or if some layer had more planned appends
 * than n_steps (the extra appends were dropped; the plan is ended all the same); HW_ERR_HIP. */
hw_status hw_plan_end(hw_ctx *ctx, void *stream);

/* Return a block's pages to the free list and set its length to 0 in every layer, e.g. after
 * its step was committed and the worker starts a fresh block (summary s8). Pages are handed
 * out again first-in-block-order-first. Later appends reuse them in stream order, so work
 * already enqueued on the context's stream still reads the old contents. */
hw_status hw_reset_block(hw_ctx *ctx, int32_t block_id);

/* Force the number of KV partitions per head for following decodes (1 .. max_splits), or
 * 0 for the automatic choice: workgroups for about three quarters of the compute units (all
 * of them with several query tokens per worker), at least 4 token groups a partition, and a
 * single partition for heads of at most 16 groups. */
hw_status hw_set_split(hw_ctx *ctx, int32_t n_splits);

/* Introspection: a block's length in a layer and its page ids in order (at most cap are
 * written; *n_out receives the count). */
hw_status hw_block_info(const hw_ctx *ctx, int32_t block_id, int32_t layer, int32_t *length,
                        int32_t *pages, int32_t cap, int32_t *n_out);

/* Introspection: pages currently on the free list. */
hw_status hw_free_pages(const hw_ctx *ctx, int32_t *n_free);

#ifdef __cplusplus
}
#endif

#endif /* HOGWILD_H */
