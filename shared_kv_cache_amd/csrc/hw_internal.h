// Internal interface between the host core (hw_host.cpp) and the gfx950 kernels
// (hw_kernels.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hogwild.h"

namespace hw {

constexpr int kTokGroup = 32;          // tokens per pool group (one MFMA K/V tile)
constexpr int kRowsPerBlock = 64;      // stacked (worker, query head) rows per decode workgroup
constexpr int kRowsPerBlockF32 = 16;   // the same for fp32 pools (exact-check path; wider operands)

// bf16 with several query tokens per worker: rows of 32 (8-wave kernels, each wave rotating
// as it enters a block). Measured on MI355X with 4 tokens per worker, against 64-row
// cooperative blocks: w4_16k 36.7 against 59.7 us per layer, w8_32k 128 against 178 us,
// although each extra row block reads the partition's K/V again; 16 rows were slower.
constexpr int kRowsPerBlockMT = 32;
inline int rows_per_block(hw_dtype dt, int n_new = 1) {
  return dt == HW_F32 ? kRowsPerBlockF32 : (n_new > 1 ? kRowsPerBlockMT : kRowsPerBlock);
}
// Waves per decode workgroup when each KV head has `rows` stacked rows (launch_decode's
// choice): bf16 blocks of up to 32 rows run on 8 waves, of 33..64 rows on 4; fp32 on 8.
inline int decode_waves(hw_dtype dt, int rows, int n_new = 1) {
  const int first = rows < rows_per_block(dt, n_new) ? rows : rows_per_block(dt, n_new);
  return (dt == HW_BF16 && first > 32) ? 4 : 8;
}
constexpr int kMaxRunsPerLaunch = 64;  // append runs carried in one launch's arguments
constexpr int kMaxBoundSplits = 255;   // partitions whose group bounds ride in the launch arguments
// Up to this many workers, 8-wave decodes read "wide" group descriptors: 8 ints per group,
// {group index of head 0, segment << 8 | valid tokens, query offset of workers 0..5 for the
// group's segment (-1: not visible; unused slots -1)}, so a group's offsets arrive with its
// descriptor through the scalar cache.
constexpr int kWideWorkers = 6;
constexpr int kWideStride = 8;


// One run of appended tokens: consecutive tokens of one block inside one page.
struct AppendRun {
  int32_t src_row;  // row of the first token in the caller's k/v input
  int32_t page;     // pool page
  int32_t slot0;    // first token slot within the page
  int32_t count;    // tokens
  int32_t pos0;     // block-local position of the first token
};

struct AppendArgs {
  void *k_layer;          // pool base of the layer
  void *v_layer;
  const void *k_src;      // [rows][n_kv_heads][head_dim]
  const void *v_src;
  const float2 *trig;     // [max_position][head_dim/2] (cos, sin)
  int32_t n_kv_heads;
  int32_t page_groups;    // page_size / 32
  int32_t n_runs;
  AppendRun runs[kMaxRunsPerLaunch];
};

struct DecodeArgs {
  // The first 96 bytes hold what the decode kernel's prologue needs; it reads them in one
  // batch of scalar loads (the offsets are checked by static_asserts in the kernel file).
  const void *k_layer;
  const void *v_layer;
  const float *q;          // [n_workers][n_q_heads][head_dim]
  const int2 *groups;      // [n_groups] {group index of head 0, segment << 8 | valid tokens}
                           // (desc_stride 2); with the group's first local position as a
                           // third int (desc_stride 4, several query tokens per worker); or
                           // wide descriptors (desc_stride = kWideStride ints per group)
  const double *turn_freq; // [head_dim/2] theta^(-2j/d) / (2 pi): rotation turns per position
  int32_t n_groups;
  int32_t n_splits;
  int32_t rows;            // stacked rows per KV head: n_workers * n_new * group
  int32_t rows_per_block;  // rows handled by one workgroup (grid z = row blocks)
  int32_t group;           // n_q_heads / n_kv_heads
  int32_t n_q_heads;
  int32_t page_groups;
  int32_t desc_stride;     // ints per group descriptor: 2, 4, or kWideStride (8-wave kernels only)
  float inv_group;         // 1 / group (rows < 2^22, so the query token of a row is exact in fp32)
  float q_scale;           // softmax_scale * log2(e)
  float inv_rpw;           // 1 / (n_new * group): rows per worker
  int32_t n_new;           // query tokens per worker (rows = n_workers * n_new * group)
  int32_t n_workers;
  int32_t n_kv_heads;
  float *out;              // [n_workers][n_q_heads][head_dim]   (written when n_splits == 1)
  float *lse;              // [n_workers][n_q_heads] or null      (idem)
  const int32_t *delta;    // [n_segments][n_workers] query offset, -1 = not visible
  float *part_o;           // [n_splits][n_kv_heads][rows][head_dim] normalised partial outputs
  float *part_lse;         // [n_splits][n_kv_heads][rows] log2-domain partial normalisers
  // Step plan: the layer's counter of planned appends (null: no plan). Descriptors are then
  // {x, segment << 8, v0, rate} and delta holds {d0, rate} pairs (see the kernel). The
  // decode sees min(counter + plan_pending, plan_n_steps) steps: plan_pending is 1 when this
  // step's append was enqueued before the decode (the counter advances after the decode).
  const int32_t *plan_step;
  int32_t plan_pending;
  int32_t plan_n_steps;
  // Fused step (hw_decode_step; null fuse_k: none): the layer's planned append, written by
  // the decode's own waves before they read the groups it fills. fuse_blocks[i] = {base
  // length, tokens per step, first input row, index in the group list of the block's first
  // group}; fuse_overflow is set to 1 by a step past the window (nothing is then written).
  const void *fuse_k;      // [rows][n_kv_heads][head_dim] bf16, rows in planned-block order
  const void *fuse_v;
  const float2 *fuse_trig; // [max_position][head_dim/2] (cos, sin)
  const int32_t *fuse_blocks;
  int32_t *fuse_overflow;
  int32_t fuse_n_blocks;
  int32_t fuse_gmin, fuse_gmax;   // list indices of the first and last group the window appends to
  // Partition p takes groups [split_begin[p], split_begin[p + 1]) when n_splits <=
  // kMaxBoundSplits (host-chosen, cost-balanced bounds); else [p * n_groups / n_splits, ...).
  int32_t split_begin[kMaxBoundSplits + 1];
};


hipError_t launch_append(hw_dtype dt, int head_dim, const AppendArgs &a, hipStream_t s);

// The append of one planned step of one layer (a step plan, hw_plan_steps): every planned
// block b takes its tokens_per_step tokens at local positions base(b) + s * tps(b) + j, s
// being the layer's counter of planned appends. The counter is NOT advanced here (every
// workgroup reads it): the kernel that follows the layer's decode advances it (the merge,
// or advance_kernel). The planned blocks and the ids of the pages the window writes ride in
// the launch arguments, so that the only dependent loads are the counter and the rope
// table's rows.
constexpr int kMaxPlanBlocks = 64;
constexpr int kMaxPlanPages = 512;
constexpr int kMaxPlanRows = 1024;   // tokens per planned step, all blocks
struct PlanBlock {
  int32_t base;       // length when the plan began
  int32_t tps;        // tokens per step
  int32_t row0;       // first input row of the block's tokens
  int32_t page0;      // index, in the block's page list, of the first page the window writes
  int32_t pages_off;  // where that page's id sits in PlanAppendArgs::pages
};
struct PlanAppendArgs {
  void *k_layer;
  void *v_layer;
  const void *k_src;       // [rows][n_kv_heads][head_dim], rows in planned-block order
  const void *v_src;
  const float2 *trig;      // [max_position][head_dim/2] (cos, sin)
  const int32_t *step;     // the layer's counter of planned appends
  int32_t *overflow;       // set to 1 by an append past the plan's last step (dropped)
  int32_t n_blocks;
  int32_t rows;            // tokens per step, all planned blocks
  int32_t n_steps;
  int32_t n_kv_heads;
  int32_t page_size;
  int32_t page_groups;
  PlanBlock blocks[kMaxPlanBlocks];
  int32_t pages[kMaxPlanPages];
};
hipError_t launch_plan_append(hw_dtype dt, int head_dim, const PlanAppendArgs &a, hipStream_t s);
struct MergeArgs {
  const float *part_o;
  const float *part_lse;
  float *out;
  float *lse;
  int32_t n_workers;   // query tokens: workers x tokens per worker, in (worker, token) order
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t group;
  int32_t rows;
  int32_t n_splits;
  // Step plan: a layer counter to advance (by one, up to advance_cap) once the decode before
  // this merge has read it; null: none.
  int32_t *advance;
  int32_t advance_cap;
};

// Advance a step plan's layer counter by one (up to cap): one thread, for decodes that
// write their output directly (no merge follows them).
hipError_t launch_advance(int32_t *counter, int32_t cap, hipStream_t s);

hipError_t launch_merge(int head_dim, const MergeArgs &a, hipStream_t s);

// Size of the static scratch that hw_concurrent_decode_noalloc keeps its split partials in,
// and its device address on the current device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t scratch_address(void **ptr);
hipError_t launch_stream_read(const void *src, size_t bytes, float *sink, int n_blocks, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop);
// ev_start/ev_stop: optional events recorded by the kernel's own dispatch (may be null).
hipError_t launch_decode(hw_dtype dt, int head_dim, const DecodeArgs &a, int row_blocks,
                         hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace hw
