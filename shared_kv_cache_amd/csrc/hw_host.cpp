// Host core of the Hogwild! concurrent-attention decode library: context, page pool,
// block registry, view resolution and the C ABI (include/hogwild.h, hogwild_debug.h).
//
// [Hogwild! Inference paper summary, gentlecold.top]
//   s5  the concatenation identity and its five steps: each block stored once, local
//       positions from 0, per-worker block offsets, a query rotation per block, one softmax;
//   s8  the step: every worker appends its token, then each worker's view is built, then
//       attention runs with the per-block query rotation;
//   s9  the cache is a common block plus one current block per worker, each holding every
//       layer's K/V at local positions; the view is computed at attention time; the kernel
//       balances work by KV entries and reduces partial results.
// [ocdem.com article on Hogwild! Inference] s2.1 neighbour blocks in ascending worker ID
//   (the caller's view lists carry that order); s3.1 page-table metadata (owner, paragraph)
//   is the caller's: this library keys blocks by caller-chosen ids only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "hogwild.h"
#include "hogwild_debug.h"
#include "hw_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kStagingSlots = 4;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct BlockState {
  std::vector<int32_t> pages;  // page ids in block order (shared by all layers)
  std::vector<int32_t> len;    // tokens per layer
  int32_t max_len() const {
    int32_t m = 0;
    for (int32_t x : len) m = std::max(m, x);
    return m;
  }
};

struct Views {
  bool set = false;
  int32_t n_workers = 0;
  std::vector<std::vector<int32_t>> blocks;
  std::vector<std::vector<int64_t>> offsets;  // empty inner vectors: running sum
  bool has_offsets = false;
  std::vector<int64_t> q_pos;
  bool has_qpos = false;
  uint64_t version = 0;
};

// What one decode uploads: per-(segment, worker) query offsets and the token-group list.
struct Resolution {
  std::vector<int32_t> seg_blocks;
  std::vector<int32_t> delta;   // [n_seg][n_workers]
  std::vector<int32_t> g_page, g_gip, g_seg, g_valid, g_start;   // g_start: local position
  int32_t n_workers = 0;
  // smallest query position over the workers whose view holds a token
  int64_t min_qpos = std::numeric_limits<int64_t>::max();
};

// A step plan (hw_plan_steps): blocks that grow by a fixed number of tokens per step in
// every layer, over a window of steps, with the views' tables resolved once for the whole
// window (affine in each layer's device-side count of planned appends).
struct Plan {
  bool active = false;
  int32_t n_steps = 0;
  std::vector<int32_t> blocks, tps, base;   // planned blocks, tokens per step, base lengths
  int32_t rows = 0;                         // tokens per step over all planned blocks
  int32_t n_workers = 0, n_groups = 0, splits = 1;
  std::vector<int32_t> bounds;              // partition bounds (splits <= kMaxBoundSplits)
  std::vector<hw::PlanBlock> append_blocks; // the planned append's launch arguments
  std::vector<int32_t> append_pages;
  // hw_decode_step: every growing planned block is in some view (its groups are in the
  // list, so some decode wave writes each of its tokens) and the decode has one row block
  bool fusable = false;
  int32_t fuse_gmin = 0, fuse_gmax = -1;    // group-list range the window's appends fall in
  // per layer: 1 while the step's append is enqueued and its decode not yet (the layer's
  // counter advances after that decode)
  std::vector<uint8_t> pending;
};

}  // namespace

struct hw_ctx {
  hw_config cfg{};
  std::vector<BlockState> blocks;
  std::vector<int32_t> free_stack;  // back() is handed out next
  uint64_t page_generation = 0;     // bumped whenever a page leaves a block
  Views views;
  std::string err;
  int32_t split_override = 0;
  int32_t num_cus = 256;

  // device workspace carve-up
  void *ws = nullptr;
  size_t ws_bytes = 0;
  size_t off_trig = 0, off_freq = 0, off_tables = 0, off_part_o = 0, off_part_lse = 0;
  size_t tables_bytes = 0;
  // step-plan region: counters [n_layers] + overflow flag, the fused step's per-block table,
  // {d0, rate} offsets, 4-int group descriptors
  size_t off_plan = 0, plan_cnt = 0, plan_fuse = 0, plan_delta = 0, plan_groups = 0;
  Plan plan;
  size_t part_o_bytes = 0, part_lse_bytes = 0, total_bytes = 0;

  // upload cache
  std::vector<int64_t> uploaded_sig;
  bool uploaded_valid = false;
  int32_t up_n_groups = 0, up_n_seg = 0, up_n_workers = 0;
  size_t up_groups_off = 0;  // byte offset of the group list inside the tables region
  int32_t up_stride = 2;     // ints per uploaded group descriptor
  int64_t up_min_qpos = 0;   // Resolution::min_qpos of the uploaded tables
  std::vector<uint8_t> up_seg_first;   // per group: 1 if it starts a block of the union
  // partition bounds of the uploaded group list, for bounds_splits partitions at bounds_alpha
  std::vector<int32_t> bounds;
  int32_t bounds_splits = -1;
  double bounds_alpha = -1.0;

  // pinned staging ring
  char *staging = nullptr;
  hipEvent_t events[kStagingSlots] = {};
  bool event_live[kStagingSlots] = {};
  int next_slot = 0;
  bool debug_sync = false;

  // device address of the static scratch on the context's device (hw_set_workspace)
  void *scratch = nullptr;

  // profiling hooks: two events per recorded decode call
  std::vector<hipEvent_t> prof_events;
  int32_t prof_capacity = 0, prof_count = 0;

  hw_status fail(hw_status s, const std::string &m) {
    err = m;
    return s;
  }
};

namespace {

thread_local std::string g_create_error;

uint64_t splitmix64_next(uint64_t &state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// Stacked query rows of one KV head: (worker, query token, head of the KV head's group).
int32_t rows_total(const hw_ctx *c, int32_t n_workers, int32_t n_new = 1) {
  return n_workers * n_new * (c->cfg.n_q_heads / c->cfg.n_kv_heads);
}

void layout_workspace(hw_ctx *c) {
  const hw_config &g = c->cfg;
  const size_t half = (size_t)g.head_dim / 2;
  const size_t max_groups = (size_t)g.n_pages * (g.page_size / hw::kTokGroup);
  const size_t max_rows = (size_t)g.max_workers * g.max_query_tokens * (g.n_q_heads / g.n_kv_heads);
  size_t off = 0;
  c->off_trig = off;
  off = align_up(off + (size_t)g.max_position * half * 2 * sizeof(float));
  c->off_freq = off;
  off = align_up(off + half * sizeof(double));
  c->off_tables = off;
  c->tables_bytes = align_up((size_t)g.max_blocks * g.max_workers * sizeof(int32_t)) +
                    align_up(max_groups * hw::kWideStride * sizeof(int32_t));
  off = align_up(off + c->tables_bytes);
  c->off_part_o = off;
  c->part_o_bytes = (size_t)g.max_splits * g.n_kv_heads * max_rows * g.head_dim * sizeof(float);
  off = align_up(off + c->part_o_bytes);
  c->off_part_lse = off;
  c->part_lse_bytes = (size_t)g.max_splits * g.n_kv_heads * max_rows * sizeof(float);
  off = align_up(off + c->part_lse_bytes);
  c->off_plan = off;
  size_t po = 0;
  c->plan_cnt = po;
  po = align_up(po + ((size_t)g.n_layers + 1) * sizeof(int32_t));
  c->plan_fuse = po;
  po = align_up(po + (size_t)hw::kMaxPlanBlocks * 4 * sizeof(int32_t));
  c->plan_delta = po;
  po = align_up(po + (size_t)g.max_blocks * g.max_workers * 2 * sizeof(int32_t));
  c->plan_groups = po;
  po = align_up(po + max_groups * 4 * sizeof(int32_t));
  off = align_up(off + po);
  c->total_bytes = off;
}

hw_status check_config(const hw_config *g, std::string &m) {
  if (!g) return m = "cfg is NULL", HW_ERR_INVALID_ARG;
  if (g->n_layers <= 0) return m = "n_layers must be > 0", HW_ERR_INVALID_ARG;
  if (g->n_kv_heads <= 0 || g->n_q_heads <= 0 || g->n_q_heads % g->n_kv_heads)
    return m = "n_q_heads must be a positive multiple of n_kv_heads", HW_ERR_INVALID_ARG;
  if (g->head_dim != 64 && g->head_dim != 128) return m = "head_dim must be 64 or 128", HW_ERR_INVALID_ARG;
  if (g->page_size <= 0 || g->page_size % hw::kTokGroup || g->page_size > 8192)
    return m = "page_size must be a multiple of 32 in [32, 8192]", HW_ERR_INVALID_ARG;
  if (g->n_pages <= 0) return m = "n_pages must be > 0", HW_ERR_INVALID_ARG;
  if (g->max_blocks <= 0 || g->max_blocks > (1 << 22)) return m = "max_blocks out of range", HW_ERR_INVALID_ARG;
  if (g->max_workers <= 0 || g->max_workers > 1024) return m = "max_workers out of range", HW_ERR_INVALID_ARG;
  if (g->max_position <= 0) return m = "max_position must be > 0", HW_ERR_INVALID_ARG;
  if (g->max_query_tokens < 0 || g->max_query_tokens > 1024)
    return m = "max_query_tokens must be in [0, 1024]", HW_ERR_INVALID_ARG;
  const int64_t mqt = std::max<int64_t>(1, g->max_query_tokens);
  if ((int64_t)g->max_workers * mqt * (g->n_q_heads / g->n_kv_heads) >= (1 << 22))
    return m = "max_workers * max_query_tokens * (n_q_heads / n_kv_heads) must be below 2^22",
           HW_ERR_INVALID_ARG;
  if ((int64_t)g->max_workers * mqt * g->n_q_heads * g->head_dim >= ((int64_t)1 << 31))
    return m = "max_workers * max_query_tokens * n_q_heads * head_dim must be below 2^31",
           HW_ERR_INVALID_ARG;
  if (g->max_splits < 0 || g->max_splits > 65535) return m = "max_splits out of range", HW_ERR_INVALID_ARG;
  // The caller's bytes are read as an integer: loading a value outside the enum's range
  // through the enum type would itself be undefined behaviour.
  int32_t dtype_raw;
  static_assert(sizeof(g->kv_dtype) == sizeof(dtype_raw), "hw_dtype is stored as a 32-bit int");
  std::memcpy(&dtype_raw, &g->kv_dtype, sizeof dtype_raw);
  if (dtype_raw != HW_BF16 && dtype_raw != HW_F32) return m = "unknown kv_dtype", HW_ERR_INVALID_ARG;
  if (!(g->rope_theta > 1.0) || !std::isfinite(g->rope_theta)) return m = "rope_theta must be > 1", HW_ERR_INVALID_ARG;
  if (!(g->softmax_scale >= 0.0f) || !std::isfinite(g->softmax_scale))
    return m = "softmax_scale must be finite and >= 0", HW_ERR_INVALID_ARG;
  if (!g->k_pool || !g->v_pool) return m = "k_pool and v_pool must be set", HW_ERR_INVALID_ARG;
  if (((uintptr_t)g->k_pool | (uintptr_t)g->v_pool) % kAlign) return m = "pools must be 256-byte aligned", HW_ERR_INVALID_ARG;
  const double elems = (double)g->n_layers * g->n_pages * g->n_kv_heads * g->page_size * g->head_dim;
  if (elems > 9.0e18 / 4) return m = "pool too large", HW_ERR_INVALID_ARG;
  return HW_OK;
}

size_t kv_elem_bytes(const hw_ctx *c) { return c->cfg.kv_dtype == HW_BF16 ? 2 : 4; }

size_t layer_elems(const hw_ctx *c) {
  const hw_config &g = c->cfg;
  return (size_t)g.n_pages * g.n_kv_heads * g.page_size * g.head_dim;
}

// ---- append planning -------------------------------------------------------------

struct AppendPlan {
  std::vector<hw::AppendRun> runs;
  std::vector<int32_t> new_pages_per_block;  // per call entry
  int32_t total_new_pages = 0;
};

hw_status plan_append(hw_ctx *c, int32_t layer, int32_t n_blocks, const int32_t *ids,
                      const int32_t *n_tokens, AppendPlan &plan) {
  const hw_config &g = c->cfg;
  if (layer < 0 || layer >= g.n_layers) return c->fail(HW_ERR_INVALID_ARG, "layer out of range");
  if (n_blocks < 0) return c->fail(HW_ERR_INVALID_ARG, "n_blocks < 0");
  if (n_blocks > 0 && (!ids || !n_tokens)) return c->fail(HW_ERR_INVALID_ARG, "block_ids/n_tokens NULL");
  std::vector<char> seen(g.max_blocks, 0);
  for (int32_t i = 0; i < n_blocks; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= g.max_blocks) return c->fail(HW_ERR_INVALID_ARG, "block id out of range");
    if (seen[b]) return c->fail(HW_ERR_INVALID_ARG, "block id repeated in one append");
    seen[b] = 1;
    if (n_tokens[i] < 0) return c->fail(HW_ERR_INVALID_ARG, "n_tokens < 0");
    const int64_t end = (int64_t)c->blocks[b].len[layer] + n_tokens[i];
    if (end > g.max_position) return c->fail(HW_ERR_INVALID_ARG, "local position would reach max_position");
    if (end > (int64_t)g.n_pages * g.page_size) return c->fail(HW_ERR_OUT_OF_PAGES, "block longer than the pool");
  }
  plan.runs.clear();
  plan.new_pages_per_block.assign(n_blocks, 0);
  plan.total_new_pages = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const BlockState &bs = c->blocks[ids[i]];
    const int32_t new_len = bs.len[layer] + n_tokens[i];
    const int32_t need = (std::max(bs.max_len(), new_len) + g.page_size - 1) / g.page_size;
    const int32_t add = std::max<int32_t>(0, need - (int32_t)bs.pages.size());
    plan.new_pages_per_block[i] = add;
    plan.total_new_pages += add;
  }
  if ((size_t)plan.total_new_pages > c->free_stack.size())
    return c->fail(HW_ERR_OUT_OF_PAGES, "not enough free pages: need " +
                                            std::to_string(plan.total_new_pages) + ", have " +
                                            std::to_string(c->free_stack.size()));
  // Pages come off the back of the free stack in call order.
  size_t taken = 0;
  int32_t row = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const BlockState &bs = c->blocks[ids[i]];
    std::vector<int32_t> pages = bs.pages;
    for (int32_t k = 0; k < plan.new_pages_per_block[i]; ++k)
      pages.push_back(c->free_stack[c->free_stack.size() - 1 - taken++]);
    int32_t pos = bs.len[layer], left = n_tokens[i];
    while (left > 0) {
      const int32_t slot = pos % g.page_size;
      const int32_t cnt = std::min(left, g.page_size - slot);
      plan.runs.push_back(hw::AppendRun{row, pages[pos / g.page_size], slot, cnt, pos});
      row += cnt;
      pos += cnt;
      left -= cnt;
    }
  }
  return HW_OK;
}

void commit_append(hw_ctx *c, int32_t layer, int32_t n_blocks, const int32_t *ids,
                   const int32_t *n_tokens, const AppendPlan &plan) {
  for (int32_t i = 0; i < n_blocks; ++i) {
    BlockState &bs = c->blocks[ids[i]];
    for (int32_t k = 0; k < plan.new_pages_per_block[i]; ++k) {
      bs.pages.push_back(c->free_stack.back());
      c->free_stack.pop_back();
    }
    bs.len[layer] += n_tokens[i];
  }
}

// ---- view resolution ---------------------------------------------------------------

int32_t row_blocks_for(const hw_ctx *c, int32_t rows, int32_t n_new = 1) {
  const int32_t rpb = hw::rows_per_block(c->cfg.kv_dtype, n_new);
  return std::max(1, (rows + rpb - 1) / rpb);
}

// Cost of a partition: one per token group, plus alpha per block of the union it touches
// (the rotation work of entering a block: once per workgroup in the cooperative kernels).
// Cuts [0, G) into n contiguous partitions with the largest cost (nearly) minimal: bisection
// on the cost bound, greedy packing at each bound (greedy is within one group's cost of the
// optimum). Trailing partitions may be empty.
bool pack_bounds(const uint8_t *first, int32_t G, int32_t n, double alpha, double cap,
                 int32_t *out) {
  int32_t p = 0;
  out[0] = 0;
  double cost = 0.0;
  for (int32_t i = 0; i < G; ++i) {
    const bool open = i == out[p];
    const double add = 1.0 + ((open || first[i]) ? alpha : 0.0);
    if (!open && cost + add > cap) {
      if (++p >= n) return false;
      out[p] = i;
      cost = 1.0 + alpha;
    } else {
      cost += add;
    }
  }
  for (int32_t q = p + 1; q <= n; ++q) out[q] = G;
  return true;
}

void partition_bounds(const uint8_t *first, int32_t G, int32_t n, double alpha, int32_t *out) {
  if (G <= 0) {
    for (int32_t q = 0; q <= n; ++q) out[q] = 0;
    return;
  }
  if (alpha == 0.0) {
    // One unit per group: the even split (floor or ceil of G / n groups each) is optimal, and
    // unlike packing at the bound it leaves no short partitions at the end, so the bytes each
    // XCD streams come out even.
    for (int32_t q = 0; q <= n; ++q) out[q] = (int32_t)((int64_t)G * q / n);
    return;
  }
  int64_t starts = 0;
  for (int32_t i = 0; i < G; ++i) starts += (first[i] || i == 0) ? 1 : 0;
  double lo = std::max(1.0 + alpha, ((double)G + alpha * (double)starts) / (double)n);
  double hi = lo + 2.0 * (1.0 + alpha);
  while (!pack_bounds(first, G, n, alpha, hi, out)) hi *= 2.0;
  for (int it = 0; it < 40 && hi - lo > 1e-6; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (pack_bounds(first, G, n, alpha, mid, out)) hi = mid;
    else lo = mid;
  }
  pack_bounds(first, G, n, alpha, hi, out);
}

// Weight of a block entry in group units, by kernel shape. Cooperative kernels (33..64 bf16
// rows) rotate every block of a partition before streaming it, and under a fused step plan
// the waves whose groups take the step's tokens also write them first. Measured on MI355X
// (w8_32k, 8 growing blocks): weights 2, 3, 4, 6, 8 give 0.345, 0.340, 0.331, 0.332 and
// 0.338 ms per fused step (0.364 and 0.353 ms for 2 and 4 with the append as its own launch).
#ifndef HW_SPLIT_ALPHA_COOP
#define HW_SPLIT_ALPHA_COOP 4.0
#endif
#ifndef HW_SPLIT_ALPHA_8W
#define HW_SPLIT_ALPHA_8W 0.0
#endif
double split_alpha(const hw_ctx *c, int32_t rows, int32_t n_new = 1) {
  const int32_t rpb = hw::rows_per_block(c->cfg.kv_dtype, n_new);
  const int32_t first = std::min(rows, rpb);
  return (c->cfg.kv_dtype == HW_BF16 && first > 32) ? HW_SPLIT_ALPHA_COOP : HW_SPLIT_ALPHA_8W;
}

int32_t auto_splits(const hw_ctx *c, int32_t n_groups, int32_t rows, int32_t n_new = 1) {
  const int32_t row_blocks = row_blocks_for(c, rows, n_new);
  const int32_t per_head = c->cfg.n_kv_heads * std::max(1, row_blocks);
  // Workgroups for about three quarters of the CUs: measured on MI355X, this still keeps
  // HBM saturated while each wave takes more groups (fixed per-wave costs amortised, less
  // tail) and fewer partials reach the merge; 24 partitions for 8 KV heads beat 32 by 2-4%.
  // Several query tokens per worker do more work per byte; filling every CU pays there:
  // w4_16k with 4 tokens runs 11% faster with 10 partitions (240 workgroups) than with 8,
  // w8_32k 19% faster with 4 (256) than with 3; one more partition each spills past one
  // workgroup per CU and is slower. The cooperative (4-wave) kernels also fill every CU:
  // w8_32k's fused step takes 0.3295 ms with 32 partitions, 0.3312 with 24, 0.3338 with 28.
  const int32_t waves = hw::decode_waves(c->cfg.kv_dtype, rows, n_new);
  const bool coop = waves == 4;
  const int32_t target = (n_new > 1 || coop) ? c->num_cus : 3 * c->num_cus / 4;
  int32_t s = std::max(1, target / per_head);
  // At least 4 groups a partition.
  s = std::min(s, std::max(1, n_groups / 4));
  // Small caches (one token per worker, 8-wave kernels): when a head's groups fit one group
  // per wave in fewer workgroups than that, the fewest such workgroups. Every wave then makes
  // one round trip, and fewer workgroups start and write partials. Measured on MI355X, w2_4k
  // (142 groups a head, replayed steps): 18 partitions (at most 8 groups each) 0.3178 ms per
  // step, 17 (some waves take two groups) 0.339, 19: 0.3197, 20: 0.3196, 24: 0.3253.
  if (!coop && n_new == 1) s = std::min(s, std::max(1, (n_groups + waves - 1) / waves));
  // A head of at most 16 groups is two groups for each wave of one workgroup: one partition
  // writes the output directly, with no merge launch (tiny_fp32: 9.3 us a step, 9.8 with two).
  if (n_groups <= 16) s = 1;
  return std::max(1, std::min(s, c->cfg.max_splits));
}

int32_t choose_splits(const hw_ctx *c, int32_t n_groups, int32_t rows, int32_t n_new = 1) {
  return c->split_override > 0 ? std::min(c->split_override, c->cfg.max_splits)
                               : auto_splits(c, n_groups, rows, n_new);
}

// Signature of everything a resolution depends on; equal signatures => equal tables.
std::vector<int64_t> signature(const hw_ctx *c, int32_t layer) {
  std::vector<int64_t> s;
  s.push_back((int64_t)c->views.version);
  s.push_back((int64_t)c->page_generation);
  for (const auto &v : c->views.blocks)
    for (int32_t b : v) {
      s.push_back(c->blocks[b].len[layer]);
      s.push_back((int64_t)c->blocks[b].pages.size());
    }
  return s;
}

hw_status resolve(hw_ctx *c, int32_t layer, Resolution &r) {
  const hw_config &g = c->cfg;
  const Views &v = c->views;
  if (!v.set) return c->fail(HW_ERR_STALE_VIEW, "no views set");
  const int32_t n = v.n_workers;
  r = Resolution();
  r.n_workers = n;
  std::vector<int32_t> seg_of(g.max_blocks, -1);
  std::vector<std::vector<int64_t>> offs(n);
  std::vector<int64_t> qpos(n);
  for (int32_t w = 0; w < n; ++w) {
    const auto &vb = v.blocks[w];
    auto &o = offs[w];
    if (v.has_offsets) {
      o = v.offsets[w];
    } else {
      int64_t acc = 0;
      for (int32_t b : vb) {
        o.push_back(acc);
        acc += c->blocks[b].len[layer];
      }
    }
    if (v.has_qpos) {
      qpos[w] = v.q_pos[w];
    } else {
      qpos[w] = vb.empty() ? -1 : o.back() + c->blocks[vb.back()].len[layer] - 1;
    }
    // overlaps and causality, over the blocks that hold tokens in this layer
    std::vector<std::pair<int64_t, int64_t>> spans;
    for (size_t i = 0; i < vb.size(); ++i) {
      const int64_t len = c->blocks[vb[i]].len[layer];
      if (len == 0) continue;
      spans.emplace_back(o[i], o[i] + len);
      if (o[i] + len - 1 > qpos[w])
        return c->fail(HW_ERR_STALE_VIEW, "worker " + std::to_string(w) + ": block " +
                                              std::to_string(vb[i]) + " has a key after q_pos");
      if (qpos[w] - o[i] >= g.max_position)
        return c->fail(HW_ERR_STALE_VIEW, "worker " + std::to_string(w) +
                                              ": query offset reaches max_position");
    }
    if (!spans.empty()) r.min_qpos = std::min(r.min_qpos, qpos[w]);
    std::sort(spans.begin(), spans.end());
    for (size_t i = 1; i < spans.size(); ++i)
      if (spans[i].first < spans[i - 1].second)
        return c->fail(HW_ERR_STALE_VIEW, "worker " + std::to_string(w) + ": overlapping blocks");
    for (int32_t b : vb)
      if (c->blocks[b].len[layer] > 0 && seg_of[b] < 0) {
        seg_of[b] = (int32_t)r.seg_blocks.size();
        r.seg_blocks.push_back(b);
      }
  }
  const int32_t n_seg = (int32_t)r.seg_blocks.size();
  r.delta.assign((size_t)n_seg * n, -1);
  for (int32_t w = 0; w < n; ++w) {
    const auto &vb = v.blocks[w];
    for (size_t i = 0; i < vb.size(); ++i) {
      const int32_t s = seg_of[vb[i]];
      if (s >= 0) r.delta[(size_t)s * n + w] = (int32_t)(qpos[w] - offs[w][i]);
    }
  }
  for (int32_t s = 0; s < n_seg; ++s) {
    const BlockState &bs = c->blocks[r.seg_blocks[s]];
    const int32_t len = bs.len[layer];
    for (int32_t t = 0; t < len; t += hw::kTokGroup) {
      r.g_page.push_back(bs.pages[t / g.page_size]);
      r.g_gip.push_back((t % g.page_size) / hw::kTokGroup);
      r.g_seg.push_back(s);
      r.g_valid.push_back(std::min(hw::kTokGroup, len - t));
      r.g_start.push_back(t);
    }
  }
  return HW_OK;
}

// ---- device helpers ----------------------------------------------------------------

hw_status hip_fail(hw_ctx *c, hipError_t e, const char *what) {
  return c->fail(HW_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hw_status ensure_staging(hw_ctx *c) {
  if (c->staging) return HW_OK;
  hipError_t e = hipHostMalloc((void **)&c->staging, c->tables_bytes * kStagingSlots, hipHostMallocDefault);
  if (e != hipSuccess) {
    c->staging = nullptr;
    return hip_fail(c, e, "hipHostMalloc(staging)");
  }
  for (int i = 0; i < kStagingSlots; ++i) {
    e = hipEventCreateWithFlags(&c->events[i], hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventCreate");
  }
  return HW_OK;
}

// Per-device addresses of the static scratch (hw_kernels.hip), resolved with the device
// current, once per device and process.
std::mutex g_scratch_mu;
void *g_scratch[256] = {};

hw_status scratch_for_current_device(hw_ctx *c, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(c, e, "hipGetDevice");
  if (dev < 0 || dev >= 256) return c->fail(HW_ERR_INVALID_ARG, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hw::scratch_address(&p);
    if (e != hipSuccess || !p) return hip_fail(c, e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HW_OK;
}

hw_status post_launch(hw_ctx *c, hipError_t e, const char *what, hipStream_t s) {
  if (e != hipSuccess) return hip_fail(c, e, what);
  if (c->debug_sync) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(c, e, what);
  }
  return HW_OK;
}

}  // namespace

// =====================================================================================
// C ABI
// =====================================================================================

extern "C" {

hw_status hw_create(const hw_config *cfg, hw_ctx **out) {
  if (!out) {
    g_create_error = "out is NULL";
    return HW_ERR_INVALID_ARG;
  }
  *out = nullptr;
  std::string m;
  hw_status st = check_config(cfg, m);
  if (st != HW_OK) {
    g_create_error = m;
    return st;
  }
  hw_ctx *c = new (std::nothrow) hw_ctx();
  if (!c) {
    g_create_error = "out of host memory";
    return HW_ERR_INVALID_ARG;
  }
  c->cfg = *cfg;
  if (c->cfg.max_splits == 0) c->cfg.max_splits = 256;
  if (c->cfg.max_query_tokens == 0) c->cfg.max_query_tokens = 1;
  if (c->cfg.softmax_scale == 0.0f) c->cfg.softmax_scale = (float)(1.0 / std::sqrt((double)cfg->head_dim));
  c->blocks.resize(cfg->max_blocks);
  for (auto &b : c->blocks) b.len.assign(cfg->n_layers, 0);
  std::vector<int32_t> order(cfg->n_pages);
  for (int32_t i = 0; i < cfg->n_pages; ++i) order[i] = i;
  if (cfg->page_seed != 0) {
    uint64_t state = cfg->page_seed;
    for (int32_t i = cfg->n_pages - 1; i >= 1; --i) {
      const int32_t j = (int32_t)(splitmix64_next(state) % (uint64_t)(i + 1));
      std::swap(order[i], order[j]);
    }
  }
  c->free_stack.assign(order.rbegin(), order.rend());
  const char *dbg = std::getenv("HW_DEBUG_SYNC");
  c->debug_sync = dbg && dbg[0] == '1';
  layout_workspace(c);
  *out = c;
  return HW_OK;
}

hw_status hw_destroy(hw_ctx *ctx) {
  if (!ctx) return HW_OK;
  for (hipEvent_t e : ctx->prof_events) (void)hipEventDestroy(e);
  for (int i = 0; i < kStagingSlots; ++i)
    if (ctx->events[i]) (void)hipEventDestroy(ctx->events[i]);
  if (ctx->staging) (void)hipHostFree(ctx->staging);
  delete ctx;
  return HW_OK;
}

const char *hw_last_error(const hw_ctx *ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

size_t hw_workspace_bytes(const hw_ctx *ctx) { return ctx ? ctx->total_bytes : 0; }

hw_status hw_set_workspace(hw_ctx *ctx, void *dev, size_t bytes) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is active: its blocks grow with hw_append_step; end it with hw_plan_end first");
  if (!dev) return ctx->fail(HW_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)dev % kAlign) return ctx->fail(HW_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < ctx->total_bytes)
    return ctx->fail(HW_ERR_WORKSPACE, "workspace too small: need " + std::to_string(ctx->total_bytes));
  const hw_config &g = ctx->cfg;
  // cos/sin of p * theta^(-2j/d), p < max_position: fp64 libm, rounded once to fp32.
  const int half = g.head_dim / 2;
  std::vector<double> inv(half);
  for (int j = 0; j < half; ++j) inv[j] = std::pow(g.rope_theta, -(2.0 * j) / (double)g.head_dim);
  std::vector<float> table((size_t)g.max_position * half * 2);
  const unsigned nthreads = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < nthreads; ++t)
    pool.emplace_back([&, t]() {
      for (int64_t p = t; p < g.max_position; p += nthreads)
        for (int j = 0; j < half; ++j) {
          const double a = (double)p * inv[j];
          table[((size_t)p * half + j) * 2] = (float)std::cos(a);
          table[((size_t)p * half + j) * 2 + 1] = (float)std::sin(a);
        }
    });
  for (auto &th : pool) th.join();
  hipError_t e = hipMemcpy((char *)dev + ctx->off_trig, table.data(), table.size() * sizeof(float),
                           hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(rope table)");
  // Query rotations: theta_j / (2 pi) in fp64, the rotation in turns per position.
  std::vector<double> turns(half);
  for (int j = 0; j < half; ++j) turns[j] = inv[j] / (2.0 * 3.14159265358979323846);
  e = hipMemcpy((char *)dev + ctx->off_freq, turns.data(), turns.size() * sizeof(double),
                hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(turn frequencies)");
  int dev_id = 0;
  if (hipGetDevice(&dev_id) == hipSuccess) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id) == hipSuccess && cus > 0)
      ctx->num_cus = cus;
  }
  // The pinned staging ring of the table uploads is allocated here, at set-up, so that no
  // append or decode allocates.
  hw_status sst = ensure_staging(ctx);
  if (sst != HW_OK) return sst;
  // The static scratch's address on this device, resolved once per device.
  sst = scratch_for_current_device(ctx, &ctx->scratch);
  if (sst != HW_OK) return sst;
  ctx->ws = dev;
  ctx->ws_bytes = bytes;
  ctx->uploaded_valid = false;
  return HW_OK;
}

hw_status hw_append_kv(hw_ctx *ctx, int32_t layer, int32_t n_blocks, const int32_t *block_ids,
                       const int32_t *n_tokens, const void *k, const void *v, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (!ctx->ws) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is active: its blocks grow with hw_append_step; end it with hw_plan_end first");
  AppendPlan plan;
  hw_status st = plan_append(ctx, layer, n_blocks, block_ids, n_tokens, plan);
  if (st != HW_OK) return st;
  if (plan.runs.empty()) return HW_OK;
  if (!k || !v) return ctx->fail(HW_ERR_INVALID_ARG, "k/v NULL");
  // Save what commit changes so a failed launch can be rolled back.
  const std::vector<int32_t> saved_free = ctx->free_stack;
  std::vector<BlockState> saved;
  for (int32_t i = 0; i < n_blocks; ++i) saved.push_back(ctx->blocks[block_ids[i]]);
  commit_append(ctx, layer, n_blocks, block_ids, n_tokens, plan);

  const hw_config &g = ctx->cfg;
  const size_t eb = kv_elem_bytes(ctx);
  hw::AppendArgs a{};
  a.k_layer = (char *)g.k_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.v_layer = (char *)g.v_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.k_src = k;
  a.v_src = v;
  a.trig = reinterpret_cast<const float2 *>((char *)ctx->ws + ctx->off_trig);
  a.n_kv_heads = g.n_kv_heads;
  a.page_groups = g.page_size / hw::kTokGroup;
  hipStream_t s = (hipStream_t)stream;
  for (size_t r0 = 0; r0 < plan.runs.size(); r0 += hw::kMaxRunsPerLaunch) {
    const size_t n = std::min(plan.runs.size() - r0, (size_t)hw::kMaxRunsPerLaunch);
    a.n_runs = (int32_t)n;
    std::memcpy(a.runs, plan.runs.data() + r0, n * sizeof(hw::AppendRun));
    hw_status ls = post_launch(ctx, hw::launch_append(g.kv_dtype, g.head_dim, a, s), "rope_append", s);
    if (ls != HW_OK) {
      ctx->free_stack = saved_free;
      for (int32_t i = 0; i < n_blocks; ++i) ctx->blocks[block_ids[i]] = saved[i];
      return ls;
    }
  }
  return HW_OK;
}

hw_status hw_set_views(hw_ctx *ctx, int32_t n_workers, const int32_t *view_len,
                       const int32_t *view_blocks, const int64_t *view_offsets,
                       const int64_t *q_pos) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is active: its blocks grow with hw_append_step; end it with hw_plan_end first");
  const hw_config &g = ctx->cfg;
  if (n_workers <= 0 || n_workers > g.max_workers)
    return ctx->fail(HW_ERR_INVALID_ARG, "n_workers must be in [1, max_workers]");
  if (!view_len) return ctx->fail(HW_ERR_INVALID_ARG, "view_len NULL");
  int64_t total = 0;
  for (int32_t w = 0; w < n_workers; ++w) {
    if (view_len[w] < 0 || view_len[w] > g.max_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "view_len out of range");
    total += view_len[w];
  }
  if (total > 0 && !view_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "view_blocks NULL");
  Views nv;
  nv.set = true;
  nv.n_workers = n_workers;
  nv.has_offsets = view_offsets != nullptr;
  nv.has_qpos = q_pos != nullptr;
  std::vector<char> seen(g.max_blocks, 0);
  int64_t k = 0;
  for (int32_t w = 0; w < n_workers; ++w) {
    std::vector<int32_t> vb(view_blocks + k, view_blocks + k + view_len[w]);
    std::vector<int64_t> vo;
    if (view_offsets) vo.assign(view_offsets + k, view_offsets + k + view_len[w]);
    k += view_len[w];
    for (int32_t b : vb)
      if (b < 0 || b >= g.max_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "view block id out of range");
    for (int32_t b : vb) {
      if (seen[b]) {
        for (int32_t x : vb) seen[x] = 0;
        return ctx->fail(HW_ERR_INVALID_ARG, "block repeated in a view");
      }
      seen[b] = 1;
    }
    for (int32_t b : vb) seen[b] = 0;
    for (int64_t o : vo)
      if (o < 0 || o >= (int64_t)1 << 40) return ctx->fail(HW_ERR_INVALID_ARG, "view offset out of range");
    if (q_pos && (q_pos[w] < -1 || q_pos[w] >= (int64_t)1 << 40))
      return ctx->fail(HW_ERR_INVALID_ARG, "q_pos out of range");
    nv.blocks.push_back(std::move(vb));
    nv.offsets.push_back(std::move(vo));
    if (q_pos) nv.q_pos.push_back(q_pos[w]);
  }
  nv.version = ctx->views.version + 1;
  ctx->views = std::move(nv);
  return HW_OK;
}

}  // extern "C"

namespace {

// Where a decode's tables are, and how its groups are split.
struct DecodeTables {
  const int2 *groups = nullptr;
  const int32_t *delta = nullptr;
  int32_t n_groups = 0, stride = 2, splits = 1;
  const int32_t *bounds = nullptr;      // splits + 1 cuts, or null: uniform cuts
  const int32_t *plan_step = nullptr;   // step plans: the layer's counter of planned appends
  int32_t plan_pending = 0, plan_n_steps = 0;
  int32_t *advance = nullptr;           // counter to advance once the decode has read it
  // hw_decode_step: the step's new keys and values, appended by the decode itself
  const void *fuse_k = nullptr, *fuse_v = nullptr;
  const int32_t *fuse_blocks = nullptr;
  int32_t *fuse_overflow = nullptr;
  int32_t fuse_n_blocks = 0;
  int32_t fuse_gmin = 0, fuse_gmax = -1;
};

// Split partials of a decode: the workspace's, or a caller-provided buffer of the same shape.
struct Partials {
  float *o = nullptr;
  float *lse = nullptr;
};

Partials workspace_partials(hw_ctx *ctx) {
  if (!ctx->ws) return Partials{};   // decode_impl rejects the call
  return Partials{reinterpret_cast<float *>((char *)ctx->ws + ctx->off_part_o),
                  reinterpret_cast<float *>((char *)ctx->ws + ctx->off_part_lse)};
}

// Enqueue the decode kernel of one layer and, with several partitions, the merge.
hw_status launch_decode_merge(hw_ctx *ctx, int32_t layer, int32_t n_new, const float *q,
                              float *out, float *lse, hipStream_t s, const DecodeTables &t,
                              Partials part) {
  const hw_config &g = ctx->cfg;
  const int32_t n = ctx->views.n_workers;
  const int32_t group = g.n_q_heads / g.n_kv_heads;
  const int32_t rows = rows_total(ctx, n, n_new);
  const size_t eb = kv_elem_bytes(ctx);
  hw::DecodeArgs a{};
  a.k_layer = (char *)g.k_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.v_layer = (char *)g.v_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.groups = t.groups;
  a.delta = t.delta;
  a.turn_freq = reinterpret_cast<const double *>((char *)ctx->ws + ctx->off_freq);
  a.part_o = part.o;
  a.part_lse = part.lse;
  a.n_groups = t.n_groups;
  a.n_workers = n;
  a.n_q_heads = g.n_q_heads;
  a.n_kv_heads = g.n_kv_heads;
  a.group = group;
  a.rows = rows;
  a.n_splits = t.splits;
  a.page_groups = g.page_size / hw::kTokGroup;
  a.rows_per_block = hw::rows_per_block(g.kv_dtype, n_new);
  a.inv_group = 1.0f / (float)group;
  a.inv_rpw = 1.0f / (float)(n_new * group);
  a.n_new = n_new;
  a.q_scale = (float)((double)g.softmax_scale * 1.4426950408889634);
  a.desc_stride = t.stride;
  a.plan_step = t.plan_step;
  a.plan_pending = t.plan_pending;
  a.plan_n_steps = t.plan_n_steps;
  a.fuse_k = t.fuse_k;
  a.fuse_v = t.fuse_v;
  a.fuse_trig = reinterpret_cast<const float2 *>((char *)ctx->ws + ctx->off_trig);
  a.fuse_blocks = t.fuse_blocks;
  a.fuse_overflow = t.fuse_overflow;
  a.fuse_n_blocks = t.fuse_n_blocks;
  a.fuse_gmin = t.fuse_gmin;
  a.fuse_gmax = t.fuse_gmax;
  if (t.bounds) std::copy(t.bounds, t.bounds + t.splits + 1, a.split_begin);
  const int32_t row_blocks = row_blocks_for(ctx, rows, n_new);
  const bool prof = ctx->prof_count < ctx->prof_capacity;
  hipEvent_t *ev = prof ? &ctx->prof_events[2 * (size_t)ctx->prof_count] : nullptr;
  hw_status st = post_launch(ctx,
                             hw::launch_decode(g.kv_dtype, g.head_dim, a, row_blocks, s,
                                               prof ? ev[0] : nullptr, prof ? ev[1] : nullptr),
                             "concurrent_decode", s);
  if (st != HW_OK) return st;
  if (prof) ctx->prof_count++;
  if (t.splits > 1) {
    hw::MergeArgs m{};
    m.part_o = part.o;
    m.part_lse = part.lse;
    m.out = out;
    m.lse = lse;
    m.n_workers = n * n_new;   // query tokens, each merged on its own
    m.n_q_heads = g.n_q_heads;
    m.n_kv_heads = g.n_kv_heads;
    m.group = group;
    m.rows = rows;
    m.n_splits = t.splits;
    m.advance = t.advance;
    m.advance_cap = t.plan_n_steps;
    st = post_launch(ctx, hw::launch_merge(g.head_dim, m, s), "lse_merge", s);
    if (st != HW_OK) return st;
  } else if (t.advance) {
    st = post_launch(ctx, hw::launch_advance(t.advance, t.plan_n_steps, s), "advance", s);
    if (st != HW_OK) return st;
  }
  return HW_OK;
}

// A decode under the active step plan: its tables were uploaded by hw_plan_steps. With fuse_k
// set (hw_decode_step) the decode also performs the layer's planned append of the step.
hw_status decode_planned(hw_ctx *ctx, int32_t layer, int32_t n_new, const float *q, float *out,
                         float *lse, hipStream_t s, Partials part, const void *fuse_k = nullptr,
                         const void *fuse_v = nullptr) {
  const Plan &p = ctx->plan;
  if (n_new != 1)
    return ctx->fail(HW_ERR_INVALID_ARG, "several query tokens per worker are not supported under a step plan");
  char *base = (char *)ctx->ws + ctx->off_plan;
  DecodeTables t;
  t.groups = reinterpret_cast<const int2 *>(base + ctx->plan_groups);
  t.delta = reinterpret_cast<const int32_t *>(base + ctx->plan_delta);
  t.n_groups = p.n_groups;
  t.stride = 4;
  t.splits = p.splits;
  t.bounds = p.splits <= hw::kMaxBoundSplits ? p.bounds.data() : nullptr;
  int32_t *counter = reinterpret_cast<int32_t *>(base + ctx->plan_cnt) + layer;
  t.plan_step = counter;
  t.plan_n_steps = p.n_steps;
  t.plan_pending = p.pending[layer];
  t.advance = p.pending[layer] ? counter : nullptr;
  if (fuse_k) {   // the step's append is this decode's: it sees one more step, then counts it
    t.plan_pending = 1;
    t.advance = counter;
    t.fuse_k = fuse_k;
    t.fuse_v = fuse_v;
    t.fuse_blocks = reinterpret_cast<const int32_t *>(base + ctx->plan_fuse);
    t.fuse_overflow = reinterpret_cast<int32_t *>(base + ctx->plan_cnt) + ctx->cfg.n_layers;
    t.fuse_n_blocks = (int32_t)p.blocks.size();
    t.fuse_gmin = p.fuse_gmin;
    t.fuse_gmax = p.fuse_gmax;
  }
  hw_status st = launch_decode_merge(ctx, layer, n_new, q, out, lse, s, t, part);
  if (st == HW_OK) ctx->plan.pending[layer] = 0;
  return st;
}

// One decode of n_new query tokens per worker (n_new = 1: the one-token step), with its split
// partials in `part`.
hw_status decode_impl(hw_ctx *ctx, int32_t layer, int32_t n_new, const float *q, float *out,
                      float *lse, hipStream_t s, Partials part) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  if (layer < 0 || layer >= g.n_layers) return ctx->fail(HW_ERR_INVALID_ARG, "layer out of range");
  if (n_new < 1 || n_new > g.max_query_tokens)
    return ctx->fail(HW_ERR_INVALID_ARG, "n_new must be in [1, max_query_tokens]");
  if (!q || !out) return ctx->fail(HW_ERR_INVALID_ARG, "q/out NULL");
  if (!ctx->ws) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
  if (!ctx->views.set) return ctx->fail(HW_ERR_STALE_VIEW, "no views set");
  const int32_t n = ctx->views.n_workers;
  char *tables = (char *)ctx->ws + ctx->off_tables;
  const int32_t rows = rows_total(ctx, n, n_new);
  // Group descriptors: wide ones (each group's offsets beside it) for the 8-wave kernels
  // when every worker fits and each worker has one token; with several tokens, the group's
  // first local position beside {x, y} for the causal mask; else {x, y} alone. The
  // cooperative kernels read the offset table per phase.
  const bool wide = n_new == 1 && n <= hw::kWideWorkers &&
                    hw::decode_waves(g.kv_dtype, rows) == 8 && rows <= hw::rows_per_block(g.kv_dtype);
  const int32_t stride = wide ? hw::kWideStride : (n_new > 1 ? 4 : 2);

  if (ctx->plan.active) return decode_planned(ctx, layer, n_new, q, out, lse, s, part);
  std::vector<int64_t> sig = signature(ctx, layer);
  if (!ctx->uploaded_valid || sig != ctx->uploaded_sig || ctx->up_stride != stride) {
    Resolution r;
    hw_status st = resolve(ctx, layer, r);
    if (st != HW_OK) return st;
    // Every check that can fail comes before the upload is staged or enqueued.
    if (r.min_qpos < (int64_t)n_new - 1)
      return ctx->fail(HW_ERR_STALE_VIEW, "a worker's first query token would sit below position 0");
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t ce = hipStreamIsCapturing(s, &cap);
    if (ce != hipSuccess) return hip_fail(ctx, ce, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
      return ctx->fail(HW_ERR_INVALID_ARG,
                       "the views' device tables need an upload (views or lengths changed), which "
                       "cannot be captured: decode once with these views and lengths before the "
                       "capture, or capture steps under a step plan (hw_plan_steps)");
    if (!ctx->staging) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
    const int32_t n_seg = (int32_t)r.seg_blocks.size();
    const int32_t n_groups = (int32_t)r.g_page.size();
    const size_t delta_bytes = align_up((size_t)n_seg * n * sizeof(int32_t));
    const size_t bytes = delta_bytes + (size_t)n_groups * stride * sizeof(int32_t);
    const int slot = ctx->next_slot;
    ctx->next_slot = (ctx->next_slot + 1) % kStagingSlots;
    if (ctx->event_live[slot]) {
      hipError_t e = hipEventSynchronize(ctx->events[slot]);
      if (e != hipSuccess) return hip_fail(ctx, e, "hipEventSynchronize(staging)");
    }
    char *stg = ctx->staging + (size_t)slot * ctx->tables_bytes;
    if (n_seg) std::memcpy(stg, r.delta.data(), (size_t)n_seg * n * sizeof(int32_t));
    int32_t *gd = reinterpret_cast<int32_t *>(stg + delta_bytes);
    const int32_t gpp = g.page_size / hw::kTokGroup;
    ctx->up_seg_first.assign((size_t)n_groups, 0);
    for (int32_t i = 0; i < n_groups; ++i) {
      int32_t *d = gd + (size_t)stride * i;
      d[0] = r.g_page[i] * g.n_kv_heads * gpp + r.g_gip[i];
      d[1] = (r.g_seg[i] << 8) | r.g_valid[i];
      if (wide) {
        for (int32_t k = 0; k < hw::kWideWorkers; ++k)
          d[2 + k] = k < n ? r.delta[(size_t)r.g_seg[i] * n + k] : -1;
      } else if (stride == 4) {
        d[2] = r.g_start[i];
        d[3] = 0;
      }
      ctx->up_seg_first[i] = (i == 0 || r.g_seg[i] != r.g_seg[i - 1]) ? 1 : 0;
    }
    ctx->bounds_splits = -1;
    if (bytes) {
      hipError_t e = hipMemcpyAsync(tables, stg, bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync(view tables)");
      e = hipEventRecord(ctx->events[slot], s);
      if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord(staging)");
      ctx->event_live[slot] = true;
    }
    ctx->uploaded_sig = std::move(sig);
    ctx->uploaded_valid = true;
    ctx->up_n_groups = n_groups;
    ctx->up_n_seg = n_seg;
    ctx->up_n_workers = n;
    ctx->up_groups_off = delta_bytes;
    ctx->up_stride = stride;
    ctx->up_min_qpos = r.min_qpos;
  }
  // Token 0 of a worker sits n_new - 1 positions before its query position.
  if (ctx->up_min_qpos < (int64_t)n_new - 1)
    return ctx->fail(HW_ERR_STALE_VIEW, "a worker's first query token would sit below position 0");

  const int32_t n_groups = ctx->up_n_groups;
  const int32_t splits = choose_splits(ctx, n_groups, rows, n_new);
  const int32_t *bounds = nullptr;
  if (splits <= hw::kMaxBoundSplits) {
    const double alpha = split_alpha(ctx, rows, n_new);
    if (ctx->bounds_splits != splits || ctx->bounds_alpha != alpha) {
      ctx->bounds.resize((size_t)splits + 1);
      partition_bounds(ctx->up_seg_first.data(), n_groups, splits, alpha, ctx->bounds.data());
      ctx->bounds_splits = splits;
      ctx->bounds_alpha = alpha;
    }
    bounds = ctx->bounds.data();
  }
  DecodeTables t;
  t.groups = reinterpret_cast<const int2 *>(tables + ctx->up_groups_off);
  t.delta = reinterpret_cast<const int32_t *>(tables);
  t.n_groups = n_groups;
  t.stride = ctx->up_stride;
  t.splits = splits;
  t.bounds = bounds;
  return launch_decode_merge(ctx, layer, n_new, q, out, lse, s, t, part);
}

}  // namespace

extern "C" {

hw_status hw_concurrent_decode(hw_ctx *ctx, int32_t layer, const float *q, float *out, float *lse,
                               void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  return decode_impl(ctx, layer, 1, q, out, lse, (hipStream_t)stream, workspace_partials(ctx));
}

hw_status hw_concurrent_decode_noalloc(hw_ctx *ctx, int32_t layer, const float *q, float *out,
                                       float *lse, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  if (!ctx->ws || !ctx->scratch) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
  if (!ctx->views.set) return ctx->fail(HW_ERR_STALE_VIEW, "no views set");
  // The partials of the partition count this decode would use must fit the static scratch.
  const int32_t n = ctx->views.n_workers;
  const int32_t rows = rows_total(ctx, n);
  int32_t splits = ctx->plan.active ? ctx->plan.splits : 0;
  if (!splits) {
    if (ctx->uploaded_valid && ctx->uploaded_sig == signature(ctx, layer)) {
      splits = choose_splits(ctx, ctx->up_n_groups, rows);
    } else {
      Resolution r;
      hw_status st = resolve(ctx, layer, r);
      if (st != HW_OK) return st;
      splits = choose_splits(ctx, (int32_t)r.g_page.size(), rows);
    }
  }
  const size_t o_bytes = align_up((size_t)splits * g.n_kv_heads * rows * g.head_dim * sizeof(float));
  const size_t need = o_bytes + (size_t)splits * g.n_kv_heads * rows * sizeof(float);
  if (need > hw::kScratchBytes)
    return ctx->fail(HW_ERR_WORKSPACE, "split partials need " + std::to_string(need) +
                                           " bytes, more than the static scratch's " +
                                           std::to_string(hw::kScratchBytes));
  Partials part{reinterpret_cast<float *>(ctx->scratch),
                reinterpret_cast<float *>((char *)ctx->scratch + o_bytes)};
  return decode_impl(ctx, layer, 1, q, out, lse, (hipStream_t)stream, part);
}

hw_status hw_concurrent_decode_tokens(hw_ctx *ctx, int32_t layer, int32_t n_new, const float *q,
                                      float *out, float *lse, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  return decode_impl(ctx, layer, n_new, q, out, lse, (hipStream_t)stream, workspace_partials(ctx));
}

hw_status hw_debug_kernel_events(hw_ctx *ctx, int32_t capacity) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (capacity < 0) return ctx->fail(HW_ERR_INVALID_ARG, "capacity < 0");
  for (hipEvent_t e : ctx->prof_events) (void)hipEventDestroy(e);
  ctx->prof_events.clear();
  ctx->prof_capacity = ctx->prof_count = 0;
  for (int32_t i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      for (hipEvent_t x : ctx->prof_events) (void)hipEventDestroy(x);
      ctx->prof_events.clear();
      return hip_fail(ctx, err, "hipEventCreate(profile)");
    }
    ctx->prof_events.push_back(e);
  }
  ctx->prof_capacity = capacity;
  return HW_OK;
}

hw_status hw_debug_kernel_elapsed(hw_ctx *ctx, float *decode_ms, int32_t cap, int32_t *n) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (n) *n = ctx->prof_count;
  for (int32_t i = 0; i < ctx->prof_count && i < cap; ++i) {
    hipEvent_t *ev = &ctx->prof_events[2 * (size_t)i];
    hipError_t e = hipEventSynchronize(ev[1]);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipEventSynchronize(profile)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipEventElapsedTime(profile)");
    if (decode_ms) decode_ms[i] = ms;
  }
  ctx->prof_count = 0;
  return HW_OK;
}

hw_status hw_debug_stream_read(const void *src, size_t bytes, float *sink, int32_t n_blocks,
                               void *stream, float *elapsed_ms) {
  if (!src || !sink || bytes == 0 || bytes % 16 || (uintptr_t)src % 16 || n_blocks < 1 ||
      n_blocks > 65535) {
    g_create_error = "hw_debug_stream_read: bad pointer, alignment, size or n_blocks";
    return HW_ERR_INVALID_ARG;
  }
  hipEvent_t ev[2] = {nullptr, nullptr};
  auto fail = [&](hipError_t e, const char *what) {
    g_create_error = std::string("hw_debug_stream_read: ") + what + ": " + hipGetErrorString(e);
    for (hipEvent_t x : ev)
      if (x) (void)hipEventDestroy(x);
    return HW_ERR_HIP;
  };
  hipError_t e;
  if (elapsed_ms)
    for (hipEvent_t &x : ev)
      if ((e = hipEventCreate(&x)) != hipSuccess) return fail(e, "hipEventCreate");
  e = hw::launch_stream_read(src, bytes, sink, n_blocks, (hipStream_t)stream, ev[0], ev[1]);
  if (e != hipSuccess) return fail(e, "launch");
  if (elapsed_ms) {
    if ((e = hipEventSynchronize(ev[1])) != hipSuccess) return fail(e, "hipEventSynchronize");
    if ((e = hipEventElapsedTime(elapsed_ms, ev[0], ev[1])) != hipSuccess) return fail(e, "hipEventElapsedTime");
    for (hipEvent_t x : ev) (void)hipEventDestroy(x);
  }
  return HW_OK;
}

hw_status hw_plan_steps(hw_ctx *ctx, int32_t n_steps, int32_t n_blocks, const int32_t *block_ids,
                        const int32_t *tokens_per_step, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is already active");
  if (g.kv_dtype != HW_BF16) return ctx->fail(HW_ERR_INVALID_ARG, "step plans need bf16 pools");
  if (!ctx->views.set) return ctx->fail(HW_ERR_STALE_VIEW, "no views set");
  const Views &v = ctx->views;
  if (v.has_offsets || v.has_qpos)
    return ctx->fail(HW_ERR_INVALID_ARG, "step plans need default offsets and query positions");
  if (n_steps < 1) return ctx->fail(HW_ERR_INVALID_ARG, "n_steps must be >= 1");
  if (n_blocks < 0 || n_blocks > g.max_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "n_blocks out of range");
  if (n_blocks > 0 && (!block_ids || !tokens_per_step))
    return ctx->fail(HW_ERR_INVALID_ARG, "block_ids/tokens_per_step NULL");
  std::vector<int64_t> grow(g.max_blocks, 0);
  std::vector<char> planned(g.max_blocks, 0);
  int64_t rows = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const int32_t b = block_ids[i];
    if (b < 0 || b >= g.max_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "block id out of range");
    if (planned[b]) return ctx->fail(HW_ERR_INVALID_ARG, "block id repeated in a plan");
    if (tokens_per_step[i] < 0) return ctx->fail(HW_ERR_INVALID_ARG, "tokens_per_step < 0");
    planned[b] = 1;
    grow[b] = (int64_t)n_steps * tokens_per_step[i];
    rows += tokens_per_step[i];
  }
  if (rows > hw::kMaxPlanRows)
    return ctx->fail(HW_ERR_INVALID_ARG, "a planned step takes at most " + std::to_string(hw::kMaxPlanRows) +
                                             " tokens over all blocks");
  if (n_blocks > hw::kMaxPlanBlocks)
    return ctx->fail(HW_ERR_INVALID_ARG, "a plan takes at most " + std::to_string(hw::kMaxPlanBlocks) + " blocks");
  // Every block of the views and of the plan must have the same length in every layer: one
  // set of tables serves all layers, each at its own count of planned appends.
  auto equal_layers = [&](int32_t b) {
    const auto &len = ctx->blocks[b].len;
    return std::all_of(len.begin(), len.end(), [&](int32_t x) { return x == len[0]; });
  };
  for (int32_t i = 0; i < n_blocks; ++i)
    if (!equal_layers(block_ids[i])) return ctx->fail(HW_ERR_INVALID_ARG, "a planned block's length differs between layers");
  for (const auto &vb : v.blocks)
    for (int32_t b : vb)
      if (!equal_layers(b)) return ctx->fail(HW_ERR_INVALID_ARG, "a view block's length differs between layers");
  auto len0 = [&](int32_t b) { return (int64_t)ctx->blocks[b].len[0]; };
  auto cap = [&](int32_t b) { return len0(b) + grow[b]; };
  for (int32_t i = 0; i < n_blocks; ++i)
    if (cap(block_ids[i]) > g.max_position)
      return ctx->fail(HW_ERR_INVALID_ARG, "a planned block would reach max_position");
  const int32_t n = v.n_workers;
  for (const auto &vb : v.blocks) {
    int64_t total = 0;
    for (int32_t b : vb) total += cap(b);
    if (total > g.max_position)
      return ctx->fail(HW_ERR_STALE_VIEW, "a view would reach max_position within the plan");
  }
  if (!ctx->ws) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
  // Pages for the whole window, taken now.
  std::vector<int32_t> add(n_blocks, 0);
  size_t need = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const BlockState &bs = ctx->blocks[block_ids[i]];
    const int64_t pages = (std::max<int64_t>(cap(block_ids[i]), bs.max_len()) + g.page_size - 1) / g.page_size;
    add[i] = (int32_t)std::max<int64_t>(0, pages - (int64_t)bs.pages.size());
    need += add[i];
  }
  if (need > ctx->free_stack.size())
    return ctx->fail(HW_ERR_OUT_OF_PAGES, "not enough free pages for the plan: need " +
                                              std::to_string(need) + ", have " +
                                              std::to_string(ctx->free_stack.size()));
  std::vector<std::vector<int32_t>> pages(n_blocks);
  {
    size_t taken = 0;
    for (int32_t i = 0; i < n_blocks; ++i) {
      pages[i] = ctx->blocks[block_ids[i]].pages;
      for (int32_t k = 0; k < add[i]; ++k)
        pages[i].push_back(ctx->free_stack[ctx->free_stack.size() - 1 - taken++]);
    }
  }
  auto page_list = [&](int32_t b) -> const std::vector<int32_t> & {
    for (int32_t i = 0; i < n_blocks; ++i)
      if (block_ids[i] == b) return pages[i];
    return ctx->blocks[b].pages;
  };
  // Segments: the blocks of the views that hold a token at the end of the plan, in order of
  // first appearance (worker 0's view first).
  std::vector<int32_t> seg_of(g.max_blocks, -1), seg_blocks;
  for (const auto &vb : v.blocks)
    for (int32_t b : vb)
      if (cap(b) > 0 && seg_of[b] < 0) {
        seg_of[b] = (int32_t)seg_blocks.size();
        seg_blocks.push_back(b);
      }
  const int32_t n_seg = (int32_t)seg_blocks.size();
  // Query offsets at step s: (sum of the lengths from the block to the end of the view) - 1,
  // i.e. d0 + s * rate with rate = the tokens per step of the view's blocks from there on.
  std::vector<int32_t> dtab((size_t)n_seg * n * 2);
  for (size_t i = 0; i < dtab.size(); i += 2) {
    dtab[i] = -1;
    dtab[i + 1] = 0;
  }
  for (int32_t w = 0; w < n; ++w) {
    const auto &vb = v.blocks[w];
    int64_t suffix = 0, rate = 0;
    for (size_t i = vb.size(); i-- > 0;) {
      suffix += len0(vb[i]);
      rate += grow[vb[i]] / n_steps;
      const int32_t sg = seg_of[vb[i]];
      if (sg >= 0) {
        dtab[((size_t)sg * n + w) * 2] = (int32_t)(suffix - 1);
        dtab[((size_t)sg * n + w) * 2 + 1] = (int32_t)rate;
      }
    }
  }
  // Groups at capacity: {page group of head 0, segment << 8, tokens at step 0 from the
  // group's start (clamped to 0..32 on the device), tokens per step}.
  const int32_t gpp = g.page_size / hw::kTokGroup;
  std::vector<int32_t> gtab;
  std::vector<uint8_t> seg_first;
  std::vector<int32_t> first_group(g.max_blocks, -1);   // list index of a block's group 0
  for (int32_t sg = 0; sg < n_seg; ++sg) {
    const int32_t b = seg_blocks[sg];
    const auto &pl = page_list(b);
    first_group[b] = (int32_t)(gtab.size() / 4);
    for (int64_t t = 0; t < cap(b); t += hw::kTokGroup) {
      gtab.push_back(pl[t / g.page_size] * g.n_kv_heads * gpp + (int32_t)((t % g.page_size) / hw::kTokGroup));
      gtab.push_back(sg << 8);
      gtab.push_back((int32_t)(len0(b) - t));
      gtab.push_back((int32_t)(grow[b] / n_steps));
      seg_first.push_back(t == 0 ? 1 : 0);
    }
  }
  const int32_t n_groups = (int32_t)(gtab.size() / 4);
  const int32_t rows_q = rows_total(ctx, n);
  const int32_t splits = choose_splits(ctx, n_groups, rows_q);
  std::vector<int32_t> bounds;
  if (splits <= hw::kMaxBoundSplits) {
    bounds.resize((size_t)splits + 1);
    partition_bounds(seg_first.data(), n_groups, splits, split_alpha(ctx, rows_q), bounds.data());
  }
  // The planned append's launch arguments: per block {base length, tokens per step, first
  // row, first page the window writes, where its id sits}, and the ids of the pages that
  // the window's positions [base, base + n_steps * tps) fall in.
  std::vector<hw::PlanBlock> ablk;
  std::vector<int32_t> apages;
  int32_t row0 = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const int64_t base = len0(block_ids[i]);
    const int32_t p0 = (int32_t)(base / g.page_size);
    const int32_t p1 = grow[block_ids[i]] > 0 ? (int32_t)((cap(block_ids[i]) - 1) / g.page_size) : p0 - 1;
    ablk.push_back(hw::PlanBlock{(int32_t)base, tokens_per_step[i], row0, p0, (int32_t)apages.size()});
    for (int32_t q = p0; q <= p1; ++q) apages.push_back(pages[i][q]);
    row0 += tokens_per_step[i];
  }
  if (apages.size() > (size_t)hw::kMaxPlanPages)
    return ctx->fail(HW_ERR_INVALID_ARG, "the plan's window spans more than " +
                                             std::to_string(hw::kMaxPlanPages) + " pages");
  // The fused step's table: per block {base length, tokens per step, first row, list index of
  // its group 0 (-1: in no view)}.
  std::vector<int32_t> ftab;
  bool fusable = row_blocks_for(ctx, rows_q) == 1;
  int32_t fgmin = 0, fgmax = -1;
  for (int32_t i = 0; i < n_blocks; ++i) {
    const hw::PlanBlock &pb = ablk[i];
    const int32_t g0 = first_group[block_ids[i]];
    ftab.insert(ftab.end(), {pb.base, pb.tps, pb.row0, g0});
    if (pb.tps > 0 && g0 < 0) fusable = false;
    if (pb.tps > 0 && g0 >= 0) {
      const int32_t ga = g0 + pb.base / hw::kTokGroup;
      const int32_t gz = g0 + (int32_t)(((int64_t)pb.base + (int64_t)n_steps * pb.tps - 1) / hw::kTokGroup);
      fgmin = fgmax < fgmin ? ga : std::min(fgmin, ga);
      fgmax = std::max(fgmax, gz);
    }
  }
  // One upload of the whole region, counters zeroed; the plan is set-up, not a step, so the
  // call waits for it.
  const size_t region = ctx->plan_groups + gtab.size() * sizeof(int32_t);
  std::vector<char> host(region, 0);
  if (!ftab.empty()) std::memcpy(host.data() + ctx->plan_fuse, ftab.data(), ftab.size() * 4);
  if (!dtab.empty()) std::memcpy(host.data() + ctx->plan_delta, dtab.data(), dtab.size() * 4);
  if (!gtab.empty()) std::memcpy(host.data() + ctx->plan_groups, gtab.data(), gtab.size() * 4);
  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus capst = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &capst);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamIsCapturing");
  if (capst != hipStreamCaptureStatusNone)
    return ctx->fail(HW_ERR_INVALID_ARG, "hw_plan_steps uploads tables and cannot be captured");
  e = hipMemcpyAsync((char *)ctx->ws + ctx->off_plan, host.data(), region, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "upload of the plan's tables");
  // Commit: the planned blocks own their pages for the whole window.
  for (int32_t i = 0; i < n_blocks; ++i) {
    BlockState &bs = ctx->blocks[block_ids[i]];
    for (int32_t k = 0; k < add[i]; ++k) {
      bs.pages.push_back(ctx->free_stack.back());
      ctx->free_stack.pop_back();
    }
  }
  Plan &p = ctx->plan;
  p = Plan();
  p.active = true;
  p.n_steps = n_steps;
  p.blocks.assign(block_ids, block_ids + n_blocks);
  p.tps.assign(tokens_per_step, tokens_per_step + n_blocks);
  for (int32_t i = 0; i < n_blocks; ++i) p.base.push_back((int32_t)len0(block_ids[i]));
  p.rows = (int32_t)rows;
  p.n_workers = n;
  p.n_groups = n_groups;
  p.splits = splits;
  p.bounds = std::move(bounds);
  p.append_blocks = std::move(ablk);
  p.append_pages = std::move(apages);
  p.fusable = fusable;
  p.fuse_gmin = fgmin;
  p.fuse_gmax = fgmax;
  p.pending.assign((size_t)g.n_layers, 0);
  ctx->uploaded_valid = false;
  return HW_OK;
}

hw_status hw_append_step(hw_ctx *ctx, int32_t layer, const void *k, const void *v, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  const Plan &p = ctx->plan;
  if (!p.active) return ctx->fail(HW_ERR_INVALID_ARG, "no step plan is active");
  if (layer < 0 || layer >= g.n_layers) return ctx->fail(HW_ERR_INVALID_ARG, "layer out of range");
  if (p.pending[layer])
    return ctx->fail(HW_ERR_INVALID_ARG, "this layer's planned step is appended but not decoded yet");
  if (p.rows > 0 && (!k || !v)) return ctx->fail(HW_ERR_INVALID_ARG, "k/v NULL");
  if (((uintptr_t)k | (uintptr_t)v) % 16) return ctx->fail(HW_ERR_INVALID_ARG, "k/v must be 16-byte aligned");
  char *base = (char *)ctx->ws + ctx->off_plan;
  const size_t eb = kv_elem_bytes(ctx);
  hw::PlanAppendArgs a{};
  a.k_layer = (char *)g.k_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.v_layer = (char *)g.v_pool + (size_t)layer * layer_elems(ctx) * eb;
  a.k_src = k;
  a.v_src = v;
  a.trig = reinterpret_cast<const float2 *>((char *)ctx->ws + ctx->off_trig);
  std::copy(p.append_blocks.begin(), p.append_blocks.end(), a.blocks);
  std::copy(p.append_pages.begin(), p.append_pages.end(), a.pages);
  a.step = reinterpret_cast<const int32_t *>(base + ctx->plan_cnt) + layer;
  a.overflow = reinterpret_cast<int32_t *>(base + ctx->plan_cnt) + g.n_layers;
  a.n_blocks = (int32_t)p.blocks.size();
  a.rows = p.rows;
  a.n_steps = p.n_steps;
  a.n_kv_heads = g.n_kv_heads;
  a.page_size = g.page_size;
  a.page_groups = g.page_size / hw::kTokGroup;
  hipStream_t s = (hipStream_t)stream;
  if (p.rows > 0) {   // (no planned token: nothing to write, the step still counts)
    hw_status st = post_launch(ctx, hw::launch_plan_append(g.kv_dtype, g.head_dim, a, s), "plan_append", s);
    if (st != HW_OK) return st;
  }
  ctx->plan.pending[layer] = 1;
  return HW_OK;
}

hw_status hw_decode_step(hw_ctx *ctx, int32_t layer, const void *k, const void *v, const float *q,
                         float *out, float *lse, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  const Plan &p = ctx->plan;
  if (!p.active) return ctx->fail(HW_ERR_INVALID_ARG, "no step plan is active");
  if (layer < 0 || layer >= g.n_layers) return ctx->fail(HW_ERR_INVALID_ARG, "layer out of range");
  if (p.pending[layer])
    return ctx->fail(HW_ERR_INVALID_ARG, "this layer's planned step is appended but not decoded yet");
  if (!p.fusable)
    return ctx->fail(HW_ERR_INVALID_ARG, "the plan has a growing block in no view, or more rows than one "
                                         "decode workgroup holds: use hw_append_step and hw_concurrent_decode");
  if (!k || !v) return ctx->fail(HW_ERR_INVALID_ARG, "k/v NULL");
  if (((uintptr_t)k | (uintptr_t)v) % 16) return ctx->fail(HW_ERR_INVALID_ARG, "k/v must be 16-byte aligned");
  if (!q || !out) return ctx->fail(HW_ERR_INVALID_ARG, "q/out NULL");
  if (!ctx->ws) return ctx->fail(HW_ERR_WORKSPACE, "no workspace set");
  return decode_planned(ctx, layer, 1, q, out, lse, (hipStream_t)stream, workspace_partials(ctx), k, v);
}

hw_status hw_plan_end(hw_ctx *ctx, void *stream) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  const hw_config &g = ctx->cfg;
  Plan &p = ctx->plan;
  if (!p.active) return ctx->fail(HW_ERR_INVALID_ARG, "no step plan is active");
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> cnt((size_t)g.n_layers + 1, 0);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess)
    e = hipMemcpy(cnt.data(), (char *)ctx->ws + ctx->off_plan + ctx->plan_cnt,
                  cnt.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(ctx, e, "read-back of the plan's step counters");
  bool freed = false;
  for (size_t i = 0; i < p.blocks.size(); ++i) {
    BlockState &bs = ctx->blocks[p.blocks[i]];
    for (int32_t l = 0; l < g.n_layers; ++l)
      bs.len[l] = p.base[i] + std::min(cnt[l] + p.pending[l], p.n_steps) * p.tps[i];
    const size_t keep = (size_t)((bs.max_len() + g.page_size - 1) / g.page_size);
    while (bs.pages.size() > keep) {
      ctx->free_stack.push_back(bs.pages.back());
      bs.pages.pop_back();
      freed = true;
    }
  }
  if (freed) ctx->page_generation++;
  const bool overflow = cnt[g.n_layers] != 0;
  p = Plan();
  ctx->uploaded_valid = false;
  if (overflow)
    return ctx->fail(HW_ERR_INVALID_ARG, "more planned appends than the plan's steps on some layer; "
                                         "the extra ones were dropped");
  return HW_OK;
}

hw_status hw_reset_block(hw_ctx *ctx, int32_t block_id) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (block_id < 0 || block_id >= ctx->cfg.max_blocks) return ctx->fail(HW_ERR_INVALID_ARG, "block id out of range");
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is active: its blocks grow with hw_append_step; end it with hw_plan_end first");
  BlockState &bs = ctx->blocks[block_id];
  for (auto it = bs.pages.rbegin(); it != bs.pages.rend(); ++it) ctx->free_stack.push_back(*it);
  if (!bs.pages.empty()) ctx->page_generation++;
  bs.pages.clear();
  std::fill(bs.len.begin(), bs.len.end(), 0);
  return HW_OK;
}

hw_status hw_set_split(hw_ctx *ctx, int32_t n_splits) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (n_splits < 0 || n_splits > ctx->cfg.max_splits)
    return ctx->fail(HW_ERR_INVALID_ARG, "n_splits must be in [0, max_splits]");
  ctx->split_override = n_splits;
  return HW_OK;
}

hw_status hw_block_info(const hw_ctx *ctx, int32_t block_id, int32_t layer, int32_t *length,
                        int32_t *pages, int32_t cap, int32_t *n_out) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  hw_ctx *c = const_cast<hw_ctx *>(ctx);
  if (block_id < 0 || block_id >= ctx->cfg.max_blocks) return c->fail(HW_ERR_INVALID_ARG, "block id out of range");
  if (layer < 0 || layer >= ctx->cfg.n_layers) return c->fail(HW_ERR_INVALID_ARG, "layer out of range");
  const BlockState &bs = ctx->blocks[block_id];
  if (length) *length = bs.len[layer];
  if (n_out) *n_out = (int32_t)bs.pages.size();
  if (pages)
    for (int32_t i = 0; i < std::min<int32_t>(cap, (int32_t)bs.pages.size()); ++i) pages[i] = bs.pages[i];
  return HW_OK;
}

hw_status hw_free_pages(const hw_ctx *ctx, int32_t *n_free) {
  if (!ctx || !n_free) return HW_ERR_INVALID_ARG;
  *n_free = (int32_t)ctx->free_stack.size();
  return HW_OK;
}

// ---- hogwild_debug.h ---------------------------------------------------------------

hw_status hw_debug_reserve(hw_ctx *ctx, int32_t layer, int32_t n_blocks, const int32_t *block_ids,
                           const int32_t *n_tokens, int32_t *runs, int32_t cap, int32_t *n_runs) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (ctx->plan.active) return ctx->fail(HW_ERR_INVALID_ARG, "a step plan is active: its blocks grow with hw_append_step; end it with hw_plan_end first");
  AppendPlan plan;
  hw_status st = plan_append(ctx, layer, n_blocks, block_ids, n_tokens, plan);
  if (st != HW_OK) return st;
  if (n_runs) *n_runs = (int32_t)plan.runs.size();
  if ((int32_t)plan.runs.size() > cap || (!runs && !plan.runs.empty()))
    return ctx->fail(HW_ERR_INVALID_ARG, "runs buffer too small");
  for (size_t i = 0; i < plan.runs.size(); ++i) {
    const hw::AppendRun &r = plan.runs[i];
    runs[5 * i] = r.src_row;
    runs[5 * i + 1] = r.page;
    runs[5 * i + 2] = r.slot0;
    runs[5 * i + 3] = r.count;
    runs[5 * i + 4] = r.pos0;
  }
  commit_append(ctx, layer, n_blocks, block_ids, n_tokens, plan);
  return HW_OK;
}

hw_status hw_debug_partition(const uint8_t *block_first, int32_t n_groups, int32_t n_splits,
                             double alpha, int32_t *bounds) {
  if (n_groups < 0 || n_splits < 1 || !(alpha >= 0.0) || !bounds || (n_groups > 0 && !block_first)) {
    g_create_error = "hw_debug_partition: invalid argument";
    return HW_ERR_INVALID_ARG;
  }
  partition_bounds(block_first, n_groups, n_splits, alpha, bounds);
  return HW_OK;
}

hw_status hw_debug_resolve(hw_ctx *ctx, int32_t layer, int32_t *segs, int32_t *delta,
                           int32_t cap_segs, int32_t *n_segs, int32_t *groups,
                           int32_t cap_groups, int32_t *n_groups, int32_t *n_splits) {
  if (!ctx) return HW_ERR_INVALID_ARG;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return ctx->fail(HW_ERR_INVALID_ARG, "layer out of range");
  Resolution r;
  hw_status st = resolve(ctx, layer, r);
  if (st != HW_OK) return st;
  const int32_t ns = (int32_t)r.seg_blocks.size(), ng = (int32_t)r.g_page.size();
  if (n_segs) *n_segs = ns;
  if (n_groups) *n_groups = ng;
  if (n_splits)
    *n_splits = ctx->plan.active ? ctx->plan.splits : choose_splits(ctx, ng, rows_total(ctx, r.n_workers));
  if (ns > cap_segs || ng > cap_groups) return ctx->fail(HW_ERR_INVALID_ARG, "buffers too small");
  if (segs) std::copy(r.seg_blocks.begin(), r.seg_blocks.end(), segs);
  if (delta) std::copy(r.delta.begin(), r.delta.end(), delta);
  if (groups)
    for (int32_t i = 0; i < ng; ++i) {
      groups[4 * i] = r.g_page[i];
      groups[4 * i + 1] = r.g_gip[i];
      groups[4 * i + 2] = r.g_seg[i];
      groups[4 * i + 3] = r.g_valid[i];
    }
  return HW_OK;
}

}  // extern "C"
