// gfx950 (CDNA4) kernels of the Hogwild! concurrent-attention decode step.
//
//   rope_append          RoPE-on-insert of new tokens at block-local positions
//                        [Hogwild! Inference paper summary, s5 steps 1-2; s9]
//   concurrent_decode    split-K attention of every (worker, query head) row of one KV head
//                        over a balanced range of 32-token groups, rotating each worker's
//                        query once per block it enters [summary s5 steps 3-5; s9 kernel]
//   lse_merge            log-sum-exp merge of the split partials [summary s9 "partial
//                        result reduction"; s5 step 5 "aggregate in the softmax weighting"]
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16; v_mfma_f32_16x16x4_f32 for fp32 pools):
//   scores   S^T[token slot, row] = K[slot, :] . Qrot^T[:, row]    A = K tile, B = Qrot
//   output   O^T[d, row]         += V^T[d, token] . P^T[token, row] A = V tile, B = P
// Rows are (worker, query head of the KV head) pairs stacked 16 per tile, so one K/V byte
// read from HBM serves every worker and every query head of its group. Both products keep
// the row index in the MFMA N dimension, so one lane owns one row in S, P and O and the
// softmax needs only two cross-lane exchanges per 32 tokens. The pool layouts (hogwild.h)
// put each lane's 16-byte operand at lane * 16 of a 1 KiB run, so every load is coalesced
// and lands in operand layout with no LDS staging.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hw_internal.h"

namespace hw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Offset of K element (token u of its 32-token group, dim i) inside the group.
__device__ __forceinline__ int k_index(int u, int i) {
  return ((((i >> 5) * 2 + ((u >> 2) & 1)) * 4 + ((i & 31) >> 3)) * 16 + 4 * (u >> 3) + (u & 3)) *
             8 + (i & 7);
}
// Offset of V element (token u, dim i) inside the group.
__device__ __forceinline__ int v_index(int u, int i) {
  return ((((i >> 4) * 4 + (u >> 3)) * 16 + (i & 15)) * 8) + (u & 7);
}

// ------------------------------------------------------------------------------------
// rope_append: one workgroup per (run, KV head).
// ------------------------------------------------------------------------------------

// (a, b) -> (a c - b s, b c + a s), every product and sum rounded to fp32.
__device__ __forceinline__ void rotate_pair(float a, float b, float c, float s, float &lo,
                                            float &hi) {
#pragma clang fp contract(off)
  lo = a * c - b * s;
  hi = b * c + a * s;
}

template <typename KV, int D>
__global__ __launch_bounds__(256) void rope_append_kernel(AppendArgs a) {
  const AppendRun run = a.runs[blockIdx.x];
  const int h = blockIdx.y;
  const int hkv = a.n_kv_heads;
  constexpr int kChunks = D / 16;  // 8-wide chunks in the low half of the head
  const size_t page_head = ((size_t)run.page * hkv + h) * a.page_groups;

  const KV *ksrc = static_cast<const KV *>(a.k_src);
  const KV *vsrc = static_cast<const KV *>(a.v_src);
  KV *kdst = static_cast<KV *>(a.k_layer);
  KV *vdst = static_cast<KV *>(a.v_layer);

  for (int it = threadIdx.x; it < run.count * kChunks; it += blockDim.x) {
    const int i = it / kChunks, c8 = it % kChunks;
    const int t = run.slot0 + i;
    const KV *src = ksrc + ((size_t)(run.src_row + i) * hkv + h) * D;
    const float2 *tr = a.trig + (size_t)(run.pos0 + i) * (D / 2) + 8 * c8;
    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x0, x1;
      if constexpr (sizeof(KV) == 2) {
        x0 = __uint_as_float((uint32_t)(*(const uint16_t *)&src[8 * c8 + e]) << 16);
        x1 = __uint_as_float((uint32_t)(*(const uint16_t *)&src[D / 2 + 8 * c8 + e]) << 16);
      } else {
        x0 = src[8 * c8 + e];
        x1 = src[D / 2 + 8 * c8 + e];
      }
      const float2 cs = tr[e];
      rotate_pair(x0, x1, cs.x, cs.y, lo[e], hi[e]);
    }
    KV *g = kdst + (page_head + t / 32) * (size_t)(32 * D);
    const int u = t & 31;
    KV *plo = g + k_index(u, 8 * c8);
    KV *phi = g + k_index(u, D / 2 + 8 * c8);
    if constexpr (sizeof(KV) == 2) {
      uint4 wlo, whi;
      wlo.x = bf16_rne_bits(lo[0]) | ((uint32_t)bf16_rne_bits(lo[1]) << 16);
      wlo.y = bf16_rne_bits(lo[2]) | ((uint32_t)bf16_rne_bits(lo[3]) << 16);
      wlo.z = bf16_rne_bits(lo[4]) | ((uint32_t)bf16_rne_bits(lo[5]) << 16);
      wlo.w = bf16_rne_bits(lo[6]) | ((uint32_t)bf16_rne_bits(lo[7]) << 16);
      whi.x = bf16_rne_bits(hi[0]) | ((uint32_t)bf16_rne_bits(hi[1]) << 16);
      whi.y = bf16_rne_bits(hi[2]) | ((uint32_t)bf16_rne_bits(hi[3]) << 16);
      whi.z = bf16_rne_bits(hi[4]) | ((uint32_t)bf16_rne_bits(hi[5]) << 16);
      whi.w = bf16_rne_bits(hi[6]) | ((uint32_t)bf16_rne_bits(hi[7]) << 16);
      *reinterpret_cast<uint4 *>(plo) = wlo;
      *reinterpret_cast<uint4 *>(phi) = whi;
    } else {
      float4 *flo = reinterpret_cast<float4 *>(plo);
      float4 *fhi = reinterpret_cast<float4 *>(phi);
      flo[0] = make_float4(lo[0], lo[1], lo[2], lo[3]);
      flo[1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
      fhi[0] = make_float4(hi[0], hi[1], hi[2], hi[3]);
      fhi[1] = make_float4(hi[4], hi[5], hi[6], hi[7]);
    }
  }

  // Values: 8 consecutive tokens of one dim are contiguous; write whole octets when the
  // run covers them, single elements at the run's ragged ends.
  const int first_oct = run.slot0 >> 3;
  const int last_oct = (run.slot0 + run.count - 1) >> 3;
  for (int it = threadIdx.x; it < (last_oct - first_oct + 1) * D; it += blockDim.x) {
    const int oct = first_oct + it / D, i = it % D;
    const int t0 = oct * 8;
    KV *g = vdst + (page_head + t0 / 32) * (size_t)(32 * D) + v_index(t0 & 31, i);
    const bool full = t0 >= run.slot0 && t0 + 8 <= run.slot0 + run.count;
    if (full) {
      KV vals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vals[e] = vsrc[((size_t)(run.src_row + t0 + e - run.slot0) * hkv + h) * D + i];
      if constexpr (sizeof(KV) == 2) {
        *reinterpret_cast<uint4 *>(g) = *reinterpret_cast<const uint4 *>(vals);
      } else {
        reinterpret_cast<float4 *>(g)[0] = make_float4(vals[0], vals[1], vals[2], vals[3]);
        reinterpret_cast<float4 *>(g)[1] = make_float4(vals[4], vals[5], vals[6], vals[7]);
      }
    } else {
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + e;
        if (t >= run.slot0 && t < run.slot0 + run.count)
          g[e] = vsrc[((size_t)(run.src_row + t - run.slot0) * hkv + h) * D + i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// concurrent_decode
// ------------------------------------------------------------------------------------

// Per-dtype pieces: the operand fragments a lane holds and the two matrix products.
template <typename KV, int D>
struct Frag;

template <int D>
struct Frag<__bf16, D> {
  static constexpr int NC = D / 32;   // 32-wide d chunks (MFMA K of the score product)
  static constexpr int NDT = D / 16;  // 16-wide d tiles (MFMA M of the output product)
  uint4 k[NC][2];                     // [chunk][token half] 8 bf16 each
  uint4 v[NDT];                       // [d tile] 8 bf16 (8 tokens of one dim)
  using QOp = bf16x8;                 // rotated query chunk
  using POp = bf16x8;                 // probabilities of 8 tokens

  __device__ __forceinline__ void load(const __bf16 *kg, const __bf16 *vg, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        k[c][hh] = *reinterpret_cast<const uint4 *>(kg + ((c * 2 + hh) * 64 + lane) * 8);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      v[dt] = *reinterpret_cast<const uint4 *>(vg + (dt * 64 + lane) * 8);
  }
  static __device__ __forceinline__ QOp make_q(const float *x) {
    QOp r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
  }
  static __device__ __forceinline__ QOp zero_q() {
    QOp r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)0.0f;
    return r;
  }
  static __device__ __forceinline__ POp make_p(const float *p) { return make_q(p); }
  __device__ __forceinline__ f32x4 score(int c, int hh, const QOp &q, f32x4 acc) const {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[c][hh]), q, acc,
                                                   0, 0, 0);
  }
  __device__ __forceinline__ f32x4 pv(int dt, const POp &p, f32x4 acc) const {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[dt]), p, acc, 0,
                                                   0, 0);
  }
};

struct F8 {
  float x[8];
};

template <int D>
struct Frag<float, D> {
  static constexpr int NC = D / 32;
  static constexpr int NDT = D / 16;
  F8 k[NC][2];
  F8 v[NDT];
  using QOp = F8;
  using POp = F8;

  __device__ __forceinline__ void load(const float *kg, const float *vg, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float4 *p = reinterpret_cast<const float4 *>(kg + ((c * 2 + hh) * 64 + lane) * 8);
        const float4 a0 = p[0], a1 = p[1];
        k[c][hh] = F8{{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w}};
      }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float4 *p = reinterpret_cast<const float4 *>(vg + (dt * 64 + lane) * 8);
      const float4 a0 = p[0], a1 = p[1];
      v[dt] = F8{{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w}};
    }
  }
  static __device__ __forceinline__ QOp make_q(const float *x) {
    QOp r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.x[e] = x[e];
    return r;
  }
  static __device__ __forceinline__ QOp zero_q() {
    QOp r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.x[e] = 0.0f;
    return r;
  }
  static __device__ __forceinline__ POp make_p(const float *p) { return make_q(p); }
  // K step e of chunk c covers dims 32c + 8g + e for lane group g on both operands.
  __device__ __forceinline__ f32x4 score(int c, int hh, const QOp &q, f32x4 acc) const {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[c][hh].x[e], q.x[e], acc, 0, 0, 0);
    return acc;
  }
  // K step e covers tokens 8g + e.
  __device__ __forceinline__ f32x4 pv(int dt, const POp &p, f32x4 acc) const {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt].x[e], p.x[e], acc, 0, 0, 0);
    return acc;
  }
};

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one row: gfx950's
// v_permlane16_swap / v_permlane32_swap exchange rows of 16 lanes without the LDS path.
__device__ __forceinline__ float wave_max_across_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_across_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The running max is only raised (and the accumulators rescaled) when a row's new scores
// exceed it by more than this many doublings; otherwise probabilities are taken against the
// stale max and stay below 2^8, well inside bf16 and fp32 range.
constexpr float kRescaleLog2 = 8.0f;

// Per-wave pipeline state: one 32-token group's operands, its descriptor (wave-uniform) and
// the query offsets of the lane's rows for the group's block.
template <typename KV, int D, int RT>
struct Stage {
  Frag<KV, D> f;
  int desc_x, desc_y;
  int delta[RT];
};

// A wave's group descriptors, 64 at a time: lane j holds descriptor base + j. One vector
// load replaces a dependent scalar load per group.
struct DescBatch {
  long long base;
  int x, y;
};

__device__ __forceinline__ void load_desc_batch(DescBatch &db, const int2 *groups, long long base,
                                                long long end, int lane) {
  db.base = base;
  int2 d = make_int2(0, 0);
  if (base + lane < end) d = groups[base + lane];
  db.x = d.x;
  db.y = d.y;
}

template <typename KV, int D, int RT>
__device__ __forceinline__ void fetch_group(Stage<KV, D, RT> &st, DescBatch &db,
                                            const DecodeArgs &a, const KV *kl, const KV *vl,
                                            size_t head_groups, long long g, long long we,
                                            const int *row_w, int lane) {
  if (g - db.base >= 64) load_desc_batch(db, a.groups, db.base + 64, we, lane);
  const int j = (int)(g - db.base);
  st.desc_x = __builtin_amdgcn_readlane(db.x, j);
  st.desc_y = __builtin_amdgcn_readlane(db.y, j);
  const int seg = st.desc_y >> 8;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) st.delta[rt] = a.delta[(size_t)seg * a.n_workers + row_w[rt]];
  const size_t gb = ((size_t)st.desc_x + head_groups) * (size_t)(32 * D);
  st.f.load(kl + gb, vl + gb, lane);
}

__device__ __forceinline__ int wave_slot() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <typename KV, int D, int RT>
__global__ __launch_bounds__(256, 1) void concurrent_decode_kernel(DecodeArgs a) {
  using F = Frag<KV, D>;
  using S = Stage<KV, D, RT>;
  using QOp = typename F::QOp;
  constexpr int NC = F::NC, NDT = F::NDT;
  // Pipeline stages per wave (NST - 1 groups in flight), as many as the registers allow.
  constexpr int NST = (RT <= 2 && sizeof(KV) == 2) ? 3 : 2;
  constexpr int QSTRIDE = D + 4;                   // padded q row (LDS bank spread)
  constexpr int Q_FLOATS = RT * 16 * QSTRIDE;
  constexpr int QOP_FLOATS = kWaves * RT * NC * 64 * (int)(sizeof(QOp) / 4);
  constexpr int SLOTS = RT * NDT * 64;             // one wave's O^T, f32x4 slots in lane order
  constexpr int M_FLOATS = kWaves * SLOTS * 4;
  constexpr int SMEM = Q_FLOATS + QOP_FLOATS > M_FLOATS ? Q_FLOATS + QOP_FLOATS : M_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM];
  __shared__ double sm_freq[D / 2];
  __shared__ float sm_m[kWaves][64];
  __shared__ float sm_l[kWaves][64];
  __shared__ float sm_rowm[64], sm_rowl[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_slot();
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int row0 = blockIdx.z * a.rows_per_block;
  const int nrows = min(a.rows_per_block, a.rows - row0);
  // Rotated query operands of this wave, in lane order: [rt][chunk][lane].
  QOp *qop_lds = reinterpret_cast<QOp *>(smem + Q_FLOATS) + (size_t)wave * RT * NC * 64;

  // This workgroup's range of token groups, cut into one contiguous range per wave.
  const long long begin = (long long)split * a.n_groups / a.n_splits;
  const long long end = (long long)(split + 1) * a.n_groups / a.n_splits;
  const long long wb = begin + (end - begin) * wave / kWaves;
  const long long we = begin + (end - begin) * (wave + 1) / kWaves;
  const KV *kl = static_cast<const KV *>(a.k_layer);
  const KV *vl = static_cast<const KV *>(a.v_layer);
  const size_t head_groups = (size_t)kvh * a.page_groups;

  int row_w[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    row_ok[rt] = r < nrows;
    row_w[rt] = row_ok[rt] ? (row0 + r) / a.group : 0;
  }

  // Issue order: descriptors, raw queries, then the first groups' K/V, so that waiting for
  // the older loads leaves the K/V loads in flight.
  DescBatch db;
  load_desc_batch(db, a.groups, wb, we, lane);
  constexpr int QPT = (RT * 16 * D + 255) / 256;   // query values per thread
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * 256;
    const int r = i / D, d = i % D;
    qv[k] = 0.0f;
    if (i < RT * 16 * D && r < nrows) {
      const int rr = row0 + r;
      const int w = rr / a.group, gq = rr % a.group;
      qv[k] = a.q[((size_t)w * a.n_q_heads + kvh * a.group + gq) * D + d];
    }
  }
  const double fq = tid < D / 2 ? a.turn_freq[tid] : 0.0;
  S st[NST];
  if (wb < we) {
#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
      fetch_group(st[k], db, a, kl, vl, head_groups, wb + k < we ? wb + k : we - 1, we, row_w, lane);
  }
  // Stage the queries, pre-scaled by softmax_scale * log2(e), and the rotation
  // frequencies in turns per position.
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * 256;
    if (i < RT * 16 * D) smem[(i / D) * QSTRIDE + i % D] = qv[k] * a.q_scale;
  }
  if (tid < D / 2) sm_freq[tid] = fq;
  __syncthreads();

  f32x4 o[RT][NDT];
  float m[RT], l[RT];
  bool rowvis[RT];
  bool rowmask[RT];   // wave-uniform: some real row of this tile does not see the block
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
    rowvis[rt] = false;
    rowmask[rt] = false;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int cur_seg = -1;

  auto process = [&](const S &sg) __attribute__((always_inline)) {
    const int seg = sg.desc_y >> 8;
    const int nvalid = sg.desc_y & 255;
    // Entering a new block: rotate each row's query by delta = q_pos(w) - offset(w, block).
    // The angle delta * theta_j is reduced to a fraction of a turn in fp64; the sine and
    // cosine of that fraction come from the hardware's fp32 units.
    if (seg != cur_seg) {
      cur_seg = seg;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int dl = sg.delta[rt];
        rowvis[rt] = row_ok[rt] && dl >= 0;
        rowmask[rt] = __builtin_amdgcn_ballot_w64(row_ok[rt] && dl < 0) != 0;
        const float *qrow = smem + (rt * 16 + col) * QSTRIDE;
        const double ddl = (double)(dl < 0 ? 0 : dl);
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
          const int j0 = 32 * c + 8 * grp;
          float lo[8], hi[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double turns = ddl * sm_freq[j0 + e];
            const float r = (float)(turns - __builtin_rint(turns));
            const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
            const float x0 = qrow[j0 + e], x1 = qrow[D / 2 + j0 + e];
            lo[e] = x0 * cs - x1 * sn;
            hi[e] = x1 * cs + x0 * sn;
          }
          qop_lds[(rt * NC + c) * 64 + lane] = rowvis[rt] ? F::make_q(lo) : F::zero_q();
          qop_lds[(rt * NC + c + NC / 2) * 64 + lane] = rowvis[rt] ? F::make_q(hi) : F::zero_q();
          // one chunk at a time: keeps the rotation's temporaries from crowding out the
          // accumulators and the stages in flight
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // Scores of the 32 tokens for every row: lane (row col, group grp) gets tokens
    // 8*grp + 4*hh + r of row rt*16 + col in sc[rt][hh][r].
    f32x4 sc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) acc = sg.f.score(c, hh, qop_lds[(rt * NC + c) * 64 + lane], acc);
        sc[rt][hh] = acc;
      }

    // Online softmax in the log2 domain, one row per lane, 8 tokens per lane. At most one
    // uniform branch for masking and one for rescaling per group, so that the MFMAs of one
    // row tile can overlap the softmax of the next. Rows past the workgroup's real rows
    // are never written out, so they need no mask.
    float v8[RT][8], mx[RT];
    bool any_mask = nvalid < 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) any_mask |= rowmask[rt];
    if (any_mask) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * grp + e;
          const float x = sc[rt][e >> 2][e & 3];
          v8[rt][e] = ((rowvis[rt] || !row_ok[rt]) && u < nvalid) ? x : -INFINITY;
        }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[rt][e] = sc[rt][e >> 2][e & 3];
    }
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x = v8[rt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) x = fmaxf(x, v8[rt][e]);
      mx[rt] = wave_max_across_groups(x);
      grow |= mx[rt] > m[rt] + kRescaleLog2;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mnew = fmaxf(m[rt], mx[rt]);
        const float alpha = __builtin_amdgcn_exp2f(m[rt] - (mnew == -INFINITY ? 0.0f : mnew));
        l[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
        m[rt] = mnew;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float msafe = m[rt] == -INFINITY ? 0.0f : m[rt];
      float p[8], sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(v8[rt][e] - msafe);
        sum += p[e];
      }
      l[rt] += sum;
      const typename F::POp pop = F::make_p(p);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = sg.f.pv(dt, pop, o[rt][dt]);
    }
  };

  // NST stages per wave: while one group is computed the next NST-1 load. The prefetch is
  // unconditional (past the end the last group is fetched again, from cache) so that the
  // wait for a stage never has to assume that no younger loads are outstanding.
  if (wb < we) {
    long long gi = wb;
    for (;;) {
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const long long gf = gi + NST - 1;
        fetch_group(st[(k + NST - 1) % NST], db, a, kl, vl, head_groups, gf < we ? gf : we - 1,
                    we, row_w, lane);
        process(st[k]);
        if (++gi >= we) goto groups_done;
      }
    }
  }
groups_done:

  // ---- combine the four waves: common max, then one LDS pass in which every wave adds
  // a quarter of the rows' slots in fixed order (w0 + w1) + (w2 + w3) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l[rt] = wave_sum_across_groups(l[rt]);
  __syncthreads();  // every wave is done with the staged queries
  if (grp == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sm_m[wave][rt * 16 + col] = m[rt];
      sm_l[wave][rt * 16 + col] = l[rt];
    }
  }
  __syncthreads();
  f32x4 *buf = reinterpret_cast<f32x4 *>(smem);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][r]);
    const float fac = m[rt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[rt] - mm);
    if (wave == 0 && grp == 0) {
      float ll = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][r];
        ll += mw == -INFINITY ? 0.0f : sm_l[w][r] * __builtin_amdgcn_exp2f(mw - mm);
      }
      sm_rowm[r] = mm;
      sm_rowl[r] = ll;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) buf[wave * SLOTS + (rt * NDT + dt) * 64 + lane] = o[rt][dt] * fac;
  }
  __syncthreads();

  const bool direct = a.n_splits == 1;
  for (int sl = tid; sl < SLOTS; sl += 256) {
    const int rt = sl / (NDT * 64), dt = (sl / 64) % NDT, ln = sl % 64;
    const int r = rt * 16 + (ln & 15);
    if (r >= nrows) continue;
    const f32x4 x = (buf[sl] + buf[SLOTS + sl]) + (buf[2 * SLOTS + sl] + buf[3 * SLOTS + sl]);
    const float L = sm_rowl[r];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int rr = row0 + r;
    float *dst;
    if (direct) {
      const int w = rr / a.group, h = kvh * a.group + rr % a.group;
      dst = a.out + ((size_t)w * a.n_q_heads + h) * D;
      if (dt == 0 && (ln >> 4) == 0 && a.lse)
        a.lse[(size_t)w * a.n_q_heads + h] =
            L > 0.0f ? (sm_rowm[r] + __log2f(L)) * 0.69314718055994531f : -INFINITY;
    } else {
      const size_t prow = ((size_t)split * a.n_kv_heads + kvh) * a.rows + rr;
      dst = a.part_o + prow * D;
      if (dt == 0 && (ln >> 4) == 0) a.part_lse[prow] = L > 0.0f ? sm_rowm[r] + __log2f(L) : -INFINITY;
    }
    *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * (ln >> 4)) =
        make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
  }
}

// ------------------------------------------------------------------------------------
// lse_merge: four lanes per (worker, query head, 4 output dims); lane j of the four merges
// partials j, j+4, ... with all of its loads in flight together, and the four running
// results are combined with lane exchanges.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  constexpr int Q4 = D / 4;
  constexpr int B = 8;   // partials per lane whose loads are in flight together
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int sub = t & 3;
  const int item = t >> 2;
  const bool live = item < a.n_workers * a.n_q_heads * Q4;
  const int it = live ? item : 0;
  const int row = it / Q4, q4 = it % Q4;
  const int w = row / a.n_q_heads, h = row % a.n_q_heads;
  const int kvh = h / a.group;
  const int rr = w * a.group + h % a.group;
  const size_t stride = (size_t)a.n_kv_heads * a.rows;
  const size_t base = (size_t)kvh * a.rows + rr;
  float mm = -INFINITY, tot = 0.0f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = sub; p0 < a.n_splits; p0 += 4 * B) {
    float lp[B];
    float4 x[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int p = p0 + 4 * i < a.n_splits ? p0 + 4 * i : 0;
      lp[i] = a.part_lse[base + p * stride];
      x[i] = reinterpret_cast<const float4 *>(a.part_o + (base + p * stride) * D)[q4];
    }
    float bm = mm;
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (p0 + 4 * i < a.n_splits) bm = fmaxf(bm, lp[i]);
    if (bm == -INFINITY) continue;
    const float sc = __builtin_amdgcn_exp2f(mm - bm);
    tot *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const float wt = (p0 + 4 * i < a.n_splits) ? __builtin_amdgcn_exp2f(lp[i] - bm) : 0.0f;
      tot += wt;
      acc += wt * f32x4{x[i].x, x[i].y, x[i].z, x[i].w};
    }
    mm = bm;
  }
#pragma unroll
  for (int off = 1; off < 4; off <<= 1) {
    const float om = __shfl_xor(mm, off);
    const float ot = __shfl_xor(tot, off);
    f32x4 oa;
#pragma unroll
    for (int k = 0; k < 4; ++k) oa[k] = __shfl_xor(acc[k], off);
    const float nm = fmaxf(mm, om);
    const float fs = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mm - nm);
    const float fo = om == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(om - nm);
    tot = tot * fs + ot * fo;
    acc = acc * fs + oa * fo;
    mm = nm;
  }
  if (!live || sub != 0) return;
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  reinterpret_cast<float4 *>(a.out + ((size_t)w * a.n_q_heads + h) * D)[q4] =
      make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (q4 == 0 && a.lse)
    a.lse[(size_t)w * a.n_q_heads + h] =
        tot > 0.0f ? (mm + __log2f(tot)) * 0.69314718055994531f : -INFINITY;
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------

hipError_t launch_append(hw_dtype dt, int head_dim, const AppendArgs &a, hipStream_t s) {
  dim3 grid(a.n_runs, a.n_kv_heads), block(256);
  if (dt == HW_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((rope_append_kernel<__bf16, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((rope_append_kernel<__bf16, 64>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((rope_append_kernel<float, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((rope_append_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Launched with hipExtLaunchKernelGGL so that optional start/stop events are recorded by
// the kernel's own dispatch (null events: a plain launch).
template <typename KV, int D>
static void launch_decode_rt(int rt, const DecodeArgs &a, dim3 grid, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1) {
  dim3 block(256);
  if constexpr (sizeof(KV) == 4) {
    if (rt == 1) hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 1>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 2>), grid, block, 0, s, e0, e1, 0, a);
  } else {
    switch (rt) {
      case 1: hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 1>), grid, block, 0, s, e0, e1, 0, a); break;
      case 2: hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 2>), grid, block, 0, s, e0, e1, 0, a); break;
      case 3: hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 3>), grid, block, 0, s, e0, e1, 0, a); break;
      default: hipExtLaunchKernelGGL((concurrent_decode_kernel<KV, D, 4>), grid, block, 0, s, e0, e1, 0, a); break;
    }
  }
}

hipError_t launch_decode(hw_dtype dt, int head_dim, const DecodeArgs &a, int row_blocks,
                         hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int rows_first = a.rows < a.rows_per_block ? a.rows : a.rows_per_block;
  const int rt = (rows_first + 15) / 16;
  dim3 grid(a.n_splits, a.n_kv_heads, row_blocks);
  if (dt == HW_BF16) {
    if (head_dim == 128) launch_decode_rt<__bf16, 128>(rt, a, grid, s, ev_start, ev_stop);
    else launch_decode_rt<__bf16, 64>(rt, a, grid, s, ev_start, ev_stop);
  } else {
    if (head_dim == 128) launch_decode_rt<float, 128>(rt, a, grid, s, ev_start, ev_stop);
    else launch_decode_rt<float, 64>(rt, a, grid, s, ev_start, ev_stop);
  }
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const MergeArgs &a, hipStream_t s) {
  const int threads = 4 * a.n_workers * a.n_q_heads * (head_dim / 4);
  dim3 grid((threads + 255) / 256), block(256);
  if (head_dim == 128) hipLaunchKernelGGL((lse_merge_kernel<128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((lse_merge_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace hw
