// gfx950 (CDNA4) kernels of the Hogwild! concurrent-attention decode step.
//
//   rope_append          RoPE-on-insert of new tokens at block-local positions
//                        [Hogwild! Inference paper summary, s5 steps 1-2; s9]
//   plan_append          the same for one planned step of a step plan (positions from the
//                        layer's device counter), and advance, which moves that counter on
//   concurrent_decode    split-K attention of every (worker, [query token,] query head) row of one KV head
//                        over a balanced range of 32-token groups, rotating each worker's
//                        query once per block it enters [summary s5 steps 3-5; s9 kernel]
//   lse_merge            log-sum-exp merge of the split partials [summary s9 "partial
//                        result reduction"; s5 step 5 "aggregate in the softmax weighting"]
//   stream_read          a plain streaming read, the bandwidth ceiling the decode is measured
//                        against (debug entry point)
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16; v_mfma_f32_16x16x4_f32 for fp32 pools):
//   scores   S^T[token slot, row] = K[slot, :] . Qrot^T[:, row]    A = K tile, B = Qrot
//   output   O^T[d, row]         += V^T[d, token] . P^T[token, row] A = V tile, B = P
// Rows are (worker, query head of the KV head) pairs, or (worker, query token, head) with
// several query tokens per worker, stacked 16 per tile, so one K/V byte read from HBM serves
// every worker and every query head of its group. Both products keep
// the row index in the MFMA N dimension, so one lane owns one row in S, P and O and the
// softmax needs only two cross-lane exchanges per 32 tokens. The pool layouts (hogwild.h)
// put each lane's 16-byte operand at lane * 16 of a 1 KiB run, so every load is coalesced
// and lands in operand layout with no shuffle: straight into registers, or (the 8-wave bf16
// kernels) through a per-wave LDS stage that LDS-DMA loads fill while the wave computes the
// previous group.
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

// One key chunk of one token and head: its 8 rotated pairs (dims 8*c8 + e and D/2 + 8*c8 + e,
// e < 8) from the raw key row ksrc (head_dim elements) and the position's (cos, sin) row
// trig (D/2 pairs), stored into slot u of the head's group kg, the chunk's 8 dims of one
// token being contiguous in the K layout (16 or 32 bytes).
template <typename KV, int D>
__device__ __forceinline__ void put_key_chunk(const KV *ksrc, const float2 *trig, KV *kg, int u, int c8) {
  constexpr int kVec = 16 / (int)sizeof(KV);   // elements per 16-byte access
  static_assert(8 % kVec == 0, "8-element chunks in 16-byte accesses");
  uint4 kl[8 / kVec], kh[8 / kVec];
#pragma unroll
  for (int j = 0; j < 8 / kVec; ++j) {
    kl[j] = *reinterpret_cast<const uint4 *>(ksrc + 8 * c8 + kVec * j);
    kh[j] = *reinterpret_cast<const uint4 *>(ksrc + D / 2 + 8 * c8 + kVec * j);
  }
  float4 cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cs[j] = reinterpret_cast<const float4 *>(trig + 8 * c8)[j];
  const KV *x0 = reinterpret_cast<const KV *>(kl), *x1 = reinterpret_cast<const KV *>(kh);
  const float *cf = reinterpret_cast<const float *>(cs);
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a0, a1;
    if constexpr (sizeof(KV) == 2) {
      a0 = __uint_as_float((uint32_t)(*(const uint16_t *)&x0[e]) << 16);
      a1 = __uint_as_float((uint32_t)(*(const uint16_t *)&x1[e]) << 16);
    } else {
      a0 = x0[e];
      a1 = x1[e];
    }
    rotate_pair(a0, a1, cf[2 * e], cf[2 * e + 1], lo[e], hi[e]);
  }
  KV *klo = kg + k_index(u, 8 * c8), *khi = kg + k_index(u, D / 2 + 8 * c8);
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
    *reinterpret_cast<uint4 *>(klo) = wlo;
    *reinterpret_cast<uint4 *>(khi) = whi;
  } else {
    reinterpret_cast<float4 *>(klo)[0] = make_float4(lo[0], lo[1], lo[2], lo[3]);
    reinterpret_cast<float4 *>(klo)[1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
    reinterpret_cast<float4 *>(khi)[0] = make_float4(hi[0], hi[1], hi[2], hi[3]);
    reinterpret_cast<float4 *>(khi)[1] = make_float4(hi[4], hi[5], hi[6], hi[7]);
  }
}

// ------------------------------------------------------------------------------------
// plan_append: the append of one planned step of one layer; one workgroup per input row.
// Every thread reads the layer's step counter s and nothing here writes it (the kernel
// after the layer's decode advances it). Values: one element per thread and pass, the
// passes' loads issued before their stores. Keys: one item = (KV head, 8-dim chunk), the 8
// rotated pairs (dims c, c + D/2 for c in the chunk), written 16 bytes at a time.
// ------------------------------------------------------------------------------------
template <typename KV, int D>
__global__ __launch_bounds__(256) void plan_append_kernel(PlanAppendArgs a) {
  constexpr int kChunks = D / 16;
  const int hkv = a.n_kv_heads;
  const KV *__restrict__ ksrc = static_cast<const KV *>(a.k_src);
  const KV *__restrict__ vsrc = static_cast<const KV *>(a.v_src);
  KV *__restrict__ kdst = static_cast<KV *>(a.k_layer);
  KV *__restrict__ vdst = static_cast<KV *>(a.v_layer);
  const int s = a.step[0];
  if (s >= a.n_steps) {   // past the plan: nothing is written, the host reports it
    if (blockIdx.x == 0 && threadIdx.x == 0) a.overflow[0] = 1;
    return;
  }
  // This workgroup's row: its block (wave-uniform search), position, page and slot.
  const int r = blockIdx.x;
  int bi = 0;
  for (int i = 0; i < a.n_blocks; ++i)
    if (r >= a.blocks[i].row0 && r < a.blocks[i].row0 + a.blocks[i].tps) bi = i;
  const PlanBlock &b = a.blocks[bi];
  const int pos = b.base + s * b.tps + (r - b.row0);
  const int page = a.pages[b.pages_off + pos / a.page_size - b.page0];
  const int t = pos % a.page_size, u = t & 31;
  const size_t head0 = (size_t)page * hkv * a.page_groups + t / 32;   // group of KV head 0
  const size_t src0 = (size_t)r * hkv * D;
  // Values: thread -> (head, dim), consecutive threads on consecutive dims.
  constexpr int VU = 4;
  for (int i0 = threadIdx.x; i0 < hkv * D; i0 += blockDim.x * VU) {
    KV val[VU];
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      const int idx = i0 + k * blockDim.x;
      val[k] = vsrc[src0 + (idx < hkv * D ? idx : 0)];
    }
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      const int idx = i0 + k * blockDim.x;
      if (idx < hkv * D) {
        const int h = idx / D, i = idx % D;
        vdst[(head0 + (size_t)h * a.page_groups) * (size_t)(32 * D) + v_index(u, i)] = val[k];
      }
    }
  }
  // Keys: thread -> (head, 8-dim chunk).
  for (int it = threadIdx.x; it < hkv * kChunks; it += blockDim.x) {
    const int c8 = it % kChunks, h = it / kChunks;
    put_key_chunk<KV, D>(ksrc + src0 + (size_t)h * D, a.trig + (size_t)pos * (D / 2),
                         kdst + (head0 + (size_t)h * a.page_groups) * (size_t)(32 * D), u, c8);
  }
}

// One thread: a step plan's layer counter, advanced by one up to cap (the decode of the
// layer has read it). Used when no merge follows the decode.
__global__ void advance_kernel(int32_t *counter, int32_t cap) {
  if (threadIdx.x == 0) {
    const int v = counter[0];
    counter[0] = v < cap ? v + 1 : v;
  }
}

// ------------------------------------------------------------------------------------
// concurrent_decode
// ------------------------------------------------------------------------------------

// Per-dtype pieces: the operand fragments a lane holds and the two matrix products.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16-byte load, with the non-temporal (streaming) hint when NT.
template <bool NT>
__device__ __forceinline__ uint4 ld16(const __bf16 *p) {
  if constexpr (NT) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  } else {
    return *reinterpret_cast<const uint4 *>(p);
  }
}

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

  // NT: the group is read by one wave only, so its loads carry the streaming hint and do
  // not evict the small tables that every launch reads first (descriptors, offsets,
  // queries). Groups read by two waves keep ordinary loads: the second read hits L2.
  template <bool NT>
  __device__ __forceinline__ void load(const __bf16 *kg, const __bf16 *vg, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        k[c][hh] = ld16<NT>(kg + ((c * 2 + hh) * 64 + lane) * 8);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) v[dt] = ld16<NT>(vg + (dt * 64 + lane) * 8);
  }
  // The same 16 loads straight into LDS (one 1 KiB slot per load, lane l's 16 bytes at
  // l * 16), with the streaming hint when NT; stage_read then picks up exactly what load
  // would have given.
  template <bool NT = true>
  __device__ __forceinline__ static void load_lds(const __bf16 *kg, const __bf16 *vg, int lane,
                                                  uint4 (*slot)[64]) {
    constexpr int aux = NT ? 2 : 0;   // cache policy: nt
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        __builtin_amdgcn_global_load_lds(kg + ((c * 2 + hh) * 64 + lane) * 8, &slot[c * 2 + hh][0], 16, 0, aux);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      __builtin_amdgcn_global_load_lds(vg + (dt * 64 + lane) * 8, &slot[NC * 2 + dt][0], 16, 0, aux);
  }
  __device__ __forceinline__ void stage_read(const uint4 (*slot)[64], int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) k[c][hh] = slot[c * 2 + hh][lane];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) v[dt] = slot[NC * 2 + dt][lane];
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
  // Zero the values of the group's slots u >= nvalid, which no token occupies: their pool
  // bytes are whatever the memory held, and a probability of 0 times a NaN is still NaN.
  // Lane l holds tokens 8 * (l / 16) + e, e = 0..7, two per dword.
  __device__ __forceinline__ void mask_tail(int nvalid, int lane) {
    const int u0 = 8 * (lane >> 4);
    uint32_t m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m[j] = (u0 + 2 * j < nvalid ? 0x0000FFFFu : 0u) | (u0 + 2 * j + 1 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v[dt].x &= m[0];
      v[dt].y &= m[1];
      v[dt].z &= m[2];
      v[dt].w &= m[3];
    }
  }
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

  template <bool NT>
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
  // As for bf16: lane l holds tokens 8 * (l / 16) + e of one dim in v[dt].x[e].
  __device__ __forceinline__ void mask_tail(int nvalid, int lane) {
    const int u0 = 8 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[dt].x[e] = u0 + e < nvalid ? v[dt].x[e] : 0.0f;
  }
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

// Group descriptors are wave-uniform: they are read through the scalar cache (constant
// address space), whose loads are counted apart from the vector loads of K and V.
typedef __attribute__((address_space(4))) const int ConstInt;
// A group descriptor: page-group index of head 0, segment << 8 | valid tokens, and the
// local position of the group's first token in its block (ls; read from 4-int descriptors,
// which several-token decodes use for their causal mask; 0 otherwise).
struct GDesc {
  int x = 0, y = 0, ls = 0;
};
// Under a step plan (PLAN) a descriptor is {x, segment << 8, v0, rate}: the group holds
// clamp(v0 + pstep * rate, 0, 32) tokens after pstep planned appends of the layer.
template <bool MT, bool PLAN = false>
__device__ __forceinline__ GDesc load_desc(const int2 *groups, long long i, int stride,
                                           int pstep = 0) {
  const ConstInt *p = (const ConstInt *)groups + (long long)stride * i;
  GDesc d;
  d.x = p[0];
  d.y = p[1];
  if constexpr (MT) d.ls = p[2];
  if constexpr (PLAN) {
    const int v = p[2] + pstep * p[3];
    d.y = (d.y & ~255) | (v < 0 ? 0 : (v > 32 ? 32 : v));
  }
  return d;
}

// A wide descriptor (kWideStride ints): the group's {x, y} and the query offsets of workers
// 0..kWideWorkers-1 for its segment, all wave-uniform, in one scalar-cache read. The offsets
// are kept as named fields (not an array) so that picking one per lane stays a register
// select.
static_assert(kWideWorkers == 6, "WideOff holds six offsets");
struct WideOff {
  int o0 = -1, o1 = -1, o2 = -1, o3 = -1, o4 = -1, o5 = -1;
};
__device__ __forceinline__ GDesc load_desc_wide(const int2 *groups, long long i, WideOff &w) {
  const ConstInt *p = (const ConstInt *)groups + (long long)kWideStride * i;
  w.o0 = p[2];
  w.o1 = p[3];
  w.o2 = p[4];
  w.o3 = p[5];
  w.o4 = p[6];
  w.o5 = p[7];
  GDesc d;
  d.x = p[0];
  d.y = p[1];
  return d;
}
// (readfirstlane of the wave-uniform fields keeps the compiler from turning the selects
// into one load at a computed offset, which would put the offsets in memory)
__device__ __forceinline__ int wide_pick(const WideOff &w, int k) {
  int v = __builtin_amdgcn_readfirstlane(w.o0);
  v = k == 1 ? __builtin_amdgcn_readfirstlane(w.o1) : v;
  v = k == 2 ? __builtin_amdgcn_readfirstlane(w.o2) : v;
  v = k == 3 ? __builtin_amdgcn_readfirstlane(w.o3) : v;
  v = k == 4 ? __builtin_amdgcn_readfirstlane(w.o4) : v;
  v = k == 5 ? __builtin_amdgcn_readfirstlane(w.o5) : v;
  return v;
}

// Per-wave pipeline state: one 32-token group's operands and its descriptor (wave-uniform).
template <typename KV, int D>
struct Stage {
  Frag<KV, D> f;
  int desc_x, desc_y, desc_ls;
};

// Issue one group's K and V loads. NTH: the group is read by one wave only (streaming
// hint). Several row blocks of one KV head read every group once each (several query
// tokens per worker): their loads are ordinary, so that all but the first read hit L2.
template <typename KV, int D, bool NTH = true>
__device__ __forceinline__ void fetch_group(Stage<KV, D> &st, GDesc desc, const KV *kl,
                                            const KV *vl, size_t head_groups, int lane) {
  st.desc_x = desc.x;
  st.desc_y = desc.y;
  st.desc_ls = desc.ls;
  const size_t gb = ((size_t)desc.x + head_groups) * (size_t)(32 * D);
  st.f.template load<NTH>(kl + gb, vl + gb, lane);
}

// The query offset of worker w for the block of segment seg. Under a step plan the table
// holds {d0, rate} pairs and the offset is d0 + pstep * rate ({-1, 0}: not visible).
template <bool PLAN>
__device__ __forceinline__ int delta_at(const DecodeArgs &a, int seg, int w, int pstep) {
  const size_t i = (size_t)seg * a.n_workers + w;
  if constexpr (PLAN) {
    const int2 e = reinterpret_cast<const int2 *>(a.delta)[i];
    return e.x + pstep * e.y;
  } else {
    return a.delta[i];
  }
}

// Issue the loads of the query offsets of the lane's rows for the block of segment seg.
template <bool PLAN, int RT>
__device__ __forceinline__ void fetch_delta(int (&dl)[RT], int seg, const DecodeArgs &a,
                                            const int *row_w, int pstep) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) dl[rt] = delta_at<PLAN>(a, seg, row_w[rt], pstep);
}

__device__ __forceinline__ int wave_slot() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A workgroup barrier for LDS only: it waits for this wave's LDS (and scalar) accesses, not
// for its vector loads, so the K/V loads and stage fills in flight keep streaming across it.
// (__syncthreads waits for every outstanding vector load first.) The memory clobber keeps
// the compiler from moving memory accesses across it.
// s_waitcnt operand that waits for every vector memory and LDS/scalar access of the wave
// (gfx9 encoding: vmcnt 0 in bits 3:0 and 15:14, expcnt 7 in bits 6:4, lgkmcnt 0 in bits
// 11:8). Issued through the builtin, the compiler's own wait tracking sees it.
constexpr unsigned kWaitAll = 0x0070;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Segments whose rotated queries one phase of the cooperative rotation holds in LDS: about
// 64 KiB of operands.
template <typename KV, int D, int RT>
constexpr int phase_segments() {
  constexpr int per_seg = RT * (D / 32) * 64 * (int)sizeof(typename Frag<KV, D>::QOp);
  constexpr int c = (64 * 1024) / per_seg;
  return c < 1 ? 1 : (c > 16 ? 16 : c);
}

// The launch arguments the decode prologue needs (the first 96 bytes of DecodeArgs, and the
// workgroup's two partition bounds), read with three scalar loads that go out together and
// one wait, instead of one round trip per field as each is first used.
typedef int i32x16a __attribute__((ext_vector_type(16), aligned(4)));
typedef int i32x8a __attribute__((ext_vector_type(8), aligned(4)));
typedef int i32x2a __attribute__((ext_vector_type(2), aligned(4)));
static_assert(offsetof(DecodeArgs, k_layer) == 0 && offsetof(DecodeArgs, v_layer) == 8 &&
                  offsetof(DecodeArgs, q) == 16 && offsetof(DecodeArgs, groups) == 24 &&
                  offsetof(DecodeArgs, turn_freq) == 32 && offsetof(DecodeArgs, n_groups) == 40 &&
                  offsetof(DecodeArgs, n_splits) == 44 && offsetof(DecodeArgs, rows) == 48 &&
                  offsetof(DecodeArgs, rows_per_block) == 52 && offsetof(DecodeArgs, group) == 56 &&
                  offsetof(DecodeArgs, n_q_heads) == 60 && offsetof(DecodeArgs, page_groups) == 64 &&
                  offsetof(DecodeArgs, desc_stride) == 68 && offsetof(DecodeArgs, inv_group) == 72 &&
                  offsetof(DecodeArgs, split_begin) % 4 == 0,
              "DecodeArgs layout read by load_head");
struct Head {
  const void *k_layer, *v_layer;
  const float *q;
  const int2 *groups;
  const double *turn_freq;
  int n_groups, n_splits, rows, rows_per_block, group, n_q_heads, page_groups, desc_stride;
  float inv_group;
  int sb0, sb1;   // split_begin[sp], split_begin[sp + 1]
};
// A device pointer rebuilt from its two halves, marked global (address space 1), so that the
// accesses through it stay global loads: as a plain generic pointer they would become flat
// loads, which also count on lgkmcnt and serialise with the scalar loads.
__device__ __forceinline__ const void *ptr_of(int lo, int hi) {
  typedef __attribute__((address_space(1))) const char GChar;
  return (const void *)(GChar *)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ Head load_head(int sp) {
  typedef __attribute__((address_space(4))) const i32x16a C16;
  typedef __attribute__((address_space(4))) const i32x8a C8;
  typedef __attribute__((address_space(4))) const i32x2a C2;
  const ConstInt *kp = (const ConstInt *)__builtin_amdgcn_kernarg_segment_ptr();
  const i32x16a h0 = *(C16 *)kp;
  const i32x8a h1 = *(C8 *)(kp + 16);
  const i32x2a sb = *(C2 *)(kp + offsetof(DecodeArgs, split_begin) / 4 + sp);
  // One wait for all three: without the scheduling barrier the compiler issues each load
  // after the first use of the one before (three round trips instead of one), and the asm
  // use keeps the partition bounds' load out of the branch that reads them. (w4_16k:
  // 1.392 against 1.411 ms per step.)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(h0[0]), "s"(h1[0]), "s"(sb[0]));
  Head h;
  h.k_layer = ptr_of(h0[0], h0[1]);
  h.v_layer = ptr_of(h0[2], h0[3]);
  h.q = static_cast<const float *>(ptr_of(h0[4], h0[5]));
  h.groups = static_cast<const int2 *>(ptr_of(h0[6], h0[7]));
  h.turn_freq = static_cast<const double *>(ptr_of(h0[8], h0[9]));
  h.n_groups = h0[10];
  h.n_splits = h0[11];
  h.rows = h0[12];
  h.rows_per_block = h0[13];
  h.group = h0[14];
  h.n_q_heads = h0[15];
  h.page_groups = h1[0];
  h.desc_stride = h1[1];
  h.inv_group = __int_as_float(h1[2]);
  h.sb0 = sb[0];
  h.sb1 = sb[1];
  return h;
}

// One workgroup = one (split, KV head, block of up to 16 * RT rows), NW waves. Every wave
// holds all RT row tiles and takes a contiguous run of the workgroup's token groups, so each
// group is read from HBM by exactly one wave.
//
// NST = 1 (NW = 8, two waves per SIMD): a group's loads are issued as soon as the previous
// group is computed, the other wave on the SIMD computing meanwhile. Each wave rotates its
// rows' query when it enters a new segment (block); that work too overlaps the other wave
// and the loads in flight.
//
// NST = 2 (NW = 4, one wave per SIMD, for row tiles whose accumulators fill the registers
// of two waves): the next group is in flight while one is computed. A wave here has no
// sibling to hide a rotation of its 64 rows, so the workgroup rotates cooperatively: its
// groups [begin, end) cover a contiguous range of segments (the group list is ordered by
// segment), and all threads rotate every (segment, row) of that range once into an LDS
// table of MFMA operands, with a table of the query offsets of its workers. A range with
// more segments than the table holds is taken in phases of phase_segments() segments,
// separated by workgroup barriers.
//
// WIDE (NST = 1, at most kWideWorkers workers, all rows in one block): the group list holds
// wide descriptors, so each group's query offsets come with its descriptor through the
// scalar cache instead of as vector loads queued behind the K/V traffic. With bf16 pools a
// WIDE wave then also keeps its next group in flight while it computes one: the next group
// streams straight into a per-wave LDS stage (LDS-DMA loads) and moves to registers once the
// group is done; the rotated query operands stay in registers.
//
// MT (several query tokens per worker, 4-int descriptors): rows are (worker, token, head) and
// each row's keys after its token are masked. One-token kernels carry none of that state.
//
// PLAN (a step plan, one token per worker, narrow 4-int descriptors): group sizes and query
// offsets are affine in the number of planned appends of the layer, read from the device
// at launch (see load_desc and delta_at), so the launch needs no host-side tables update
// from step to step.
template <typename KV, int D, int RT, int NW, int NST, bool WIDE, bool MT, bool PLAN, bool LATE = false>
__global__ __launch_bounds__(NW * 64, 1) void concurrent_decode_kernel(DecodeArgs a) {
  static_assert(NST == 1 || NST == 2, "one or two stages");
  static_assert(!WIDE || NST == 1, "wide descriptors: single-stage kernels");
  static_assert(!(WIDE && MT), "wide descriptors: one token per worker");
  static_assert(!(PLAN && (WIDE || MT)), "step plans: narrow descriptors, one token");
  static_assert(!LATE || (WIDE && NST == 1 && std::is_same<KV, __bf16>::value), "late group 0: staged wide kernels");
  constexpr bool COOP = NST == 2;
  using F = Frag<KV, D>;
  using S = Stage<KV, D>;
  using QOp = typename F::QOp;
  constexpr int NC = F::NC, NDT = F::NDT;
  constexpr int NT = NW * 64;
  constexpr int CAP = COOP ? phase_segments<KV, D, RT>() : 1;   // segments per phase
  constexpr int NWMAX = RT * 16;                    // workers a block's rows can span
  constexpr int QSTRIDE = D + 4;                    // padded q row (LDS bank spread)
  constexpr int Q_FLOATS = RT * 16 * QSTRIDE;
  // Rotated query operands: per phase segment (COOP) or per wave, [rt][chunk][lane] each.
  constexpr bool LDSST = NST == 1 && std::is_same<KV, __bf16>::value;   // LDS stage, see above
  constexpr int NLOAD = NC * 2 + NDT;               // 16-byte loads per lane per group
  constexpr int QT_FLOATS = LDSST ? 0 : (COOP ? CAP : NW) * RT * NC * 64 * (int)(sizeof(QOp) / 4);
  constexpr int STAGE_FLOATS = LDSST ? NW * NLOAD * 64 * 4 : 0;
  constexpr int SLOTS = RT * NDT * 64;              // one wave's O^T, f32x4 slots in lane order
  constexpr int M_FLOATS = NW * SLOTS * 4;
  // LDSST keeps the staged queries in an LDS array of their own, apart from the stage: the
  // compiler orders reads of an array after the LDS fills into it, and the rotation must not
  // wait for the group in flight.
  constexpr int LOOP_FLOATS = (LDSST ? 0 : Q_FLOATS) + QT_FLOATS + STAGE_FLOATS;  // live until the loop ends
  constexpr int SMEM = LOOP_FLOATS > M_FLOATS ? LOOP_FLOATS : M_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM];
  __shared__ __attribute__((aligned(16))) float sm_q[LDSST ? Q_FLOATS : 4];
  float *const qrows = LDSST ? sm_q : smem;   // staged queries [16 * RT][QSTRIDE]
  __shared__ int sm_dl[COOP ? CAP * NWMAX : 1];     // query offsets [segment of phase][worker]
  __shared__ double sm_freq[D / 2];
  __shared__ float sm_m[NW][16 * RT];
  __shared__ float sm_l[NW][16 * RT];
  __shared__ __attribute__((aligned(16))) float sm_f[16 * RT][NW];   // combine factors per row
  __shared__ float sm_inv[16 * RT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_slot();
  const int col = lane & 15, grp = lane >> 4;
  // Grid (KV head, partition, row block): dispatch deals consecutive workgroups to the 8 XCDs
  // in turn, so with 8 KV heads each XCD takes one head's partitions, the same mix of the
  // group list on every XCD.
  const int kvh = blockIdx.x, split = blockIdx.y;
  const int sp = split < kMaxBoundSplits ? split : kMaxBoundSplits - 1;
  const Head hd = load_head(sp);
  const int row0 = blockIdx.z * hd.rows_per_block;
  const int nrows = min(hd.rows_per_block, hd.rows - row0);
  QOp *qt = reinterpret_cast<QOp *>(smem + (LDSST ? 0 : Q_FLOATS));
  QOp *qop_wave = qt + (size_t)wave * RT * NC * 64;   // NST = 1 without LDSST: this wave's operands
  // LDSST: this wave's stage, NLOAD slots of 64 lanes x 16 bytes
  uint4 (*stage)[64] = reinterpret_cast<uint4 (*)[64]>(smem + QT_FLOATS) + wave * NLOAD;
  QOp qreg[RT][NC];   // LDSST: the rotated query operands of the current segment

  // Stacked row rr = (query token wt, head rr - wt * group of the KV head's group) with
  // wt = rr / group, and query token wt = (worker wt / n_new, token wt % n_new): both
  // quotients as floor((x + 0.5) * (1 / y)) in fp32, exact while rr < 2^22 (the error of
  // the product stays below 0.5 / y). With one token per worker, wt is the worker.
  const float inv_group = hd.inv_group;
  auto tok_of = [=](int rr) { return (int)(((float)rr + 0.5f) * inv_group); };

  // Prologue, ordered for latency. The raw queries and the rotation frequencies go out
  // first: they need only launch arguments, and are in flight before the first K/V loads
  // of every wave flood the memory system (the queries gate the barrier before the first
  // group is computed).
  // Loads are unconditional (a padding row reads row 0 of the block, zeroed at staging), so
  // that no wait is needed until the values are staged.
  constexpr int QV4 = (RT * 16 * D / 4 + NT - 1) / NT;   // float4 of queries per thread
  float4 qv[QV4];
  bool qok[QV4];
#pragma unroll
  for (int k = 0; k < QV4; ++k) {
    const int i = tid + k * NT;                      // float4 index in [RT*16][D/4]
    qok[k] = i < RT * 16 * D / 4 && i / (D / 4) < nrows;
    const int r = qok[k] ? i / (D / 4) : 0, d4 = i % (D / 4);
    const int rr = row0 + r;
    const int wt = tok_of(rr), gq = rr - wt * hd.group;
    qv[k] = reinterpret_cast<const float4 *>(hd.q + ((size_t)wt * hd.n_q_heads + kvh * hd.group + gq) * D)[d4];
  }
  const double fq = hd.turn_freq[tid % (D / 2)];

  // This workgroup's token groups [begin, end); this wave's contiguous run of them. Both
  // launch-argument bounds are read unconditionally, so that the scalar loads go out in one
  // batch instead of one round trip after another.
  // Beyond kMaxBoundSplits partitions, the uniform cuts floor(p * n_groups / n_splits) in
  // fp64 (exact: the product stays far below 2^53).
  const int n_splits = hd.n_splits, n_groups = hd.n_groups;
  int begin = hd.sb0, end = hd.sb1;
  if (n_splits > kMaxBoundSplits) {
    begin = (int)((double)split * n_groups / n_splits);
    end = (int)((double)(split + 1) * n_groups / n_splits);
  }
  const int wfirst = begin + (int)((long long)(end - begin) * wave / NW);
  const int wcount = begin + (int)((long long)(end - begin) * (wave + 1) / NW) - wfirst;
  const int wlast = wfirst + (wcount > 0 ? wcount - 1 : 0);
  const KV *kl = static_cast<const KV *>(hd.k_layer);
  const KV *vl = static_cast<const KV *>(hd.v_layer);
  const size_t head_groups = (size_t)kvh * hd.page_groups;

  auto worker_of = [&](int rr) {
    if constexpr (MT) return (int)(((float)rr + 0.5f) * a.inv_rpw);
    else return tok_of(rr);
  };
  // n_new - 1 - t for the token of row rr: it sits that many positions before q_pos
  auto back_of = [&](int rr) {
    if constexpr (MT) return a.n_new - 1 - (tok_of(rr) - worker_of(rr) * a.n_new);
    else return 0;
  };
  // A row's offset into a block: the worker's offset (query position minus block start,
  // -1 if not visible) moved back to the row's token; -1 when the block starts after it.
  auto row_offset = [](int dl, int back) {
    if constexpr (MT) return dl < back ? -1 : dl - back;
    else return dl;
  };
  // The lane's rows: row rt * 16 + col of the workgroup's block.
  int row_w[RT], row_back[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    row_ok[rt] = r < nrows;
    row_w[rt] = row_ok[rt] ? worker_of(row0 + r) : 0;
    row_back[rt] = row_ok[rt] ? back_of(row0 + r) : 0;
  }
  constexpr bool causal = MT;   // several tokens per worker: mask keys after each token
  // Workers of the block's rows: wlo .. wlo + nw - 1 (nw <= NWMAX, one per row at most).
  const int wlo = __builtin_amdgcn_readfirstlane(worker_of(row0));
  const int nw = __builtin_amdgcn_readfirstlane(worker_of(row0 + nrows - 1)) - wlo + 1;

  // Then the scalar loads of this wave's first descriptors (and, COOP, the workgroup's
  // segment range), the offsets (of the first phase, or of this wave's first two groups)
  // and group 0's K/V; only then the waits for the queries and offsets, which leave the
  // K/V loads in flight.
  // A fetch with nothing to fetch (no group for this wave, or past the end of its run)
  // still issues its loads, from descriptor (0, 0): page 0 of the head and the first row of
  // the offset table, both always allocated; the data goes unused. Loads issued
  // unconditionally keep the waits for each stage exact.
  // Step plan: planned appends of this layer so far (wave-uniform, scalar cache).
  int pstep = 0, pcount = 0;
  if constexpr (PLAN) {
    pcount = *(const ConstInt *)a.plan_step;
    const int c = pcount + a.plan_pending;
    pstep = c < a.plan_n_steps ? c : a.plan_n_steps;
  }
  int s_lo = 0, s_hi = -1;
  if constexpr (COOP) {
    // both ends' descriptors loaded unconditionally (indices clamped), one round trip
    const int lastg = n_groups > 0 ? n_groups - 1 : 0;
    const int y0 = load_desc<MT>(hd.groups, min(begin, lastg), hd.desc_stride).y;
    const int y1 = load_desc<MT>(hd.groups, max(min(end - 1, lastg), 0), hd.desc_stride).y;   // (segments: no plan term)
    if (end > begin) {
      s_lo = y0 >> 8;
      s_hi = y1 >> 8;
    }
  }
  const int nph = COOP ? (s_hi - s_lo + CAP) / CAP : 1;   // COOP phases (0 without groups)
  GDesc desc, next, next2;
  // WIDE: the offsets of workers 0.. for the segments of desc, next, next2
  WideOff ow, ow_next, ow_next2;
  auto desc_at = [&](long long i, WideOff &off) __attribute__((always_inline)) {
    if constexpr (WIDE) return load_desc_wide(hd.groups, i, off);
    else return load_desc<MT, PLAN>(hd.groups, i, hd.desc_stride, pstep);
  };
  // The first three descriptors of this wave's run, loaded unconditionally (indices clamped
  // into the list) so that the three loads go out together; a descriptor past the run is then
  // replaced by (0, 0).
  {
    const int lastg = n_groups > 0 ? n_groups - 1 : 0;
    desc = desc_at(min(wfirst, lastg), ow);
    next = desc_at(min(wfirst + 1, lastg), ow_next);
    next2 = desc_at(min(wfirst + 2, lastg), ow_next2);
    if (wcount <= 0) desc = GDesc();
    if (wcount <= 1) next = GDesc();
    if (wcount <= 2) next2 = GDesc();
  }
  // WIDE: the lane's rows' offsets (all rows in one block: worker index = row_w)
  auto wide_rows = [&](int (&dl)[RT], const WideOff &off) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) dl[rt] = wide_pick(off, row_w[rt]);
  };
  // COOP: offsets of the phase starting at segment seg_lo: sm_dl[s * nw + k] = delta of
  // worker wlo + k for segment seg_lo + s (-1: the block is not in that worker's view).
  constexpr int DLPT = COOP ? (CAP * NWMAX + NT - 1) / NT : 1;
  int dlv[DLPT];
  auto load_offsets = [&](int seg_lo) __attribute__((always_inline)) {
    const int cnt = min(CAP, s_hi + 1 - seg_lo) * nw;
#pragma unroll
    for (int k = 0; k < DLPT; ++k) {
      const int t = tid + k * NT;
      dlv[k] = t < cnt ? delta_at<PLAN>(a, seg_lo + t / nw, wlo + t % nw, pstep) : -1;
    }
  };
  auto store_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < DLPT; ++k)
      if (tid + k * NT < CAP * NWMAX) sm_dl[tid + k * NT] = dlv[k];
  };
  S st, st2;   // st: the group being computed; st2 (NST = 2): the group in flight
  int dl_cur[RT], dl_next[RT];   // NST = 1: offsets of the lane's rows for groups i, i+1

  // Fused step: this step's planned append. Every (KV head, group) is read by exactly one
  // wave, so the wave whose run holds a group that the step's tokens fall in writes those
  // tokens for its KV head (the values, and the keys rotated at their positions, byte for
  // byte as plan_append writes them), then makes its writes visible to its own later reads
  // of the group. Positions of block i at count s: base + s * tps + j, j < tps; the block's
  // groups are consecutive in the list from index g0, position p in group g0 + p / 32.
  if constexpr (PLAN && std::is_same<KV, __bf16>::value) {
    if (a.fuse_k != nullptr) {
      if (pcount >= a.plan_n_steps) {   // past the window: nothing is written, the host reports it
        if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) a.fuse_overflow[0] = 1;
      } else if (wcount > 0 && wfirst <= a.fuse_gmax && wlast >= a.fuse_gmin) {
        bool wrote = false;
        KV *const kw = const_cast<KV *>(kl), *const vw = const_cast<KV *>(vl);
        for (int bi = 0; bi < a.fuse_n_blocks; ++bi) {
          const ConstInt *fb = (const ConstInt *)a.fuse_blocks + 4 * bi;
          const int base = fb[0], tps = fb[1], frow = fb[2], g0 = fb[3];
          if (tps <= 0 || g0 < 0) continue;
          const int pa = base + pcount * tps, pb = pa + tps - 1;
          const int ga = max(g0 + (pa >> 5), wfirst), gz = min(g0 + (pb >> 5), wlast);
          for (int gl = ga; gl <= gz; ++gl) {
            const GDesc gd = load_desc<false, true>(hd.groups, gl, hd.desc_stride, pstep);
            const size_t gbase = ((size_t)gd.x + head_groups) * (size_t)(32 * D);
            const int p0 = max(pa, (gl - g0) * 32), p1 = min(pb, (gl - g0) * 32 + 31);
            for (int pos = p0; pos <= p1; ++pos) {
              const size_t src = ((size_t)(frow + pos - pa) * a.n_kv_heads + kvh) * D;
              const KV *ks = static_cast<const KV *>(a.fuse_k) + src;
              const KV *vs = static_cast<const KV *>(a.fuse_v) + src;
              const int u = pos & 31;
              for (int i = lane; i < D; i += 64) vw[gbase + v_index(u, i)] = vs[i];
              if (lane < D / 16)
                put_key_chunk<KV, D>(ks, a.fuse_trig + (size_t)pos * (D / 2), kw + gbase, u, lane);
              wrote = true;
            }
          }
        }
        if (wrote) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
      }
    }
  }
  if constexpr (COOP) {
    load_offsets(s_lo);
    fetch_group(st2, desc, kl, vl, head_groups, lane);
  } else if constexpr (WIDE) {
    // LDSST: the queries land before group 0 is requested, ahead of the flood of every
    // wave's K/V loads (they gate the barrier below)
    if constexpr (LDSST) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (!LATE) fetch_group(st, desc, kl, vl, head_groups, lane);
    wide_rows(dl_cur, ow);
  } else if constexpr (LDSST) {
    // narrow descriptors: the offsets of groups 0 and 1 are vector loads, in before group 0
    // is requested, as the queries are
    fetch_delta<PLAN>(dl_cur, desc.y >> 8, a, row_w, pstep);
    fetch_delta<PLAN>(dl_next, next.y >> 8, a, row_w, pstep);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    fetch_group<KV, D, !MT>(st, desc, kl, vl, head_groups, lane);
  } else {
    fetch_delta<PLAN>(dl_cur, desc.y >> 8, a, row_w, pstep);
    fetch_group<KV, D, !MT>(st, desc, kl, vl, head_groups, lane);
    fetch_delta<PLAN>(dl_next, next.y >> 8, a, row_w, pstep);
  }
  // Stage the queries, pre-scaled by softmax_scale * log2(e), the offsets and the rotation
  // frequencies in turns per position.
#pragma unroll
  for (int k = 0; k < QV4; ++k) {
    const int i = tid + k * NT;
    if (i < RT * 16 * D / 4) {
      const float4 x = qok[k] ? qv[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4 *>(qrows + (i / (D / 4)) * QSTRIDE + (i % (D / 4)) * 4) =
          make_float4(x.x * a.q_scale, x.y * a.q_scale, x.z * a.q_scale, x.w * a.q_scale);
    }
  }
  if constexpr (COOP) store_offsets();
  if (tid < D / 2) sm_freq[tid] = fq;
  lds_barrier();   // the first groups' loads stay in flight
  // LATE (waves of at most about one group): group 0 is requested only now, once every wave's
  // queries are staged. With nothing to overlap it with, an early request only delays the
  // other waves' queries behind the first burst of K/V loads (w2_4k: 0.352 against 0.364 ms
  // per step); with several groups a wave, the early request wins (w4_16k: 1.373 against
  // 1.462 ms).
  if constexpr (LATE) fetch_group(st, desc, kl, vl, head_groups, lane);

  // Rotation of one row's query by delta = q_pos(w) - offset(w, block), for the 8 pairs
  // (j, j + D/2), j = j0 .. j0 + 7: the angle delta * theta_j is reduced to a fraction of a
  // turn in fp64; the sine and cosine of that fraction come from the hardware's fp32 units.
  // rotate8r takes the pairs' values (x0: dims j, x1: dims j + D/2) and frequencies from
  // registers; rotate8 reads them from the staged row and the frequency table.
  auto rotate8r = [&](const float *x0, const float *x1, const double *fv, int dl, float *lo,
                      float *hi) __attribute__((always_inline)) {
    const double ddl = (double)dl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double turns = ddl * fv[e];
      const float fr = (float)(turns - __builtin_rint(turns));
      const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
      lo[e] = x0[e] * cs - x1[e] * sn;
      hi[e] = x1[e] * cs + x0[e] * sn;
    }
  };
  auto rotate8 = [&](const float *qrow, int j0, int dl, float *lo, float *hi) __attribute__((always_inline)) {
    float x0[8], x1[8];
    double fv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x0[e] = qrow[j0 + e];
      x1[e] = qrow[D / 2 + j0 + e];
      fv[e] = sm_freq[j0 + e];
    }
    rotate8r(x0, x1, fv, dl, lo, hi);
  };
  // COOP: rotate every (segment, row) of a phase of nseg segments, all threads together. One
  // item is (segment, row tile, chunk pair, lane).
  auto rotate_phase = [&](int nseg) __attribute__((always_inline)) {
    const int items = nseg * RT * (NC / 2) * 64;
    for (int it = tid; it < items; it += NT) {
      const int ln = it & 63;
      int rest = it >> 6;
      const int c = rest % (NC / 2);
      rest /= NC / 2;
      const int rt = rest % RT, sl = rest / RT;
      const int row = rt * 16 + (ln & 15);
      float lo[8], hi[8];
      bool vis = false;
      if (row < nrows) {
        const int dl = row_offset(sm_dl[sl * nw + worker_of(row0 + row) - wlo], back_of(row0 + row));
        vis = dl >= 0;
        rotate8(qrows + row * QSTRIDE, 32 * c + 8 * (ln >> 4), vis ? dl : 0, lo, hi);
      }
      QOp *dst = qt + ((size_t)(sl * RT + rt) * NC + c) * 64 + ln;
      dst[0] = vis ? F::make_q(lo) : F::zero_q();
      dst[(NC / 2) * 64] = vis ? F::make_q(hi) : F::zero_q();
    }
  };

  f32x4 o[RT][NDT];
  float m[RT], l[RT];
  bool rowvis[RT];
  bool rowmask[RT];   // wave-uniform: some real row of this tile does not see the block
  int rowoff[RT];     // the row's offset into the current block (its keys j <= rowoff)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
    rowvis[rt] = false;
    rowmask[rt] = false;
    rowoff[rt] = -1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int cur_seg = -1;

  // The visibility part of entering a group (NST = 1): the lane's rows' offsets into the
  // group's block.
  auto enter_rows = [&](const int (&delta)[RT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int dl = row_offset(delta[rt], row_back[rt]);
      rowoff[rt] = dl;
      rowvis[rt] = row_ok[rt] && dl >= 0;
      rowmask[rt] = __builtin_amdgcn_ballot_w64(row_ok[rt] && dl < 0) != 0;
    }
  };

  // One group: visibility and (NST = 1, new segment) rotation, scores, online softmax, PV.
  // seg_lo: first segment of the current phase (COOP); delta: the lane's rows' offsets for
  // the group's block (NST = 1).
  // Entering a group: its rows' visibility of the group's block and, when the block is new
  // to the wave (NST = 1), the rotation of the rows' queries. The rotation reads LDS, and
  // the compiler makes an LDS read wait for every LDS-DMA fill in flight, so the staged
  // loop enters a group before it issues the next fill.
  auto enter = [&](const S &sg, int seg_lo, const int (&delta)[RT]) __attribute__((always_inline)) {
    const int seg = sg.desc_y >> 8;
    if constexpr (COOP) {
      const int sl = seg - seg_lo;                   // segment within the phase
      if (seg != cur_seg) {
        cur_seg = seg;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int dl = row_ok[rt] ? row_offset(sm_dl[sl * nw + row_w[rt] - wlo], row_back[rt]) : -1;
          rowoff[rt] = dl;
          rowvis[rt] = row_ok[rt] && dl >= 0;
          rowmask[rt] = __builtin_amdgcn_ballot_w64(row_ok[rt] && dl < 0) != 0;
        }
      }
    } else {
      enter_rows(delta);
      if (seg != cur_seg) {
        cur_seg = seg;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int dl = rowoff[rt];
#pragma unroll
          for (int c = 0; c < NC / 2; ++c) {
            float lo[8], hi[8];
            rotate8(qrows + (rt * 16 + col) * QSTRIDE, 32 * c + 8 * grp, dl < 0 ? 0 : dl, lo, hi);
            if constexpr (LDSST) {
              qreg[rt][c] = rowvis[rt] ? F::make_q(lo) : F::zero_q();
              qreg[rt][c + NC / 2] = rowvis[rt] ? F::make_q(hi) : F::zero_q();
            } else {
              qop_wave[(rt * NC + c) * 64 + lane] = rowvis[rt] ? F::make_q(lo) : F::zero_q();
              qop_wave[(rt * NC + c + NC / 2) * 64 + lane] = rowvis[rt] ? F::make_q(hi) : F::zero_q();
            }
            // one chunk at a time: keeps the rotation's temporaries from crowding out the
            // accumulators and the stage in flight
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };

  // One group after enter: scores, online softmax, PV.
  auto compute = [&](S &sg, int seg_lo) __attribute__((always_inline)) {
    const int seg = sg.desc_y >> 8;
    const int nvalid = sg.desc_y & 255;
    const QOp *qs = COOP ? qt + (size_t)(seg - seg_lo) * RT * NC * 64 + lane : qop_wave + lane;

    // Scores of the 32 tokens for every row: lane (row col, group grp) gets tokens
    // 8*grp + 4*hh + r of row tile rt in sc[rt][hh][r].
    f32x4 sc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc = sg.f.score(c, hh, LDSST ? qreg[rt][c] : qs[(rt * NC + c) * 64], acc);
        sc[rt][hh] = acc;
      }

    // Online softmax in the log2 domain, one row per lane, 8 tokens per lane, with at most
    // one uniform branch for masking and one for rescaling. Rows past the workgroup's real
    // rows are never written out, so they need no mask.
    float v8[RT][8], mx[RT];
    bool any_mask = nvalid < 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) any_mask |= rowmask[rt];
    // Several tokens per worker: a visible row also loses the group's keys after its token
    // (local position ls + u above its offset into the block).
    const int ls = sg.desc_ls;
    if constexpr (causal) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        any_mask |= __builtin_amdgcn_ballot_w64(rowvis[rt] && ls + nvalid - 1 > rowoff[rt]) != 0;
    }
    if (any_mask) {
      if (nvalid < 32) sg.f.mask_tail(nvalid, lane);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * grp + e;
          const float x = sc[rt][e >> 2][e & 3];
          const bool key_ok = !causal || !row_ok[rt] || ls + u <= rowoff[rt];
          v8[rt][e] = ((rowvis[rt] || !row_ok[rt]) && u < nvalid && key_ok) ? x : -INFINITY;
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
  auto process = [&](S &sg, int seg_lo, const int (&delta)[RT]) __attribute__((always_inline)) {
    enter(sg, seg_lo, delta);
    compute(sg, seg_lo);
  };

  if constexpr (LDSST) {
    // Group 0 is in registers; group 1 streams into the stage now, after the queries' LDS
    // writes (the compiler waits for every vector load, fills included, before an LDS
    // write that follows a fill). Group i >= 1 is read from the stage, the fill of group
    // i+1 issued, then group i computed. The compiler does not order stage
    // reads after fills or count fills in its waits, so the waits are explicit: a fill is
    // the only vector load in flight when the stage is read (vmcnt(0) waits for exactly it),
    // and the stage read completes before the refill. Group 0 is computed outside the loop
    // so that no loop iteration carries its register loads (whose waits would then drain
    // the stage in flight).
    // A wave raises its priority while it takes its group from the stage and issues the next
    // fill, and drops it to compute: the other wave on the SIMD, mid-compute, then yields
    // the issue slots to the one whose data has landed, which keeps the fills going.
    //
    // Group 0: the first rotation's inputs are read from LDS into registers, then group 1's
    // fill goes out, then the rotation runs on the registers while both groups stream. The
    // compiler cannot tell which of a mix of pending fills and ordinary loads has completed,
    // so group 0's scores wait for group 1's fill as well. With several tokens per worker
    // the wave first waits for group 0 alone (its row blocks share the groups through L2,
    // and group 0 has mostly landed by then), so that group 0 is computed while group 1
    // streams; a one-token decode's group 0 comes from HBM in the first burst of requests,
    // and waiting for it would hold group 1's request back. (Measured on MI355X, against
    // the first rotation before the fill: w4_16k 1.400 against 1.450 ms per step; w4_16k
    // with 4 tokens 1.770 against 1.831 ms.)
    {
      float qa[RT][NC / 2][8], qb[RT][NC / 2][8];
      double fa[NC / 2][8];
#pragma unroll
      for (int c = 0; c < NC / 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) fa[c][e] = sm_freq[32 * c + 8 * grp + e];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < NC / 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            qa[rt][c][e] = qrows[(rt * 16 + col) * QSTRIDE + 32 * c + 8 * grp + e];
            qb[rt][c][e] = qrows[(rt * 16 + col) * QSTRIDE + D / 2 + 32 * c + 8 * grp + e];
          }
      if constexpr (MT) __builtin_amdgcn_s_waitcnt(kWaitAll);   // group 0 (and the reads above)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      if (wcount > 1) {
        const size_t gb = ((size_t)next.x + head_groups) * (size_t)(32 * D);
        F::template load_lds<!MT>(kl + gb, vl + gb, lane, stage);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (wcount > 0) {
        enter_rows(dl_cur);
        cur_seg = st.desc_y >> 8;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int c = 0; c < NC / 2; ++c) {
            float lo[8], hi[8];
            rotate8r(qa[rt][c], qb[rt][c], fa[c], rowoff[rt] < 0 ? 0 : rowoff[rt], lo, hi);
            qreg[rt][c] = rowvis[rt] ? F::make_q(lo) : F::zero_q();
            qreg[rt][c + NC / 2] = rowvis[rt] ? F::make_q(hi) : F::zero_q();
          }
        compute(st, 0);
      }
    }
    for (int i = 1; i < wcount; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // group i's fill has landed
      st.f.stage_read(stage, lane);
      st.desc_x = next.x;
      st.desc_y = next.y;
      st.desc_ls = next.ls;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // stage read before it is refilled
      next = next2;                                         // group i + 1
      if constexpr (WIDE) {
        ow = ow_next;
        ow_next = ow_next2;
        wide_rows(dl_cur, ow);                              // group i's offsets
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) dl_cur[rt] = dl_next[rt];   // loaded with group i
      }
      enter(st, 0, dl_cur);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < wcount) {
        const size_t gb = ((size_t)next.x + head_groups) * (size_t)(32 * D);
        F::template load_lds<!MT>(kl + gb, vl + gb, lane, stage);
      }
      // narrow descriptors: group i + 1's offsets, in when its fill is
      if constexpr (!WIDE) fetch_delta<PLAN>(dl_next, next.y >> 8, a, row_w, pstep);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      next2 = desc_at(min(wfirst + i + 2, wlast), ow_next2);
      compute(st, 0);
    }
  } else if constexpr (!COOP) {
    // Group i: its descriptor and offsets came with group i-1; group i+1's descriptor is
    // in and group i+2's on its way.
    for (int i = 0; i < wcount; ++i) {
      if (i > 0) {
        desc = next;
        next = next2;
        fetch_group<KV, D, !MT>(st, desc, kl, vl, head_groups, lane);
        if constexpr (WIDE) {
          ow = ow_next;
          ow_next = ow_next2;
          wide_rows(dl_cur, ow);
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) dl_cur[rt] = dl_next[rt];
          fetch_delta<PLAN>(dl_next, next.y >> 8, a, row_w, pstep);
        }
        next2 = desc_at(min(wfirst + i + 2, wlast), ow_next2);
      }
      process(st, 0, dl_cur);
    }
  } else {
    // Phases: rotate the phase's segments, then every wave computes its groups that lie in
    // them. Group i is in flight in st2 when its step starts; it moves to st and group i+1
    // (descriptor next, in since the last step) is issued into st2 before group i is
    // computed; group i+2's descriptor is on its way.
    int i = 0;
    for (int ph = 0; ph < nph; ++ph) {
      const int seg_lo = s_lo + ph * CAP;
      if (ph > 0) {
        lds_barrier();                               // the previous phase's table is done
        load_offsets(seg_lo);
        store_offsets();
        lds_barrier();
      }
      rotate_phase(min(CAP, s_hi + 1 - seg_lo));
      lds_barrier();
      while (i < wcount && (desc.y >> 8) < seg_lo + CAP) {
        st = st2;
        fetch_group(st2, i + 1 < wcount ? next : GDesc(), kl, vl, head_groups, lane);
        process(st, seg_lo, dl_cur);
        desc = next;
        next = next2;
        next2 = load_desc<MT, PLAN>(a.groups, min(wfirst + i + 3, wlast), a.desc_stride, pstep);
        ++i;
      }
    }
  }

  // ---- combine the waves: each wave leaves its (m, l) per row and its raw O in LDS, then
  // every slot of the output is summed over the waves in a fixed order, each wave's part
  // scaled to the common maximum (results do not depend on timing) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l[rt] = wave_sum_across_groups(l[rt]);
  // LDSST: a wave's O goes into its own stage (no other wave touches it) once its last fill
  // has landed; otherwise into smem, once every wave is done with the queries staged there.
  constexpr int WSTRIDE = LDSST ? NLOAD * 64 : SLOTS;   // f32x4 slots between waves' parts
  static_assert(!LDSST || NLOAD * 64 >= SLOTS, "a wave's O fits its stage");
  if constexpr (LDSST) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else lds_barrier();
  f32x4 *buf = reinterpret_cast<f32x4 *>(smem);
  if (grp == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sm_m[wave][rt * 16 + col] = m[rt];
      sm_l[wave][rt * 16 + col] = l[rt];
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) buf[wave * WSTRIDE + (rt * NDT + dt) * 64 + lane] = o[rt][dt];
  lds_barrier();

  // Per row, once: the common maximum, each wave's factor 2^(m_t - max), 1 / sum and the
  // normaliser (lse); then every output slot is the factor-weighted sum of the waves' parts.
  const bool direct = a.n_splits == 1;
  if (tid < 16 * RT) {
    const int r = tid;
    float mm = -INFINITY;
#pragma unroll
    for (int t = 0; t < NW; ++t) mm = fmaxf(mm, sm_m[t][r]);
    float L = 0.0f;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const float mt = sm_m[t][r];
      const float f = mt == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mt - mm);
      sm_f[r][t] = f;
      L += sm_l[t][r] * f;
    }
    sm_inv[r] = L > 0.0f ? 1.0f / L : 0.0f;
    if (r < nrows) {
      const int rr = row0 + r;
      if (direct) {
        const int wt = tok_of(rr), h = kvh * a.group + rr - wt * a.group;
        if (a.lse)
          a.lse[(size_t)wt * a.n_q_heads + h] =
              L > 0.0f ? (mm + __log2f(L)) * 0.69314718055994531f : -INFINITY;
      } else {
        const size_t prow = ((size_t)split * a.n_kv_heads + kvh) * a.rows + rr;
        a.part_lse[prow] = L > 0.0f ? mm + __log2f(L) : -INFINITY;
      }
    }
  }
  lds_barrier();
  constexpr int ITER = (SLOTS + NT - 1) / NT;
#pragma unroll
  for (int k = 0; k < ITER; ++k) {
    const int q = tid + k * NT;
    const int rt = q / (NDT * 64), dt = (q / 64) % NDT, ln = q % 64;
    const int r = rt * 16 + (ln & 15);
    if (q >= SLOTS || r >= nrows) continue;
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NW; ++t) x += buf[t * WSTRIDE + q] * sm_f[r][t];
    const float inv = sm_inv[r];
    const int rr = row0 + r;
    float *dst;
    if (direct) {
      const int wt = tok_of(rr), h = kvh * a.group + rr - wt * a.group;
      dst = a.out + ((size_t)wt * a.n_q_heads + h) * D;
    } else {
      dst = a.part_o + (((size_t)split * a.n_kv_heads + kvh) * a.rows + rr) * D;
    }
    *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * (ln >> 4)) =
        make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
  }
}

// ------------------------------------------------------------------------------------
// lse_merge: four lanes per (worker, query head, 4 output dims); lane j of the four merges
// partials j, j+4, ... with all of its loads in flight together, and the four running
// results are combined with lane exchanges. Workgroup b serves KV head b mod n_kv_heads:
// dispatch deals workgroups to the 8 XCDs in turn, as it dealt the decode's workgroups
// (KV head fastest), so a head's partials are merged on the XCD whose L2 they were
// written through.
// The arguments that address the partials come first, as scalars of their own: the dispatch
// preloads leading kernel arguments into scalar registers (gfx950 kernel-argument
// preloading, enabled by the build), so the partials' loads go out as the waves start
// rather than one kernel-argument round trip later. Measured on MI355X (replayed steps):
// w4_16k 1.311 against 1.327 ms per step, w4_16k with 4 tokens per worker 1.710 against
// 1.728, w8_32k 0.309 against 0.311, w2_4k 0.327 against 0.323. The same preloading of the
// decode kernel's prologue arguments gained nothing on w4_16k and cost w2_4k 1.4%, so the
// decode kernel keeps taking one struct.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float *part_o, const float *part_lse,
                                                         int n_kv_heads, int rows, int n_splits, int group,
                                                         MergeArgs a) {
  constexpr int Q4 = D / 4;
  constexpr int B = 8;   // partials per lane whose loads are in flight together
  const int kvh = blockIdx.x % n_kv_heads;
  const int item = (blockIdx.x / n_kv_heads) * 64 + (threadIdx.x >> 2);   // in this KV head
  const int sub = threadIdx.x & 3;
  const bool live = item < rows * Q4;
  const int it = live ? item : 0;
  const int rr = it / Q4, q4 = it % Q4;        // stacked row (query token, head of the group)
  const int w = rr / group, h = kvh * group + rr % group;
  const size_t stride = (size_t)n_kv_heads * rows;
  const size_t base = (size_t)kvh * rows + rr;
  float mm = -INFINITY, tot = 0.0f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = sub; p0 < n_splits; p0 += 4 * B) {
    float lp[B];
    float4 x[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int p = p0 + 4 * i < n_splits ? p0 + 4 * i : 0;
      lp[i] = part_lse[base + p * stride];
      x[i] = reinterpret_cast<const float4 *>(part_o + (base + p * stride) * D)[q4];
    }
    // All sixteen loads go out before the first is used, and the combine below has no branch
    // on their values: otherwise the compiler issued the partials' loads only once the
    // normalisers had arrived, two round trips instead of one (w4_16k step 1.292 against
    // 1.322 ms, w2_4k 0.320 against 0.334 ms).
    __builtin_amdgcn_sched_barrier(0);
    float bm = mm;
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (p0 + 4 * i < n_splits) bm = fmaxf(bm, lp[i]);
    const bool any = bm != -INFINITY;   // else every partial so far is empty
    const float sc = any ? __builtin_amdgcn_exp2f(mm - bm) : 1.0f;
    tot *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const float wt = (any && p0 + 4 * i < n_splits) ? __builtin_amdgcn_exp2f(lp[i] - bm) : 0.0f;
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
  if (a.advance && blockIdx.x == 0 && threadIdx.x == 0) {   // the decode has read the counter
    const int v = a.advance[0];
    a.advance[0] = v < a.advance_cap ? v + 1 : v;
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
// Static scratch of hw_concurrent_decode_noalloc: the split partials of a decode, in a
// file-scope device array instead of the caller's workspace. Each GPU the library runs on
// holds one copy until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, per device.
// ------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)); }

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

hipError_t launch_advance(int32_t *counter, int32_t cap, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, counter, cap);
  return hipGetLastError();
}

hipError_t launch_plan_append(hw_dtype dt, int head_dim, const PlanAppendArgs &a, hipStream_t s) {
  dim3 grid(a.rows > 0 ? a.rows : 1), block(256);
  if (dt == HW_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((plan_append_kernel<__bf16, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((plan_append_kernel<__bf16, 64>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((plan_append_kernel<float, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((plan_append_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Launched with hipExtLaunchKernelGGL so that optional start/stop events are recorded by
// the kernel's own dispatch (null events: a plain launch). bf16 pools: up to 32 rows per
// workgroup run on 8 single-stage waves; 33..64 rows on 4 two-stage waves.
template <int D, bool MT>
static hipError_t launch_decode_bf16(int rt, const DecodeArgs &a, dim3 grid, hipStream_t s,
                                     hipEvent_t e0, hipEvent_t e1) {
  const dim3 b8(8 * 64), b4(4 * 64);
  const bool wide = !MT && a.desc_stride == kWideStride;
  if constexpr (!MT) {
    if (a.plan_step) {   // a step plan: narrow descriptors, affine in the layer's step count
      if (rt == 1) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 1, 8, 1, false, false, true>), grid, b8, 0, s, e0, e1, 0, a);
      else if (rt == 2) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 2, 8, 1, false, false, true>), grid, b8, 0, s, e0, e1, 0, a);
      else if (rt == 3) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 3, 4, 2, false, false, true>), grid, b4, 0, s, e0, e1, 0, a);
      else hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 4, 4, 2, false, false, true>), grid, b4, 0, s, e0, e1, 0, a);
      return hipSuccess;
    }
  }
  // at most about 1.5 groups for each of a workgroup's 8 waves: group 0 requested late
  const bool late = wide && a.n_groups <= 12 * a.n_splits;
  if (rt == 1 && wide && late) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 1, 8, 1, !MT, MT, false, !MT>), grid, b8, 0, s, e0, e1, 0, a);
  else if (rt == 1 && wide) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 1, 8, 1, !MT, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
  else if (rt == 1) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 1, 8, 1, false, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
  else if (rt == 2 && wide && late) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 2, 8, 1, !MT, MT, false, !MT>), grid, b8, 0, s, e0, e1, 0, a);
  else if (rt == 2 && wide) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 2, 8, 1, !MT, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
  else if (rt == 2) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 2, 8, 1, false, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
  else if constexpr (MT) return hipErrorInvalidValue;   // several tokens: blocks of <= 32 rows
  else if (rt == 3) hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 3, 4, 2, false, MT, false>), grid, b4, 0, s, e0, e1, 0, a);
  else hipExtLaunchKernelGGL((concurrent_decode_kernel<__bf16, D, 4, 4, 2, false, MT, false>), grid, b4, 0, s, e0, e1, 0, a);
  return hipSuccess;
}

template <int D, bool MT>
static void launch_decode_f32(const DecodeArgs &a, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 b8(8 * 64);
  if (!MT && a.desc_stride == kWideStride)
    hipExtLaunchKernelGGL((concurrent_decode_kernel<float, D, 1, 8, 1, !MT, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL((concurrent_decode_kernel<float, D, 1, 8, 1, false, MT, false>), grid, b8, 0, s, e0, e1, 0, a);
}

// Several query tokens per worker (n_new > 1) run the MT kernels; wide descriptors are only
// uploaded for one token.
hipError_t launch_decode(hw_dtype dt, int head_dim, const DecodeArgs &a, int row_blocks,
                         hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int rows_first = a.rows < a.rows_per_block ? a.rows : a.rows_per_block;
  const int rt = (rows_first + 15) / 16;
  dim3 grid(a.n_kv_heads, a.n_splits, row_blocks);
  const bool mt = a.n_new > 1;
  if (dt == HW_BF16) {
    const hipError_t e = head_dim == 128
                             ? (mt ? launch_decode_bf16<128, true>(rt, a, grid, s, ev_start, ev_stop)
                                   : launch_decode_bf16<128, false>(rt, a, grid, s, ev_start, ev_stop))
                             : (mt ? launch_decode_bf16<64, true>(rt, a, grid, s, ev_start, ev_stop)
                                   : launch_decode_bf16<64, false>(rt, a, grid, s, ev_start, ev_stop));
    if (e != hipSuccess) return e;
  } else {   // fp32 pools: one 16-row tile per workgroup
    if (head_dim == 128) mt ? launch_decode_f32<128, true>(a, grid, s, ev_start, ev_stop)
                            : launch_decode_f32<128, false>(a, grid, s, ev_start, ev_stop);
    else mt ? launch_decode_f32<64, true>(a, grid, s, ev_start, ev_stop)
            : launch_decode_f32<64, false>(a, grid, s, ev_start, ev_stop);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// stream_read: the streaming-read ceiling. Workgroup g reads 16-byte units [b, e) of the
// buffer, b = n16 * g / G, e = n16 * (g + 1) / G, four loads in flight per thread.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *p, size_t n16, float *sink) {
  const size_t b = n16 * blockIdx.x / gridDim.x, e = n16 * (blockIdx.x + 1) / gridDim.x;
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
  uint32_t acc = 0;
  size_t i = b + threadIdx.x;
  for (; i + 768 < e; i += 1024) {
    const u32x4 x0 = __builtin_nontemporal_load(q + i), x1 = __builtin_nontemporal_load(q + i + 256);
    const u32x4 x2 = __builtin_nontemporal_load(q + i + 512), x3 = __builtin_nontemporal_load(q + i + 768);
    acc ^= x0.x ^ x1.y ^ x2.z ^ x3.w;
  }
  for (; i < e; i += 256) acc ^= __builtin_nontemporal_load(q + i).x;
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = 1.0f;
}

hipError_t launch_stream_read(const void *src, size_t bytes, float *sink, int n_blocks, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
  hipExtLaunchKernelGGL(stream_read_kernel, dim3(n_blocks), dim3(256), 0, s, ev_start, ev_stop, 0,
                        static_cast<const uint4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const MergeArgs &a, hipStream_t s) {
  const int per_head = (a.rows * (head_dim / 4) + 63) / 64;   // workgroups of 64 items
  dim3 grid(per_head * a.n_kv_heads), block(256);
  // the partials' addressing arguments ahead of MergeArgs (preloaded at dispatch)
  if (head_dim == 128)
    hipLaunchKernelGGL((lse_merge_kernel<128>), grid, block, 0, s, a.part_o, a.part_lse, a.n_kv_heads, a.rows,
                       a.n_splits, a.group, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<64>), grid, block, 0, s, a.part_o, a.part_lse, a.n_kv_heads, a.rows,
                       a.n_splits, a.group, a);
  return hipGetLastError();
}

}  // namespace hw
