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

__device__ __forceinline__ float wave_max_across_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_across_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <typename KV, int D, int RT>
__global__ __launch_bounds__(256, 1) void concurrent_decode_kernel(DecodeArgs a) {
  using F = Frag<KV, D>;
  constexpr int NC = F::NC, NDT = F::NDT;
  constexpr int QSTRIDE = D + 4;                   // padded q row (LDS bank spread)
  constexpr int Q_FLOATS = RT * 16 * QSTRIDE;
  constexpr int BUF_F4 = RT * NDT * 64;            // one wave's O^T in lane layout
  constexpr int M_FLOATS = 2 * BUF_F4 * 4;
  constexpr int SMEM = Q_FLOATS > M_FLOATS ? Q_FLOATS : M_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM];
  __shared__ float sm_m[kWaves][64];
  __shared__ float sm_l[kWaves][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int row0 = blockIdx.z * kRowsPerBlock;
  const int nrows = min(kRowsPerBlock, a.rows - row0);

  // Stage this workgroup's raw query rows, pre-scaled by softmax_scale * log2(e).
  for (int i = tid; i < RT * 16 * D; i += 256) {
    const int r = i / D, d = i % D;
    float val = 0.0f;
    if (r < nrows) {
      const int rr = row0 + r;
      const int w = rr / a.group, gq = rr % a.group;
      val = a.q[((size_t)w * a.n_q_heads + kvh * a.group + gq) * D + d] * a.q_scale;
    }
    smem[r * QSTRIDE + d] = val;
  }
  __syncthreads();

  const long long begin = (long long)split * a.n_groups / a.n_splits;
  const long long end = (long long)(split + 1) * a.n_groups / a.n_splits;
  const KV *kl = static_cast<const KV *>(a.k_layer);
  const KV *vl = static_cast<const KV *>(a.v_layer);
  const size_t head_groups = (size_t)kvh * a.page_groups;

  f32x4 o[RT][NDT];
  float m[RT], l[RT];
  typename F::QOp qop[RT][NC];
  bool rowvis[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
    rowvis[rt] = false;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[rt][c] = F::zero_q();
  }
  int cur_seg = -1;

  long long gi = begin + wave;
  F cur, nxt;
  int2 dcur = make_int2(0, 0), dnxt = make_int2(0, 0);
  if (gi < end) {
    dcur = a.groups[gi];
    const size_t gb = ((size_t)dcur.x + head_groups) * (size_t)(32 * D);
    cur.load(kl + gb, vl + gb, lane);
  }
  for (; gi < end; gi += kWaves) {
    // Prefetch the wave's next group while this one is computed.
    const long long gn = gi + kWaves;
    if (gn < end) {
      dnxt = a.groups[gn];
      const size_t gb = ((size_t)dnxt.x + head_groups) * (size_t)(32 * D);
      nxt.load(kl + gb, vl + gb, lane);
    }
    const int seg = dcur.y >> 8;
    const int nvalid = dcur.y & 255;

    // Entering a new block: rotate each row's query by q_pos(w) - offset(w, block).
    if (seg != cur_seg) {
      cur_seg = seg;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + col;
        int dl = -1;
        if (r < nrows) dl = a.delta[(size_t)seg * a.n_workers + (row0 + r) / a.group];
        rowvis[rt] = dl >= 0;
        const float *qrow = smem + r * QSTRIDE;
        const float2 *tr = a.trig + (size_t)(dl < 0 ? 0 : dl) * (D / 2);
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
          const int j0 = 32 * c + 8 * grp;
          float lo[8], hi[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 cs = tr[j0 + e];
            const float x0 = qrow[j0 + e], x1 = qrow[D / 2 + j0 + e];
            lo[e] = x0 * cs.x - x1 * cs.y;
            hi[e] = x1 * cs.x + x0 * cs.y;
          }
          if (rowvis[rt]) {
            qop[rt][c] = F::make_q(lo);
            qop[rt][c + NC / 2] = F::make_q(hi);
          } else {
            qop[rt][c] = F::zero_q();
            qop[rt][c + NC / 2] = F::zero_q();
          }
        }
      }
    }

    // Scores of the 32 tokens for every row: lane (row col, group grp) gets tokens
    // 8*grp + 4*hh + r of row rt*16 + col in s[rt][hh][r].
    f32x4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) acc = cur.score(c, hh, qop[rt][c], acc);
        s[rt][hh] = acc;
      }

    // Online softmax (log2 domain), one row per lane, 8 tokens per lane.
    typename F::POp pop[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float v8[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = 8 * grp + e;
        const float x = s[rt][e >> 2][e & 3];
        v8[e] = (rowvis[rt] && u < nvalid) ? x : -INFINITY;
        mx = fmaxf(mx, v8[e]);
      }
      mx = wave_max_across_groups(mx);
      const float mnew = fmaxf(m[rt], mx);
      const float msafe = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m[rt] - msafe);
      float p[8], sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(v8[e] - msafe);
        sum += p[e];
      }
      l[rt] = l[rt] * alpha + sum;
      m[rt] = mnew;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
      pop[rt] = F::make_p(p);
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = cur.pv(dt, pop[rt], o[rt][dt]);

    cur = nxt;
    dcur = dnxt;
  }

  // ---- combine the four waves (fixed order: (w0 + w2) + (w1 + w3)) ----
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
  float mrow[RT], lrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][r]);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][r];
      ll += mw == -INFINITY ? 0.0f : sm_l[w][r] * __builtin_amdgcn_exp2f(mw - mm);
    }
    mrow[rt] = mm;
    lrow[rt] = ll;
    const float fac = m[rt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[rt] - mm);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= fac;
  }
  f32x4 *buf = reinterpret_cast<f32x4 *>(smem);
  if (wave >= 2) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        buf[(wave - 2) * BUF_F4 + (rt * NDT + dt) * 64 + lane] = o[rt][dt];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        o[rt][dt] += buf[wave * BUF_F4 + (rt * NDT + dt) * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) buf[(rt * NDT + dt) * 64 + lane] = o[rt][dt];
  }
  __syncthreads();
  if (wave != 0) return;

  const bool direct = a.n_splits == 1;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + col;
    if (r >= nrows) continue;
    const int rr = row0 + r;
    const float L = lrow[rt];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const float lse2 = L > 0.0f ? mrow[rt] + __log2f(L) : -INFINITY;
    float *dst;
    if (direct) {
      const int w = rr / a.group, h = kvh * a.group + rr % a.group;
      dst = a.out + ((size_t)w * a.n_q_heads + h) * D;
      if (grp == 0 && a.lse) a.lse[(size_t)w * a.n_q_heads + h] = lse2 * 0.69314718055994531f;
    } else {
      const size_t prow = ((size_t)split * a.n_kv_heads + kvh) * a.rows + rr;
      dst = a.part_o + prow * D;
      if (grp == 0) a.part_lse[prow] = lse2;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f32x4 x = (o[rt][dt] + buf[(rt * NDT + dt) * 64 + lane]) * inv;
      *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * grp) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
}

// ------------------------------------------------------------------------------------
// lse_merge: one wave per (worker, query head) row.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n_workers * a.n_q_heads) return;
  const int w = row / a.n_q_heads, h = row % a.n_q_heads;
  const int kvh = h / a.group;
  const int rr = w * a.group + h % a.group;
  const size_t stride = (size_t)a.n_kv_heads * a.rows;
  const size_t base = (size_t)kvh * a.rows + rr;
  float mm = -INFINITY;
  for (int p = 0; p < a.n_splits; ++p) mm = fmaxf(mm, a.part_lse[base + p * stride]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float tot = 0.0f;
  for (int p = 0; p < a.n_splits; ++p) {
    const float lp = a.part_lse[base + p * stride];
    const float wt = lp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lp - mm);
    tot += wt;
    const float *src = a.part_o + (base + p * stride) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += wt * src[lane * PER + i];
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  float *dst = a.out + ((size_t)w * a.n_q_heads + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[lane * PER + i] = acc[i] * inv;
  if (lane == 0 && a.lse)
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

template <typename KV, int D>
static void launch_decode_rt(int rt, const DecodeArgs &a, dim3 grid, hipStream_t s) {
  dim3 block(256);
  switch (rt) {
    case 1: hipLaunchKernelGGL((concurrent_decode_kernel<KV, D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((concurrent_decode_kernel<KV, D, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((concurrent_decode_kernel<KV, D, 3>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((concurrent_decode_kernel<KV, D, 4>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_decode(hw_dtype dt, int head_dim, const DecodeArgs &a, int row_blocks,
                         hipStream_t s) {
  const int rows_first = a.rows < kRowsPerBlock ? a.rows : kRowsPerBlock;
  const int rt = (rows_first + 15) / 16;
  dim3 grid(a.n_splits, a.n_kv_heads, row_blocks);
  if (dt == HW_BF16) {
    if (head_dim == 128) launch_decode_rt<__bf16, 128>(rt, a, grid, s);
    else launch_decode_rt<__bf16, 64>(rt, a, grid, s);
  } else {
    if (head_dim == 128) launch_decode_rt<float, 128>(rt, a, grid, s);
    else launch_decode_rt<float, 64>(rt, a, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const MergeArgs &a, hipStream_t s) {
  const int rows = a.n_workers * a.n_q_heads;
  dim3 grid((rows + 3) / 4), block(256);
  if (head_dim == 128) hipLaunchKernelGGL((lse_merge_kernel<128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((lse_merge_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace hw
