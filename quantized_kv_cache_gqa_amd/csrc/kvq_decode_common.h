// Pieces shared by the decode kernels: dequantization of one row segment, the
// online-softmax merge factor, and the chunk epilogue (cross-wavefront merge,
// partial write, arrival counter, and the finalize run by the last work-group of
// each (request, KV head)).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LAZY = 8.0f;  // log2 headroom before a running maximum moves
constexpr int WAVES = 4;

__device__ __forceinline__ float merge_factor(float m, float mnew) {
  return m == NEG_INF ? 0.0f : fast_exp2(m - mnew);
}

// Dequantize the 16 values (dims 16j..16j+15) of one stored row.
// FP8: returns the E4M3 values (the per-token scale is applied by the caller).
// INT8: s_c (code - xi) with the block scales and the regenerated dither.
template <int F>
__device__ __forceinline__ void load_row16(const void *base, size_t row, int j, float *v,
                                           const uint16_t *i8_scale, uint32_t tok,
                                           uint32_t tag, uint32_t stream, uint32_t k0,
                                           uint32_t k1) {
  if constexpr (F == KVQ_FMT_FP8_E4M3) {
    const uint4 w = *reinterpret_cast<const uint4 *>((const uint8_t *)base + row * D + 16 * j);
    e4m3x4(w.x, v + 0);
    e4m3x4(w.y, v + 4);
    e4m3x4(w.z, v + 8);
    e4m3x4(w.w, v + 12);
  } else if constexpr (F == KVQ_FMT_BF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>((const uint8_t *)base + row * (2 * D) + 32 * j);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {  // INT8 with subtractive dither
    const uint4 w = *reinterpret_cast<const uint4 *>((const uint8_t *)base + row * D + 16 * j);
    const uint4 *sp = reinterpret_cast<const uint4 *>(i8_scale + 16 * j);
    const uint4 sa = sp[0], sb = sp[1];
    const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    const uint32_t cw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float xi[4];
      dither4(tok, (uint32_t)(4 * j + g), tag, stream, k0, k1, xi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        const float code = (float)(int)(int8_t)(cw[g] >> (8 * e));
        const float s = fp16_bits_to_f32((sw[i >> 1] >> (16 * (i & 1))) & 0xffffu);
        v[i] = s * (code - xi[e]);
      }
    }
  }
}

// Per-wavefront states are in part_s[w][h][...] (m~, z~, m', z', m_e, z_e, -, -,
// acc[128]).  Merges the wavefronts into this chunk's partial.  When the group
// (b, kvh) has several chunks, the partial goes to the workspace and the
// arrival is counted; the last arrival runs the finalize over all partials.  A
// group with a single chunk finalizes from LDS directly (no cross-work-group
// traffic, fences or counters).  The finalize: exact LSE merge of every chunk
// (in chunk order) into out, log A, bound, meter, then the TV over the spilled
// logit pairs.  Called by all 256 threads.
template <int G>
__device__ void chunk_epilogue(const DecodeLaunch &d, float (*part_s)[G][PART_STRIDE], int grp,
                               int chunk_idx, int b, int kvh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const bool do_tv = d.has_tv != 0;
  const bool do_meter = d.has_meter != 0;
  __shared__ int last_s;
  __shared__ float merged_s[G][PART_STRIDE];
  __syncthreads();
  const int total_chunks = d.total_chunks;
  const bool single = total_chunks == 1;
  float *part_g = single ? &merged_s[0][0]
                         : d.partials + ((size_t)grp * total_chunks + d.chunk_base + chunk_idx) * G * PART_STRIDE;
  for (int idx = tid; idx < G * PART_STRIDE; idx += 256) {
    const int h = idx / PART_STRIDE, k = idx - h * PART_STRIDE;
    if (k == 6 || k == 7) continue;
    const int mk = (k >= 8) ? 0 : (k & ~1);          // which maximum governs this field
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, part_s[w][h][mk]);
    float r;
    if (k < 6 && (k & 1) == 0) {
      r = M;
    } else {
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) r += part_s[w][h][k] * merge_factor(part_s[w][h][mk], M);
    }
    part_g[idx] = r;
  }
  if (single) {
    // spill rows and merged_s were written by this work-group only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = atomicAdd(d.counters + grp, 1u);
      last_s = (old == (unsigned)(total_chunks - 1));
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
  }

  // ================= finalize: this work-group arrived last for (b, kvh)
  __shared__ float fin_s[G][6];   // M~, 1/Z~, M_e, 1/Z_e (log2 units)
  __shared__ float tv_s[WAVES][G];
  const float *pg = single ? &merged_s[0][0] : d.partials + (size_t)grp * total_chunks * G * PART_STRIDE;
  const int suf_len = d.suffix_lengths ? min(max(d.suffix_lengths[b], 0), d.suffix_cap) : d.suffix_cap;
  const int S = d.prefix_len + suf_len;
  for (int h = wv; h < G; h += WAVES) {
    float Mq = NEG_INF, Mm = NEG_INF, Me = NEG_INF;
    for (int c = 0; c < total_chunks; ++c) {
      const float *pc = pg + ((size_t)c * G + h) * PART_STRIDE;
      Mq = fmaxf(Mq, pc[0]);
      Mm = fmaxf(Mm, pc[2]);
      Me = fmaxf(Me, pc[4]);
    }
    float Zq = 0.0f, Zm = 0.0f, Ze = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c = 0; c < total_chunks; ++c) {
      const float *pc = pg + ((size_t)c * G + h) * PART_STRIDE;
      const float fq = merge_factor(pc[0], Mq);
      Zq += pc[1] * fq;
      Zm += pc[3] * merge_factor(pc[2], Mm);
      Ze += pc[5] * merge_factor(pc[4], Me);
      o0 += pc[8 + lane] * fq;
      o1 += pc[8 + 64 + lane] * fq;
    }
    const size_t qh = (size_t)b * d.h_q + (size_t)kvh * G + h;
    if (d.has_out) {
      const float inv = Zq > 0.0f ? 1.0f / Zq : 0.0f;
      d.out[qh * D + lane] = o0 * inv;
      d.out[qh * D + 64 + lane] = o1 * inv;
    }
    if (lane == 0) {
      double log_a = 0.0;
      if (do_meter && Zq > 0.0f && Zm > 0.0f)
        log_a = ((double)Mm - (double)Mq) * 0.69314718055994530942 + log((double)Zm) - log((double)Zq);
      double bound = 0.5 * expm1(2.0 * log_a);
      const float bf = bound > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)bound;
      if (d.log_a) d.log_a[qh] = (float)log_a;
      if (d.bound_raw) d.bound_raw[qh] = bf;
      if (d.meter) d.meter[qh] = fminf(1.0f, bf);
      fin_s[h][0] = Mq;
      fin_s[h][1] = Zq > 0.0f ? 1.0f / Zq : 0.0f;
      fin_s[h][2] = Me;
      fin_s[h][3] = Ze > 0.0f ? 1.0f / Ze : 0.0f;
    }
  }
  __syncthreads();
  if (d.tv) {
    float tvp[G];
#pragma unroll
    for (int h = 0; h < G; ++h) tvp[h] = 0.0f;
    if (do_tv) {
      const float *sp = d.spill + (size_t)grp * (d.prefix_len + d.suffix_cap) * (2 * G);
      for (int t = tid; t < S; t += 256) {
        const float *r = sp + (size_t)t * (2 * G);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pt = fast_exp2(r[2 * h] - fin_s[h][0]) * fin_s[h][1];
          const float pe = fast_exp2(r[2 * h + 1] - fin_s[h][2]) * fin_s[h][3];
          tvp[h] += fabsf(pe - pt);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float s = wave_sum(tvp[h]);
      if (lane == 0) tv_s[wv][h] = s;
    }
    __syncthreads();
    if (tid < G) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += tv_s[w][tid];
      d.tv[(size_t)b * d.h_q + (size_t)kvh * G + tid] = 0.5f * s;
    }
  }
  if (tid == 0 && !single) d.counters[grp] = 0u;   // ready for the next call
}

}  // namespace kvq
