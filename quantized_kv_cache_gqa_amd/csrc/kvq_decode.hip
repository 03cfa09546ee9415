// Read path: single-query grouped-query attention over a quantized KV cache with
// the fused risk meter (WitCert Sec. 6: one data pass computes output and meter,
// merged across KV splits under the attention's LSE weights, Sec. 6.2.2) and
// the exact total variation between exact-key and stored-key attention (Sec. 3).
//
// Work decomposition.  One work-group (4 wavefronts) per (request, KV head,
// chunk of the region's tokens).  A wavefront walks 8 tokens per step: lane
// octet s = lane / 8 owns token base + s and lane j = lane % 8 owns dims
// 16j..16j+15 of that token, so every octet issues one 16-byte load per
// 128-byte row segment.  The G query heads of the KV head are processed
// together, so K and V bytes are read once per step for all of them.
//
// Per token and query head (all logits in log2 units: q is pre-scaled by
// sm_scale * log2 e):
//   l~ = <q, k^>  (stored keys, dequantized in registers),  l = <q, k> (exact keys)
//   c  = sum_b ||q_b|| w_b                                     (Theorem 2)
// Three online log-sum-exp accumulators run side by side: (m~, z~, acc) over l~
// (attention output), (m', z') over l~ + c (Theorem 1's A, log domain), and
// (m_e, z_e) over l (exact normalizer for the TV).  A running maximum is only
// moved when a logit exceeds it by more than 8 (weights stay below 2^8), which
// keeps the rescale of the 16G accumulators off the common path.
//
// The TV needs both global normalizers before any term can be summed, so each
// (l, l~) pair is written to a spill buffer; the last work-group to finish a
// (request, KV head) merges all chunk partials (exactly, in chunk order), then
// sums 1/2 |p - p~| over the spill and writes out, tv, log A, bound and meter.
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

template <int G, int KF, int VF>
__global__ __launch_bounds__(256, 2) void decode_kernel(const DecodeLaunch d) {
  const RegionDev &R = d.region;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int slot = lane >> 3, j = lane & 7;

  // XCD-aware order: consecutive logical blocks (the chunks of one group) run
  // on the same XCD, which shares one L2.
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const unsigned n_work = (unsigned)d.batch * d.h_kv * d.n_chunks;
  if (L >= n_work) return;
  const int chunk_idx = (int)(L % (unsigned)d.n_chunks);
  const int grp = (int)(L / (unsigned)d.n_chunks);
  const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;

  const int len = R.is_prefix ? R.length : (R.lengths ? min(max(R.lengths[b], 0), R.length) : R.length);
  const int c0 = chunk_idx * d.chunk;
  const int c1 = min(c0 + d.chunk, len);

  const bool do_tv = d.has_tv != 0;
  const bool do_meter = d.has_meter != 0;
  const bool has_exact = R.exact_fmt != EX_NONE;
  const bool has_wit = R.witness != nullptr;

  // query rows of this KV head, pre-scaled into log2 units
  const float qs = d.sm_scale * LOG2E;
  float qv[G][16];
  float qn[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float *qp = d.q + ((size_t)b * d.h_q + (size_t)kvh * G + h) * D;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float4 t = *reinterpret_cast<const float4 *>(qp + 16 * j + i);
      qv[h][i] = t.x * qs;
      qv[h][i + 1] = t.y * qs;
      qv[h][i + 2] = t.z * qs;
      qv[h][i + 3] = t.w * qs;
    }
    // band norms of bands 2j and 2j+1 (coordinates 4b..4b+3 and 64+4b..64+4b+3)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int bb = 2 * j + e;
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = qp[4 * bb + i], c = qp[64 + 4 * bb + i];
        ss += a * a + c * c;
      }
      qn[h][e] = sqrtf(ss) * qs;
    }
  }

  float mq[G], zq[G], mm[G], zm[G], me[G], ze[G];
  float acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mq[h] = mm[h] = me[h] = NEG_INF;
    zq[h] = zm[h] = ze[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;
  }

  // region addressing
  const size_t sh = R.is_prefix ? (size_t)kvh : (size_t)b * d.h_kv + kvh;
  const size_t dense_row0 = sh * (size_t)R.length;
  const int32_t *ptab = R.paged ? R.page_table + (size_t)b * R.max_pages : nullptr;
  const uint32_t stream = (uint32_t)(R.is_prefix ? R.stream_id
                                                 : (R.stream_ids ? R.stream_ids[b] : R.stream_id + b));
  const uint32_t ktag = dither_tag(0, R.layer, kvh), vtag = dither_tag(1, R.layer, kvh);
  const int nblk_cap = (R.length + BLK - 1) / BLK;
  float *spill_g = d.spill + ((size_t)grp * (d.prefix_len + d.suffix_cap) +
                              (R.is_prefix ? 0 : d.prefix_len)) * (2 * G);

  for (int base = c0 + wv * 8; base < c1; base += 8 * WAVES) {
    const int t = base + slot;
    const bool valid = t < c1;
    const int tc = valid ? t : c0;
    size_t row;
    if (R.paged) {
      const int pg = ptab[tc / R.page_size];
      row = ((size_t)pg * d.h_kv + kvh) * R.page_size + (tc % R.page_size);
    } else {
      row = dense_row0 + tc;
    }

    // ---- keys: stored, exact, witness
    float kv[16];
    const uint16_t *ksc8 = nullptr;
    if constexpr (KF == KVQ_FMT_INT8_DITHER)
      ksc8 = (const uint16_t *)R.k_scale + ((sh * nblk_cap + tc / BLK) * D);
    load_row16<KF>(R.k, row, j, kv, ksc8, (uint32_t)tc, ktag, stream, R.seed_lo, R.seed_hi);
    float ks = 1.0f;
    if constexpr (KF == KVQ_FMT_FP8_E4M3) ks = reinterpret_cast<const float *>(R.k_scale)[row];

    float pq[G], pe[G], pc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s = fmaf(qv[h][i], kv[i], s);
      pq[h] = s;
      pe[h] = 0.0f;
      pc[h] = 0.0f;
    }
    if (do_tv && has_exact) {
      float ke[16];
      if (R.exact_fmt == EX_BF16) {
        load_row16<KVQ_FMT_BF16>(R.k_exact, row, j, ke, nullptr, 0, 0, 0, 0, 0);
      } else {
        const float4 *p = reinterpret_cast<const float4 *>((const float *)R.k_exact + row * D + 16 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 x = p[i];
          ke[4 * i] = x.x; ke[4 * i + 1] = x.y; ke[4 * i + 2] = x.z; ke[4 * i + 3] = x.w;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s = fmaf(qv[h][i], ke[i], s);
        pe[h] = s;
      }
    }
    if (do_meter && has_wit) {
      const uint32_t w = reinterpret_cast<const uint32_t *>(R.witness + row * NB)[j];
      const float w0 = fp16_bits_to_f32(w & 0xffffu), w1 = fp16_bits_to_f32(w >> 16);
#pragma unroll
      for (int h = 0; h < G; ++h) pc[h] = fmaf(qn[h][0], w0, qn[h][1] * w1);
    }

    float lq[G], le[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lq[h] = sum8(pq[h]) * ks;
      le[h] = (do_tv && has_exact) ? sum8(pe[h]) : lq[h];
    }

    // ---- spill (l~, l) for the TV pass
    if (do_tv && valid && j == 0) {
      float *sp = spill_g + (size_t)t * (2 * G);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sp[2 * h] = lq[h];
        sp[2 * h + 1] = le[h];
      }
    }

    // ---- online accumulators
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = valid ? lq[h] : NEG_INF;
      if (x > mq[h] + LAZY) {
        const float f = merge_factor(mq[h], x);
        zq[h] *= f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] *= f;
        mq[h] = x;
      }
      p[h] = valid ? fast_exp2(x - mq[h]) : 0.0f;
      zq[h] += p[h];
    }
    if (do_meter) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float c = has_wit ? sum8(pc[h]) : 0.0f;
        const float y = valid ? lq[h] + c : NEG_INF;
        if (y > mm[h] + LAZY) {
          zm[h] *= merge_factor(mm[h], y);
          mm[h] = y;
        }
        zm[h] += valid ? fast_exp2(y - mm[h]) : 0.0f;
      }
    }
    if (do_tv) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float y = valid ? le[h] : NEG_INF;
        if (y > me[h] + LAZY) {
          ze[h] *= merge_factor(me[h], y);
          me[h] = y;
        }
        ze[h] += valid ? fast_exp2(y - me[h]) : 0.0f;
      }
    }

    // ---- values
    if constexpr (VF != VF_NONE) {
      float vv[16];
      const uint16_t *vsc8 = nullptr;
      if constexpr (VF == KVQ_FMT_INT8_DITHER)
        vsc8 = (const uint16_t *)R.v_scale + ((sh * nblk_cap + tc / BLK) * D);
      load_row16<VF>(R.v, row, j, vv, vsc8, (uint32_t)tc, vtag, stream, R.seed_lo, R.seed_hi);
      float vs = 1.0f;
      if constexpr (VF == KVQ_FMT_FP8_E4M3) vs = reinterpret_cast<const float *>(R.v_scale)[row];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = p[h] * vs;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = fmaf(w, vv[i], acc[h][i]);
      }
    }
  }

  // ---- merge the 8 token slots of the wavefront (lanes l, l^8, l^16, l^32)
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      {
        const float m2 = __shfl_xor(mq[h], off), z2 = __shfl_xor(zq[h], off);
        const float m = fmaxf(mq[h], m2);
        const float f1 = merge_factor(mq[h], m), f2 = merge_factor(m2, m);
        zq[h] = zq[h] * f1 + z2 * f2;
        if constexpr (VF != VF_NONE) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[h][i] = acc[h][i] * f1 + __shfl_xor(acc[h][i], off) * f2;
        }
        mq[h] = m;
      }
      if (do_meter) {
        const float m2 = __shfl_xor(mm[h], off), z2 = __shfl_xor(zm[h], off);
        const float m = fmaxf(mm[h], m2);
        zm[h] = zm[h] * merge_factor(mm[h], m) + z2 * merge_factor(m2, m);
        mm[h] = m;
      }
      if (do_tv) {
        const float m2 = __shfl_xor(me[h], off), z2 = __shfl_xor(ze[h], off);
        const float m = fmaxf(me[h], m2);
        ze[h] = ze[h] * merge_factor(me[h], m) + z2 * merge_factor(m2, m);
        me[h] = m;
      }
    }
  }

  // ---- merge the 4 wavefronts through LDS and write this chunk's partial
  __shared__ float part_s[WAVES][G][PART_STRIDE];
  __shared__ int last_s;
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        part_s[wv][h][0] = mq[h]; part_s[wv][h][1] = zq[h];
        part_s[wv][h][2] = mm[h]; part_s[wv][h][3] = zm[h];
        part_s[wv][h][4] = me[h]; part_s[wv][h][5] = ze[h];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) part_s[wv][h][8 + 16 * lane + i] = acc[h][i];
    }
  }
  __syncthreads();
  const int total_chunks = d.total_chunks;
  float *part_g = d.partials + ((size_t)grp * total_chunks + d.chunk_base + chunk_idx) * G * PART_STRIDE;
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
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = atomicAdd(d.counters + grp, 1u);
    last_s = (old == (unsigned)(total_chunks - 1));
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();

  // ================= finalize: this work-group arrived last for (b, kvh)
  __shared__ float fin_s[G][6];   // M~, 1/Z~, M_e, 1/Z_e (log2 units)
  __shared__ float tv_s[WAVES][G];
  const float *pg = d.partials + (size_t)grp * total_chunks * G * PART_STRIDE;
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
  if (tid == 0) d.counters[grp] = 0u;   // ready for the next call
}

// ------------------------------------------------------------------ dispatch

template <int G, int KF, int VF>
static hipError_t launch_t(const DecodeLaunch &d, hipStream_t stream) {
  const long work = (long)d.batch * d.h_kv * d.n_chunks;
  const long grid = (work + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_kernel<G, KF, VF>), dim3((unsigned)grid), dim3(256), 0, stream, d);
  return hipGetLastError();
}

template <int G, int KF>
static hipError_t launch_v(const DecodeLaunch &d, hipStream_t s) {
  switch (d.v_format) {
    case KVQ_FMT_BF16: return launch_t<G, KF, KVQ_FMT_BF16>(d, s);
    case KVQ_FMT_FP8_E4M3: return launch_t<G, KF, KVQ_FMT_FP8_E4M3>(d, s);
    case KVQ_FMT_INT8_DITHER: return launch_t<G, KF, KVQ_FMT_INT8_DITHER>(d, s);
    case VF_NONE: return launch_t<G, KF, VF_NONE>(d, s);
  }
  return hipErrorInvalidValue;
}

template <int G>
static hipError_t launch_k(const DecodeLaunch &d, hipStream_t s) {
  switch (d.k_format) {
    case KVQ_FMT_BF16: return launch_v<G, KVQ_FMT_BF16>(d, s);
    case KVQ_FMT_FP8_E4M3: return launch_v<G, KVQ_FMT_FP8_E4M3>(d, s);
    case KVQ_FMT_INT8_DITHER: return launch_v<G, KVQ_FMT_INT8_DITHER>(d, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t s) {
  switch (d.group) {
    case 1: return launch_k<1>(d, s);
    case 2: return launch_k<2>(d, s);
    case 4: return launch_k<4>(d, s);
    case 8: return launch_k<8>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
