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

#include "kvq_decode_common.h"

namespace kvq {

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
  // Tier B (WitCert Sec. 4.2): zb accumulates p~ e^{u} on the attention's
  // maximum, tb_l = log(2 S / delta) with S the request's tokens
  const bool do_b = d.has_tier_b != 0;
  float tb_l = 0.0f;
  if (do_b) {
    const int sl = d.suffix_cap > 0
                       ? (d.suffix_lengths ? min(max(d.suffix_lengths[b], 0), d.suffix_cap) : d.suffix_cap)
                       : 0;
    tb_l = logf(2.0f * (float)(d.prefix_len + sl)) + d.tier_b_log_inv_delta;
  }

  // query rows of this KV head, pre-scaled into log2 units
  const float qs = d.sm_scale * LOG2E;
  float qv[G][16];
  float qn[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float *qp = d.q + ((size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h) * D;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float4 t = *reinterpret_cast<const float4 *>(qp + 16 * j + i);
      qv[h][i] = t.x * qs;
      qv[h][i + 1] = t.y * qs;
      qv[h][i + 2] = t.z * qs;
      qv[h][i + 3] = t.w * qs;
    }
    // band norms of bands 2j and 2j+1 (coordinates 4b..4b+3 and 64+4b..64+4b+3)
    // (raised: c formed from them with 5 more roundings of non-negative
    // terms stays at or above its exact value)
#pragma unroll
    for (int e = 0; e < 2; ++e) qn[h][e] = band_factor_up(qp, 2 * j + e, d.c_factor);
  }

  // value side (WitCert Sec. 3 output bound): zv = sum p~ rho on the attention
  // maximum, vmax = the largest ||v|| of the chunk's tokens
  const bool do_v = d.has_value != 0;
  // two-sided form (WitCert Prop. 1): a running state over l~ - c for A-
  const bool do_n = d.has_two_sided != 0;
  // block report: spill (l~, l) and c of every token-head, the Tier B radius
  // of every INT8 block
  const bool do_r = d.has_report != 0;
  // fixed outlier pairs of group-scale keys (WitCert Sec. 6.2.5): byp16 marks
  // the bypassed channels among this lane's 16 (their dequantized value is
  // replaced by 0), qo holds q at the channels of outlier values 4 j .. 4 j + 3
  uint32_t byp16 = 0;
  float qo[G][4];
  const int n_op = KF == KVQ_FMT_INT8_G32 ? R.n_op : 0;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) qo[h][e] = 0.0f;
  if (n_op > 0) {
    const int32_t *opp = R.opairs + (size_t)kvh * n_op;
    for (int i = 0; i < n_op; ++i) {                     // pair P: channels P and P + 64
      const int P = opp[i];
      if (P >= 0 && P < 64 && (P >> 4) == (j & 3)) byp16 |= 1u << (P & 15);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * j + e, slot = k >> 1;
      if (k < 2 * n_op) {
        const int P = opp[slot];
        bool act = P >= 0 && P < 64;
        for (int i = 0; i < slot; ++i) act = act && opp[i] != P;
        if (act) {
#pragma unroll
          for (int h = 0; h < G; ++h)
            qo[h][e] = d.q[((size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h) * D + P + 64 * (k & 1)] * qs;
        }
      }
    }
  }

  float mq[G], zq[G], mm[G], zm[G], me[G], ze[G], zb[G], zv[G], mn[G], zn[G], cmx[G];
  float vmax = 0.0f;
  float acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mq[h] = mm[h] = me[h] = mn[h] = NEG_INF;
    zq[h] = zm[h] = ze[h] = zb[h] = zv[h] = zn[h] = cmx[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;
  }

  // region addressing
  const size_t sh = R.is_prefix ? (size_t)kvh : (size_t)b * d.h_kv + kvh;
  const size_t dense_row0 = sh * (size_t)R.length;
  const int32_t *ptab = R.paged ? R.page_table + (size_t)b * R.max_pages : nullptr;
  const uint32_t stream = (uint32_t)(R.is_prefix ? R.stream_id
                                                 : (R.stream_ids ? R.stream_ids[b] : R.stream_id + b));
  const uint32_t ktag = dither_tag(R.layer, kvh), vtag = ktag;     // (shared by keys and values)
  const int nblk_cap = (R.length + BLK - 1) / BLK;
  float *spill_g = (do_tv || do_r) ? spill_region<G>(d, grp, R.is_prefix != 0) : nullptr;
  float *rspill_g = do_r ? rspill_region<G>(d, grp, R.is_prefix != 0) : nullptr;

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
    if constexpr (KF == KVQ_FMT_INT8_G32) ksc8 = (const uint16_t *)R.k_scale + row * 4;
    load_row16<KF>(R.k, row, j, kv, ksc8, (uint32_t)tc, ktag, stream, R.seed_lo, R.seed_hi);
    if (byp16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) kv[i] = ((byp16 >> i) & 1u) ? 0.0f : kv[i];
    }
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
    if (n_op > 0) {                                      // the bypassed channels, exact
      const uint16_t *op = R.kout + row * (size_t)(2 * n_op);
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * j + e;
        ov[e] = k < 2 * n_op ? __uint_as_float((uint32_t)op[k] << 16) : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) pq[h] = fmaf(qo[h][e], ov[e], pq[h]);
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

    // ---- spill (l~, l) for the TV pass and the block report, c for the report
    if ((do_tv || do_r) && valid && j == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        st_pair(spill_g + 2 * spill_entry<G>(t, h), lq[h], le[h], d.total_chunks > 1);
    }
    if (do_r) {
      float cr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) cr[h] = (do_meter && has_wit) ? sum8(pc[h]) : 0.0f;
      if (valid && j == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float *rp = rspill_g + spill_entry<G>(t, h);
          if (d.total_chunks > 1)
            st_dev(rp, cr[h]);
          else
            *rp = cr[h];
        }
      }
    }

    // ---- Tier B radius of this token: u log2(e) = sqrt(sum_c (q_c s_c)^2 tb_l / 6)
    //      in log2 units (INT8 keys: s = the key's scale; other keys: u = 0)
    float eub[G];
#pragma unroll
    for (int h = 0; h < G; ++h) eub[h] = 1.0f;
    if constexpr (KF == KVQ_FMT_INT8_G32) {
      if (do_b) {                                        // one scale on the lane's 16 channels
        const float s = fp16_bits_to_f32(ksc8[j >> 1]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float ss = 0.0f;                               // bypassed channels: no dither
#pragma unroll
          for (int i = 0; i < 16; ++i) ss = ((byp16 >> i) & 1u) ? ss : fmaf(qv[h][i], qv[h][i], ss);
          eub[h] = exp2f(sqrtf(sum8(ss * s * s) * tb_l * (1.0f / 6.0f)));
        }
      }
    }
    if constexpr (KF == KVQ_FMT_INT8_DITHER) {
      if (do_b) {
        float sc[16];
        const uint4 *sp = reinterpret_cast<const uint4 *>(ksc8 + 16 * j);
#pragma unroll
        for (int v4 = 0; v4 < 2; ++v4) {
          const uint4 w = sp[v4];
          const uint32_t sw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) sc[8 * v4 + i] = fp16_bits_to_f32((sw[i >> 1] >> (16 * (i & 1))) & 0xffffu);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float ss = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = qv[h][i] * sc[i];
            ss = fmaf(x, x, ss);
          }
          const float ub = sqrtf(sum8(ss) * tb_l * (1.0f / 6.0f));
          eub[h] = exp2f(ub);
          // the block's radius, once per block and chunk (first token of the block here)
          if (do_r && valid && j == 0 && (t % BLK == 0 || t == c0)) {
            float *up = d.ublk + ((size_t)grp * d.n_blocks + (R.is_prefix ? 0 : d.pre_blocks) + t / BLK) * G + h;
            if (d.total_chunks > 1)
              st_dev(up, ub);
            else
              *up = ub;
          }
        }
      }
    }

    float rho = 0.0f;
    if (do_v) {
      const uint32_t vr = *reinterpret_cast<const uint32_t *>(R.v_witness + row * 2);
      rho = fp16_bits_to_f32(vr & 0xffffu);
      if (valid) vmax = fmaxf(vmax, fp16_bits_to_f32(vr >> 16));
    }

    // ---- online accumulators
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = valid ? lq[h] : NEG_INF;
      if (x > mq[h] + LAZY) {
        const float f = merge_factor(mq[h], x);
        zq[h] *= f;
        zb[h] *= f;
        zv[h] *= f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] *= f;
        mq[h] = x;
      }
      p[h] = valid ? fast_exp2(x - mq[h]) : 0.0f;
      zq[h] += p[h];
      if (do_b) zb[h] = fmaf(p[h], eub[h], zb[h]);
      if (do_v) zv[h] = fmaf(p[h], rho, zv[h]);
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
        if (do_n) {
          const float yn = valid ? lq[h] - c : NEG_INF;
          if (yn > mn[h] + LAZY) {
            zn[h] *= merge_factor(mn[h], yn);
            mn[h] = yn;
          }
          zn[h] += valid ? fast_exp2(yn - mn[h]) : 0.0f;
          if (valid) cmx[h] = fmaxf(cmx[h], c);
        }
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
      if constexpr (VF == KVQ_FMT_INT8_G32) vsc8 = (const uint16_t *)R.v_scale + row * 4;
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
        if (do_b) zb[h] = zb[h] * f1 + __shfl_xor(zb[h], off) * f2;
        if (do_v) zv[h] = zv[h] * f1 + __shfl_xor(zv[h], off) * f2;
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
      if (do_n) {
        const float m2 = __shfl_xor(mn[h], off), z2 = __shfl_xor(zn[h], off);
        const float m = fmaxf(mn[h], m2);
        zn[h] = zn[h] * merge_factor(mn[h], m) + z2 * merge_factor(m2, m);
        mn[h] = m;
        cmx[h] = fmaxf(cmx[h], __shfl_xor(cmx[h], off));
      }
      if (do_tv) {
        const float m2 = __shfl_xor(me[h], off), z2 = __shfl_xor(ze[h], off);
        const float m = fmaxf(me[h], m2);
        ze[h] = ze[h] * merge_factor(me[h], m) + z2 * merge_factor(m2, m);
        me[h] = m;
      }
    }
  }

  if (do_v) {
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }

  // ---- per-wavefront states to LDS, then the shared chunk epilogue
  __shared__ float part_s[WAVES][G][PART_STRIDE];
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        part_s[wv][h][0] = mq[h]; part_s[wv][h][1] = zq[h];
        part_s[wv][h][2] = mm[h]; part_s[wv][h][3] = zm[h];
        part_s[wv][h][4] = me[h]; part_s[wv][h][5] = ze[h];
        part_s[wv][h][6] = zb[h];
        part_s[wv][h][7] = zv[h];
        part_s[wv][h][PART_VMAX] = vmax;
        part_s[wv][h][PART_MN] = mn[h];
        part_s[wv][h][PART_ZN] = zn[h];
        part_s[wv][h][PART_CMAX] = cmx[h];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) part_s[wv][h][8 + 16 * lane + i] = acc[h][i];
    }
  }
  chunk_epilogue<G>(d, part_s, grp, chunk_idx, b, kvh);
}

// ------------------------------------------------------------- finish launch
// Deferred finalize of the per-chunk plan (several chunks per group): the
// decode launch's last work-group per group published the normalizers; here
// work-group (group, range r) takes the range's FIN_BLOCKS 256-token blocks
// (the prefix's blocks first, then the suffix's, as the block report numbers
// them), adds its tokens' TV terms and, for the report, each block's mass
// and contribution (WitCert Sec. 6.3.5).  The group's last arrival sums the
// ranges' TV partials in range order and ranks the blocks.  One work-group
// per group would stream the whole spill alone; spread this way the pass
// runs at the device's bandwidth.
template <int G>
__global__ __launch_bounds__(256) void finish_kernel(const DecodeLaunch d) {
  constexpr float LN2 = 0.69314718055994530942f;
  constexpr int NIT = (256 * G + 511) / 512;         // float4 loads per thread and block
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int groups = d.batch * d.h_kv;
  const int grp = (int)(blockIdx.x / (unsigned)d.fin_ranges);
  const int r = (int)(blockIdx.x - (unsigned)grp * d.fin_ranges);
  if (grp >= groups) return;                          // (the grid is exact)
  const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;
  const int suf_len = d.suffix_lengths ? min(max(d.suffix_lengths[b], 0), d.suffix_cap) : d.suffix_cap;
  const int pre_nb = (d.prefix_len + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK;
  __shared__ float fin_s[G][4];
  __shared__ float tvw_s[WAVES][G];
  __shared__ int last_s;
  if (tid < 4 * G) fin_s[tid >> 2][tid & 3] = d.fin[(size_t)grp * 4 * G + tid];
  __syncthreads();

  // ---- TV terms of the range's tokens: thread tid reads entries
  //      2 tid + 512 k of each block (two entries of head hmine per float4)
  // TV requested (0 where no region holds exact keys: stored keys are exact)
  const bool do_tv = d.tv != nullptr;
  if (do_tv) {
    const int hmine = ((2 * tid) % (4 * G)) / 4;
    const float Mt = fin_s[hmine][0], iZt = fin_s[hmine][1];
    const float Me = fin_s[hmine][2], iZe = fin_s[hmine][3];
    float4 x[FIN_BLOCKS][NIT];
#pragma unroll
    for (int i = 0; i < FIN_BLOCKS; ++i) {           // all loads first
      const int j = r * FIN_BLOCKS + i;
      const bool pre = j < pre_nb;
      const int jj = pre ? j : j - pre_nb;
      const int cap = pre ? d.prefix_len : d.suffix_cap;
      const float *sp = spill_region<G>(d, grp, pre);
      const int e_max = round16(cap) * G - 2;        // the region's last entry pair
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int e = min(KVQ_INT8_BLOCK * G * jj + 2 * tid + 512 * k, e_max);
        x[i][k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (d.has_tv && j < d.fin_blocks && e >= 0) x[i][k] = *reinterpret_cast<const float4 *>(sp + 2 * (size_t)e);
      }
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < FIN_BLOCKS; ++i) {
      const int j = r * FIN_BLOCKS + i;
      if (j >= d.fin_blocks || !d.has_tv) break;
      const bool pre = j < pre_nb;
      const int jj = pre ? j : j - pre_nb;
      const int n = pre ? d.prefix_len : suf_len;
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int el = 2 * tid + 512 * k;            // entry within the block
        if (el >= KVQ_INT8_BLOCK * G) break;
        const int e = KVQ_INT8_BLOCK * G * jj + el;
        const int tile = e / (16 * G), rr = e % (16 * G);
        const int t = 16 * tile + 4 * (rr / (4 * G)) + (rr & 3);
        if (t < n) tvp_add(acc, x[i][k].x, x[i][k].y, Mt, iZt, Me, iZe);
        if (t + 1 < n) tvp_add(acc, x[i][k].z, x[i][k].w, Mt, iZt, Me, iZe);
      }
    }
    const float sum = head_share_sum<G>(acc, tvw_s);
    if (tid < G) st_dev(d.tvp + ((size_t)grp * d.fin_ranges + r) * G + tid, sum);
  }

  // ---- block report: wavefront w takes block r FIN_BLOCKS + w
  if (d.has_report) {
    const int j = r * FIN_BLOCKS + wv;
    if (j < d.fin_blocks) {
      const bool pre = j < pre_nb;
      const int jj = pre ? j : j - pre_nb;
      const int cap = pre ? d.prefix_len : d.suffix_cap;
      const int n = pre ? d.prefix_len : suf_len;
      const bool i8 = (pre ? d.pre_int8 : d.suf_int8) != 0;
      const float *sp = spill_region<G>(d, grp, pre);
      const float *rp = rspill_region<G>(d, grp, pre);
      const int hmine = (lane % (4 * G)) / 4;
      const float Mt = fin_s[hmine][0], iZt = fin_s[hmine][1];
      float lt[4 * G], cr[4 * G];
#pragma unroll
      for (int i = 0; i < 4 * G; ++i) {
        const int e = min(KVQ_INT8_BLOCK * G * jj + lane + 64 * i, round16(cap) * G - 1);
        lt[i] = sp[2 * (size_t)e];
        cr[i] = rp[e];
      }
      float ms = 0.0f, ex = 0.0f;
#pragma unroll
      for (int i = 0; i < 4 * G; ++i) {
        const int e = KVQ_INT8_BLOCK * G * jj + lane + 64 * i;
        const int tile = e / (16 * G), rr = e % (16 * G);
        const int t = 16 * tile + 4 * (rr / (4 * G)) + (rr & 3);
        if (t < n) {
          const float pt = fast_exp2(lt[i] - Mt) * iZt;
          ms += pt;
          if (pt > 0.0f) ex += pt * expm1f(c_or_inf(cr[i]) * LN2);
        }
      }
      for (int off = 1; off < 64; off <<= 1) {
        if (off >= 4 && off < 4 * G) continue;       // the head bits
        ms += __shfl_xor(ms, off);
        ex += __shfl_xor(ex, off);
      }
      if (lane < 4 * G && (lane & 3) == 0) {
        const int h = lane >> 2;
        float Eb = 0.0f;
        if (d.has_tier_b && i8 && ms > 0.0f)
          Eb = ms * expm1f(d.ublk[((size_t)grp * d.n_blocks + j) * G + h] * LN2);
        const size_t o = ((size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h) * d.n_blocks + j;
        const bool hv = d.qh0 + h < d.qg;              // a query head (not a padding head)
        if (d.block_mass && hv) d.block_mass[o] = ms;
        if (d.block_excess && hv) d.block_excess[o] = ex;
        if (d.block_excess_b && hv) d.block_excess_b[o] = Eb;
        if (d.block_order) st_dev(d.rkey + ((size_t)grp * G + h) * d.n_blocks + j, d.has_tier_b ? Eb : ex);
      }
    }
  }

  // ---- the group's last arrival: TV sum in range order, block ranking
  wait_own_stores();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(d.counters + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = (old == (unsigned)(d.fin_ranges - 1));
  }
  __syncthreads();
  if (!last_s) return;
  if (do_tv && tid < G) {
    float sum = 0.0f;
    for (int q = 0; q < d.fin_ranges; ++q) sum += ld_dev(d.tvp + ((size_t)grp * d.fin_ranges + q) * G + tid);
    if (d.qh0 + tid < d.qg) d.tv[(size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + tid] = 0.5f * sum;
  }
  if (d.has_report && d.block_order) {               // rank = blocks ahead of j
    __shared__ float rkey_s[G][512];
    const int nbt = d.n_blocks;
    for (int i = tid; i < G * nbt; i += 256) rkey_s[i / nbt][i % nbt] = ld_dev(d.rkey + (size_t)grp * G * nbt + i);
    __syncthreads();
    for (int i = tid; i < G * nbt; i += 256) {
      const int h = i / nbt, j = i - h * nbt;
      const float kj = rkey_s[h][j];
      int rank = 0;
      for (int k = 0; k < nbt; ++k) {
        const float kk = rkey_s[h][k];
        rank += (kk > kj || (kk == kj && k < j)) ? 1 : 0;
      }
      if (d.qh0 + h < d.qg) d.block_order[((size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h) * nbt + rank] = j;
    }
  }
  if (tid == 0) __hip_atomic_store(d.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G>
static hipError_t launch_finish_g(const DecodeLaunch &d, hipStream_t s) {
  const long grid = (long)d.batch * d.h_kv * d.fin_ranges;
  hipLaunchKernelGGL((finish_kernel<G>), dim3((unsigned)grid), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_finish(const DecodeLaunch &d, hipStream_t s) {
  switch (d.group) {
    case 1: return launch_finish_g<1>(d, s);
    case 2: return launch_finish_g<2>(d, s);
    case 4: return launch_finish_g<4>(d, s);
    case 8: return launch_finish_g<8>(d, s);
  }
  return hipErrorInvalidValue;
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
    case KVQ_FMT_INT8_G32:                               // values in the same layout, or none
      if (d.v_format == KVQ_FMT_INT8_G32) return launch_t<G, KVQ_FMT_INT8_G32, KVQ_FMT_INT8_G32>(d, s);
      if (d.v_format == VF_NONE) return launch_t<G, KVQ_FMT_INT8_G32, VF_NONE>(d, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t s) {
  // KVQ_PLAN_VECTOR_ALU selects the vector-ALU kernel for every shape (the
  // tests run both kernels against the oracle on the same inputs)
  const bool generic = (d.plan_flags & KVQ_PLAN_VECTOR_ALU) != 0;
  if (!generic && mfma_path_supports(d)) return launch_decode_mfma(d, s);
  switch (d.group) {
    case 1: return launch_k<1>(d, s);
    case 2: return launch_k<2>(d, s);
    case 4: return launch_k<4>(d, s);
    case 8: return launch_k<8>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
