// Pieces shared by the decode kernels: dequantization of one row segment, the
// online-softmax merge factor, and the chunk epilogue (cross-wavefront merge,
// partial write, arrival counter, and the finalize run by the last work-group of
// each (request, KV head)), with the agent-scope accessors they exchange through.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LAZY = 8.0f;  // log2 headroom before a running maximum moves
constexpr int WAVES = 4;

// Spill layout of the (l~, l) pairs of one (request, KV head): per region,
// tiles of 16 tokens; inside a tile, 4 groups of 4 tokens; inside a group the
// entries are head-major, token-minor.  Entry index of (region token t, head h):
//   16 G (t / 16) + 4 G ((t % 16) / 4) + 4 h + t % 4.
// A wavefront of the matrix-core kernel writes its tile's 64 entries in lane
// order.  Each region's part is padded to whole tiles.
__device__ __forceinline__ int round16(int n) { return (n + 15) & ~15; }

__device__ __forceinline__ void tvp_add(float &acc, float lt, float le, float Mt, float iZt,
                                        float Me, float iZe) {
  acc += fabsf(fast_exp2(le - Me) * iZe - fast_exp2(lt - Mt) * iZt);
}

template <int G>
__device__ __forceinline__ size_t spill_entry(int t, int h) {
  return (size_t)(16 * G) * (t >> 4) + 4 * G * ((t & 15) >> 2) + 4 * h + (t & 3);
}

template <int G>
__device__ __forceinline__ float *spill_region(const DecodeLaunch &d, int grp, bool is_prefix) {
  const size_t rows = (size_t)round16(d.prefix_len) + round16(d.suffix_cap);
  return d.spill + ((size_t)grp * rows + (is_prefix ? 0 : round16(d.prefix_len))) * (2 * G);
}

// c (log2 units) of every spill entry, for the block report: one float per entry
template <int G>
__device__ __forceinline__ float *rspill_region(const DecodeLaunch &d, int grp, bool is_prefix) {
  const size_t rows = (size_t)round16(d.prefix_len) + round16(d.suffix_cap);
  return d.rspill + ((size_t)grp * rows + (is_prefix ? 0 : round16(d.prefix_len))) * G;
}

// Words that other work-groups read (partials, and the spill when a group
// has several chunks) go through agent-scope stores and loads, each coherent
// at device scope by itself, so no fence has to write back or invalidate a
// whole cache; a writer waits for its own stores (vmcnt 0) before it counts
// itself in.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// one (l~, l) spill pair; `dev`: read by another work-group
__device__ __forceinline__ void st_pair(float *p, float a, float b, bool dev) {
  if (dev) {
    const uint64_t w = ((uint64_t)__float_as_uint(b) << 32) | __float_as_uint(a);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
  }
}
__device__ __forceinline__ float2 ld_pair_dev(const float *p) {
  const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
}
__device__ __forceinline__ void wait_own_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float merge_factor(float m, float mnew) {
  return m == NEG_INF ? 0.0f : fast_exp2(m - mnew);
}

// Theorem 2's c_t = sm_scale sum_b ||q_b|| w_{t,b} (WitCert Sec. 4.1), in log2
// units, must not fall below its exact value for the stored witness.  The
// band factor ||q_b|| sm_scale log2(e) (band b: coordinates 4b..4b+3 and
// 64+4b..64+4b+3 of the fp32 query) is formed in fp32 against c_factor =
// sm_scale log2(e) (1 + 2^-19) rounded up: the sum of squares takes 8
// roundings of non-negative terms, the square root one more (it halves the
// sum's relative error), the product one: at most 6 units of 2^-24 below the
// raised value.  The sums c is formed with later lose at most 17 more (17
// roundings to nearest of non-negative terms); 23 < 32 = the raise, so c is
// at or above its exact value.
__device__ __forceinline__ float band_factor_up(float4 a, float4 c, float c_factor) {
#pragma clang fp contract(off)                         // (the product is rounded by itself)
  float ss = a.x * a.x;
  ss = fmaf(c.x, c.x, ss);
  ss = fmaf(a.y, a.y, ss);
  ss = fmaf(c.y, c.y, ss);
  ss = fmaf(a.z, a.z, ss);
  ss = fmaf(c.z, c.z, ss);
  ss = fmaf(a.w, a.w, ss);
  ss = fmaf(c.w, c.w, ss);
  return sqrtf(ss) * c_factor;
}
__device__ __forceinline__ float band_factor_up(const float *qp, int bb, float c_factor) {
  return band_factor_up(*reinterpret_cast<const float4 *>(qp + 4 * bb),
                        *reinterpret_cast<const float4 *>(qp + 64 + 4 * bb), c_factor);
}

// A spilled c for the block report: NaN (an overflowed witness dot whose
// band had witness 0) counts as +inf, the trivial contribution.
__device__ __forceinline__ float c_or_inf(float c) { return c == c ? c : __builtin_huge_valf(); }

// log A (WitCert Thm. 1, in nats) from the attention state (Mq, Zq) and the
// state (Mm, Zm) over l~ + c, both in log2 units.  A is evaluated in the log
// domain; when a term of its sum overflowed (c or l~ + c reached +inf, which
// leaves Mm = +inf or Zm not finite) the result is +inf, the trivial bound
// (WitCert Sec. 3 numerics, Sec. 6.2.4), never a truncated c.
__device__ __forceinline__ double meter_log_a(float Mq, float Zq, float Mm, float Zm) {
  if (!(Zq > 0.0f)) return 0.0;                     // no token: empty sums
  if (Mm == __builtin_huge_valf() || !(Zm <= 3.4028234663852886e38f)) return __builtin_huge_val();
  if (!(Zm > 0.0f)) return 0.0;
  return ((double)Mm - (double)Mq) * 0.69314718055994530942 + log((double)Zm) - log((double)Zq);
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
  } else if constexpr (F == KVQ_FMT_INT8_G32) {  // i8_scale: the row's 4 group scales
    const uint4 w = *reinterpret_cast<const uint4 *>((const uint8_t *)base + row * D + 16 * j);
    const float s = fp16_bits_to_f32(i8_scale[j >> 1]);
    const uint32_t cw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float xi[4];
      dither4(tok, (uint32_t)(4 * j + g), tag, stream, k0, k1, xi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float code = (float)(int)(int8_t)(cw[g] >> (8 * e));
        v[4 * g + e] = s * (code - xi[e]);
      }
    }
  } else {  // INT8 with subtractive dither, block scales
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

// TV shares of a 256-thread work-group whose thread t holds a partial sum of
// head (t % 2G) / 2: per head, a butterfly over the wavefront's lanes of that
// head (lane bit 0 and the bits from log2(2G) up), then the four wavefronts'
// sums in wavefront order.  Returns head tid's total in threads tid < G
// (fixed order: bitwise reproducible).  Every thread of the work-group must
// call it.
template <int G>
__device__ __forceinline__ float head_share_sum(float x, float (*tvw)[G]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  x += __shfl_xor(x, 1);
#pragma unroll
  for (int off = 2 * G; off < 64; off <<= 1) x += __shfl_xor(x, off);
  if (lane < 2 * G && (lane & 1) == 0) tvw[wv][lane >> 1] = x;
  __syncthreads();
  float s = 0.0f;
  if (tid < G) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += tvw[w][tid];
  }
  return s;
}

// Block-decomposable risk report (WitCert Sec. 6.3.5), run by the finalizing
// work-group after the normalizers are known: for every 256-token block j of
// each region (aligned at the region's start) and head h, from the spilled
// l~ and c of its tokens:
//   mass_j = sum p~_t,  excess_j = sum p~_t (e^{c_t} - 1),
//   excess_b_j = mass_j (e^{u_j} - 1) with the block's Tier B radius,
// then the blocks ranked by decreasing excess (Tier B's when requested), ties
// by lower index.  Wavefront w takes blocks w, w + 4, ...; lane l reads the
// block's entries l + 64 i, all of head (l % 4G) / 4, and the sums reduce
// over the other lane bits in a fixed order (bitwise reproducible).
template <int G>
__device__ __forceinline__ void block_report_pass(const DecodeLaunch &d, int grp, int b, int kvh, bool single, int suf_len,
                                  const float (*fin)[6]) {
  constexpr float LN2 = 0.69314718055994530942f;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ float rkey_s[G][512];
  const int hmine = (lane % (4 * G)) / 4;
  const float Mt = fin[hmine][0], iZt = fin[hmine][1];
  auto rd = [&](const float *p) { return single ? *p : ld_dev(p); };
  for (int region = 0; region < 2; ++region) {
    const int cap = region == 0 ? d.prefix_len : d.suffix_cap;
    const int n = region == 0 ? d.prefix_len : suf_len;
    const int nb = (cap + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK;
    const int gb0 = region == 0 ? 0 : d.pre_blocks;
    const bool i8 = (region == 0 ? d.pre_int8 : d.suf_int8) != 0;
    if (nb == 0) continue;
    const float *sp = spill_region<G>(d, grp, region == 0);
    const float *rp = rspill_region<G>(d, grp, region == 0);
    for (int j = wv; j < nb; j += WAVES) {         // uniform over the wavefront
      float ms = 0.0f, ex = 0.0f;
#pragma unroll 4
      for (int i = 0; i < 4 * G; ++i) {
        const int e = KVQ_INT8_BLOCK * G * j + lane + 64 * i;
        const int tile = e / (16 * G), r = e % (16 * G);
        const int t = 16 * tile + 4 * (r / (4 * G)) + (r & 3);
        if (t < n) {
          const float pt = fast_exp2(rd(sp + 2 * (size_t)e) - Mt) * iZt;
          ms += pt;
          if (pt > 0.0f) ex += pt * expm1f(c_or_inf(rd(rp + e)) * LN2);
        }
      }
      for (int off = 1; off < 64; off <<= 1) {
        if (off >= 4 && off < 4 * G) continue;     // the head bits
        ms += __shfl_xor(ms, off);
        ex += __shfl_xor(ex, off);
      }
      if (lane < 4 * G && (lane & 3) == 0) {
        const int h = lane >> 2;
        float Eb = 0.0f;
        if (d.has_tier_b && i8 && ms > 0.0f)
          Eb = ms * expm1f(rd(d.ublk + ((size_t)grp * d.n_blocks + gb0 + j) * G + h) * LN2);
        const size_t o = ((size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h) * d.n_blocks + gb0 + j;
        const bool hv = d.qh0 + h < d.qg;
        if (d.block_mass && hv) d.block_mass[o] = ms;
        if (d.block_excess && hv) d.block_excess[o] = ex;
        if (d.block_excess_b && hv) d.block_excess_b[o] = Eb;
        if (d.block_order) rkey_s[h][gb0 + j] = d.has_tier_b ? Eb : ex;
      }
    }
  }
  if (d.block_order) {                             // rank = blocks ahead of j
    __syncthreads();
    const int nbt = d.n_blocks;
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
}

// Per-wavefront states are in part_s[w][h][...] (m~, z~, m', z', m_e, z_e,
// z_b, z_v, acc[128], max ||v||, m-, z-, pad); z_b (Tier B's sum of p~ e^u),
// z_v (the value side's sum of p~ rho) and acc share m~; (m-, z-) is the
// running state over l~ - c of the two-sided form.  Merges the wavefronts into this chunk's partial.  When the group
// (b, kvh) has several chunks, the partial goes to the workspace and the
// arrival is counted; the last arrival runs the finalize over all partials.  A
// group with a single chunk finalizes from LDS directly (no cross-work-group
// traffic, fences or counters).  The finalize: exact LSE merge of every chunk
// (in chunk order) into out, log A, bound, meter, then the TV over the spilled
// logit pairs.  Called by all 256 threads.
template <int G>
__device__ __forceinline__ void chunk_epilogue(const DecodeLaunch &d, float (*part_s)[G][PART_STRIDE], int grp,
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
    if ((k == 6 && !d.has_tier_b) || (k == 7 && !d.has_value) || k > PART_CMAX ||
        (k == PART_VMAX && !d.has_value) || (k >= PART_MN && !d.has_two_sided))
      continue;
    // which maximum governs this field: its own (m~, m', m_e, m-) or m~
    const int mk = k < 6 ? (k & ~1) : ((k == PART_MN || k == PART_ZN) ? PART_MN : 0);
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, part_s[w][h][mk]);
    float r;
    if (k == PART_VMAX || k == PART_CMAX) {          // a plain maximum
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) r = fmaxf(r, part_s[w][h][k]);
    } else if ((k < 6 && (k & 1) == 0) || k == PART_MN) {
      r = M;
    } else {
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) r += part_s[w][h][k] * merge_factor(part_s[w][h][mk], M);
    }
    if (single)
      part_g[idx] = r;
    else
      st_dev(&part_g[idx], r);
  }
  // (requested before the arrival count, whose round trip hides it)
  const int suf_len = d.suffix_lengths ? min(max(d.suffix_lengths[b], 0), d.suffix_cap) : d.suffix_cap;
  if (single) {
    // spill rows and merged_s were written by this work-group only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    wait_own_stores();              // this thread's partial and spill words are out
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(d.counters + grp, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      last_s = (old == (unsigned)(total_chunks - 1));
    }
    __syncthreads();
    if (!last_s) return;
  }
  auto rd = [&](const float *p) { return single ? *p : ld_dev(p); };

  // ================= finalize: this work-group arrived last for (b, kvh)
  __shared__ float fin_s[G][6];   // M~, 1/Z~, M_e, 1/Z_e (log2 units)
  const float *pg = single ? &merged_s[0][0] : d.partials + (size_t)grp * total_chunks * G * PART_STRIDE;
  // Wavefront h merges head h.  Lane c holds the states of chunk cb + c of a
  // batch of 64, all requested at once, together with the first 8 chunks'
  // output words; maxima reduce over the lanes (exact), sums run over the
  // chunks in order through lane reads (the same arithmetic as a loop over
  // the chunks).  A finalize of up to 8 chunks takes one round trip.
  const bool two = d.has_two_sided != 0, val = d.has_value != 0, tb = d.has_tier_b != 0;
  const int nc = total_chunks;
  auto lane_f = [](float x, int i) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i)); };
  for (int h = wv; h < G; h += WAVES) {
    struct St {
      float m0, z1, m2, z3, m4, z5, zb, zv, vmax, mn, zn, cmax;
    };
    auto load_st = [&](int c) {                     // chunk c's states (NEG_INF / 0: no chunk)
      St x{NEG_INF, 0.0f, NEG_INF, 0.0f, NEG_INF, 0.0f, 0.0f, 0.0f, 0.0f, NEG_INF, 0.0f, 0.0f};
      if (c < nc) {
        const float *pc = pg + ((size_t)c * G + h) * PART_STRIDE;
        x.m0 = rd(pc + 0); x.z1 = rd(pc + 1); x.m2 = rd(pc + 2); x.z3 = rd(pc + 3);
        x.m4 = rd(pc + 4); x.z5 = rd(pc + 5);
        if (tb) x.zb = rd(pc + 6);
        if (val) { x.zv = rd(pc + 7); x.vmax = rd(pc + PART_VMAX); }
        if (two) { x.mn = rd(pc + PART_MN); x.zn = rd(pc + PART_ZN); x.cmax = rd(pc + PART_CMAX); }
      }
      return x;
    };
    const St st0 = load_st(lane);
    float a0[8], a1[8];                             // output words of chunks 0..7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a0[j] = a1[j] = 0.0f;
      if (j < nc) {
        const float *pc = pg + ((size_t)j * G + h) * PART_STRIDE;
        a0[j] = rd(pc + 8 + lane);
        a1[j] = rd(pc + 8 + 64 + lane);
      }
    }
    float Mq = st0.m0, Mm = st0.m2, Me = st0.m4, Mn = st0.mn;
    for (int cb = 64; cb < nc; cb += 64) {          // more than 64 chunks
      const St x = load_st(cb + lane);
      Mq = fmaxf(Mq, x.m0); Mm = fmaxf(Mm, x.m2); Me = fmaxf(Me, x.m4); Mn = fmaxf(Mn, x.mn);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      Mq = fmaxf(Mq, __shfl_xor(Mq, off));
      Mm = fmaxf(Mm, __shfl_xor(Mm, off));
      Me = fmaxf(Me, __shfl_xor(Me, off));
      if (two) Mn = fmaxf(Mn, __shfl_xor(Mn, off));
    }
    float Zn = 0.0f, Cmax = 0.0f;
    float Zq = 0.0f, Zm = 0.0f, Ze = 0.0f, Zb = 0.0f, Zv = 0.0f, Vmax = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int cb = 0; cb < nc; cb += 64) {
      const St x = cb == 0 ? st0 : load_st(cb + lane);
      // this lane's chunk: its merge factors on the group's maxima; the sums
      // take each chunk's term as one fused multiply-add, in chunk order
      const float fq = merge_factor(x.m0, Mq), fm = merge_factor(x.m2, Mm), fe = merge_factor(x.m4, Me);
      const float fn = merge_factor(x.mn, Mn);
      const int n = min(64, nc - cb);
      for (int i = 0; i < n; ++i) {
        const float f = lane_f(fq, i);
        Zq = fmaf(lane_f(x.z1, i), f, Zq);
        if (tb) Zb = fmaf(lane_f(x.zb, i), f, Zb);
        if (val) {
          Zv = fmaf(lane_f(x.zv, i), f, Zv);
          Vmax = fmaxf(Vmax, lane_f(x.vmax, i));
        }
        if (two) {
          Zn = fmaf(lane_f(x.zn, i), lane_f(fn, i), Zn);
          Cmax = fmaxf(Cmax, lane_f(x.cmax, i));
        }
        Zm = fmaf(lane_f(x.z3, i), lane_f(fm, i), Zm);
        Ze = fmaf(lane_f(x.z5, i), lane_f(fe, i), Ze);
      }
      // outputs: 8 chunks' words in flight at a time (the first 8 are loaded)
      for (int i0 = 0; i0 < n; i0 += 8) {
        if (cb + i0 >= 8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            a0[j] = a1[j] = 0.0f;
            if (i0 + j < n) {
              const float *pc = pg + ((size_t)(cb + i0 + j) * G + h) * PART_STRIDE;
              a0[j] = rd(pc + 8 + lane);
              a1[j] = rd(pc + 8 + 64 + lane);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (i0 + j < n) {
            const float f = lane_f(fq, i0 + j);
            o0 = fmaf(a0[j], f, o0);
            o1 = fmaf(a1[j], f, o1);
          }
        }
      }
    }
    const size_t qh = (size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + h;
    const bool hv = d.qh0 + h < d.qg;               // a query head (not a padding head)
    if (d.has_out && hv) {
      const float inv = Zq > 0.0f ? 1.0f / Zq : 0.0f;
      d.out[qh * D + lane] = o0 * inv;
      d.out[qh * D + 64 + lane] = o1 * inv;
    }
    if (lane == 0) {
      const double log_a = do_meter ? meter_log_a(Mq, Zq, Mm, Zm) : 0.0;
      const double bound = log_a == 0.0 ? 0.0 : 0.5 * expm1(2.0 * log_a);   // (no witness: 0)
      const float bf = bound > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)bound;
      if (d.log_a && hv) d.log_a[qh] = (float)log_a;
      if (d.bound_raw && hv) d.bound_raw[qh] = bf;
      if (d.meter && hv) d.meter[qh] = fminf(1.0f, bf);
      if (d.log_a_minus || d.bound_two_sided || d.meter_two_sided || d.bound_tanh) {
        // two-sided form (WitCert Prop. 1): 1/2 (A/A- - A-/A) = sinh(log A - log A-)
        double log_am = 0.0;
        if (d.has_two_sided && Zq > 0.0f && Zn > 0.0f)
          log_am = ((double)Mn - (double)Mq) * 0.69314718055994530942 + log((double)Zn) - log((double)Zq);
        const double two = sinh(log_a - log_am);
        const float tf = two > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)two;
        if (d.log_a_minus && hv) d.log_a_minus[qh] = (float)log_am;
        if (d.bound_two_sided && hv) d.bound_two_sided[qh] = tf;
        if (d.meter_two_sided && hv) d.meter_two_sided[qh] = fminf(fminf(1.0f, bf), tf);
        // tanh shape: tanh(max_t c_t), c in natural units
        // (a meter sum that overflowed, log A = +inf, had a c of +inf or NaN,
        // which a maximum skips: the trivial bound then, as for log A)
        if (d.bound_tanh && hv)
          d.bound_tanh[qh] = log_a == __builtin_huge_val() ? 1.0f : (float)tanh((double)Cmax * 0.69314718055994530942);
      }
      if (d.has_value) {
        // value side and the joint output bound (WitCert Sec. 3): the meter
        // bounds TV (0 when every region's keys are stored exactly)
        const float verr = Zq > 0.0f ? Zv / Zq : 0.0f;
        const float tvb = do_meter ? fminf(1.0f, bf) : 0.0f;
        if (d.value_err && hv) d.value_err[qh] = verr;
        if (d.v_norm_max && hv) d.v_norm_max[qh] = Vmax;
        if (d.out_bound && hv) d.out_bound[qh] = 2.0f * tvb * Vmax + verr;
      }
      if (d.has_tier_b) {
        // log A_B = log(sum p~ e^u / sum p~), both sums on the maximum M~
        const double log_ab = (Zq > 0.0f && Zb > 0.0f) ? log((double)Zb) - log((double)Zq) : 0.0;
        const double bb = 0.5 * expm1(2.0 * log_ab);
        const float bbf = bb > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)bb;
        if (d.log_a_b && hv) d.log_a_b[qh] = (float)log_ab;
        if (d.bound_b_raw && hv) d.bound_b_raw[qh] = bbf;
        if (d.meter_b && hv) d.meter_b[qh] = fminf(1.0f, bbf);
      }
      fin_s[h][0] = Mq;
      fin_s[h][1] = Zq > 0.0f ? 1.0f / Zq : 0.0f;
      fin_s[h][2] = Me;
      fin_s[h][3] = Ze > 0.0f ? 1.0f / Ze : 0.0f;
    }
  }
  __syncthreads();
  if (d.defer_tv) {
    // the TV and the block report run in the finish launch, spread over many
    // work-groups: publish this group's normalizers for it
    if (tid < 4 * G) d.fin[(size_t)grp * 4 * G + tid] = fin_s[tid >> 2][tid & 3];
    if (tid == 0) __hip_atomic_store(d.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (d.tv && !do_tv) {
    // no region holds exact keys: the stored keys are exact, TV = 0
    if (tid < G && d.qh0 + tid < d.qg) d.tv[(size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + tid] = 0.0f;
  } else if (d.tv) {
    // Thread tid reads entries 2 tid + 512 k (a float4: two entries of one
    // head); 512 is a multiple of 4G, so the head of its entries never changes.
    // (a group with several chunks runs this pass in the finish launch
    // instead, spread over many work-groups)
    constexpr int TV_U = 4;
    __shared__ float tvw_s[WAVES][G];
    const int hmine = ((2 * tid) % (4 * G)) / 4;
    float acc_tv = 0.0f;
    if (do_tv) {
      const float Mt = fin_s[hmine][0], iZt = fin_s[hmine][1];
      const float Me = fin_s[hmine][2], iZe = fin_s[hmine][3];
#pragma unroll
      for (int region = 0; region < 2; ++region) {
        const int n = region == 0 ? d.prefix_len : suf_len;
        if (n == 0) continue;
        const float *sp = spill_region<G>(d, grp, region == 0);
        const int n_entries = round16(n) * G;
        for (int e0 = 2 * tid; e0 < n_entries; e0 += TV_U * 512) {
          float4 x[TV_U];
#pragma unroll
          for (int u = 0; u < TV_U; ++u) {
            const int e = min(e0 + 512 * u, n_entries - 2);
            if (single) {
              x[u] = *reinterpret_cast<const float4 *>(sp + 2 * (size_t)e);
            } else {
              const float2 a = ld_pair_dev(sp + 2 * (size_t)e), c = ld_pair_dev(sp + 2 * (size_t)e + 2);
              x[u] = make_float4(a.x, a.y, c.x, c.y);
            }
          }
#pragma unroll
          for (int u = 0; u < TV_U; ++u) {
            const int e = e0 + 512 * u;
            if (e >= n_entries) break;
            // entries e and e + 1: tokens of the same head
            const int tile = e / (16 * G), r = e % (16 * G);
            const int t = 16 * tile + 4 * (r / (4 * G)) + (r & 3);
            if (t < n) tvp_add(acc_tv, x[u].x, x[u].y, Mt, iZt, Me, iZe);
            if (t + 1 < n) tvp_add(acc_tv, x[u].z, x[u].w, Mt, iZt, Me, iZe);
          }
        }
      }
    }
    const float s = head_share_sum<G>(acc_tv, tvw_s);
    if (tid < G && d.qh0 + tid < d.qg) d.tv[(size_t)b * d.h_q + (size_t)kvh * d.qg + d.qh0 + tid] = 0.5f * s;
  }
  if (d.has_report) block_report_pass<G>(d, grp, b, kvh, single, suf_len, fin_s);
  if (tid == 0 && !single)                          // ready for the next call
    __hip_atomic_store(d.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq
