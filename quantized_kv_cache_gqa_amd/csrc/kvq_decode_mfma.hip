// Read path, matrix-core variant for GQA group 4: the per-token contractions
// of the step run on MFMA, the softmax bookkeeping on the vector ALUs.
//
// Tiles of 16 tokens per wavefront step.
//
// Logits (v_mfma_f32_16x16x32_bf16): the tile's keys are the A operand (row i =
// token i; lane l holds row l%16 and 8 consecutive k), the query is the B
// operand with 16 columns j = 4h + p: head h in {0..3}, piece p of an exact
// three-way bf16 split of the fp32 query (p = 3 is zero).  Summing the pieces
// (two quad DPP adds) gives fp32-accurate logits for the four heads.  The
// contraction over the 128 dims is permuted per lane group (lane group g reads
// dims 32g..32g+31 as one contiguous row segment) and q is permuted the same
// way.  Stored (FP8 -> bf16, exact) and exact (bf16) keys use the same B.
// Witness dot (v_mfma_f32_16x16x16_f16): fp16 witness as A, a two-piece fp16
// split of the scaled band norms as B, same column layout.
//
// After the piece sum lane 16g + 4h + p owns (token 4g + p, head h): its
// stored-key logit, exact logit and c.  One exp per lane and accumulator
// covers the tile.  The attention maximum is uniform per head (all tokens of a
// head share the output accumulator) and moves only when a logit exceeds it by
// more than 8 (log2 units).
//
// Output (FP8 values, v_mfma_f32_16x16x16_f16): A = the tile's weights
// p~ * s_v in fp16 (row = head, k = token), B = the values in fp16 (exact for
// E4M3).  Column j of N-tile n stands for dim 8j + n, so lane l loads bytes
// 8j..8j+7 of four token rows (a contiguous 512-byte span per load across the
// wavefront) and a byte transpose in registers (v_perm) forms, for each n, the
// four tokens' bytes of dim 8j + n.  The 8 N-tiles accumulate the whole output
// of the four heads (lanes 0..15 hold it).  BF16 values use vector-ALU FMAs.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_decode_common.h"

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_round(float x) {
  return __uint_as_float(f32_to_bf16_bits(x) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// 8 E4M3 codes (two dwords) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// 4 E4M3 codes (one dword) -> 4 fp16, exact.
__device__ __forceinline__ f16x4_t fp8x4_to_f16(uint32_t w) {
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return f16x4_t{a[0], a[1], b[0], b[1]};
}

// Sum of the 4 lanes of a quad (every lane gets the same bits), then lane p
// keeps register p: the value of (token 4g + p, head h).
__device__ __forceinline__ float collapse(f32x4_t x, int p) {
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = x[i] + dpp<DPP_QUAD_XOR1>(x[i]);
    r[i] = t + dpp<DPP_QUAD_XOR2>(t);
  }
  const float a01 = (p & 1) ? r[1] : r[0];
  const float a23 = (p & 1) ? r[3] : r[2];
  return (p & 2) ? a23 : a01;
}

// Byte transpose: t[e] = dword of token e (4 dims); out[n] = byte n of the four
// tokens, token e in byte e.
__device__ __forceinline__ void transpose4x4(const uint32_t t[4], uint32_t out[4]) {
  const uint32_t a01 = __builtin_amdgcn_perm(t[1], t[0], 0x05010400u);  // t0b0 t1b0 t0b1 t1b1
  const uint32_t a23 = __builtin_amdgcn_perm(t[1], t[0], 0x07030602u);  // t0b2 t1b2 t0b3 t1b3
  const uint32_t b01 = __builtin_amdgcn_perm(t[3], t[2], 0x05010400u);
  const uint32_t b23 = __builtin_amdgcn_perm(t[3], t[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(b01, a01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(b01, a01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(b23, a23, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(b23, a23, 0x07060302u);
}

// Two signed INT8 codes -> two bf16 (exact: |code| <= 127), packed.
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int byte0) {
  const float a = (float)(int)(int8_t)(w >> (8 * byte0));
  const float b = (float)(int)(int8_t)(w >> (8 * byte0 + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// The dither of 8 channels (two generator calls), split into two exact-sum
// bf16 pieces of -xi: -xi = hi + lo + r with |r| <= 2^-18 |xi|.
__device__ __forceinline__ void neg_dither8_bf16(uint32_t token, uint32_t g0, uint32_t tag, uint32_t stream,
                                                 uint32_t k0, uint32_t k1, bf16x8_t &hi, bf16x8_t &lo) {
  float xi[8];
  dither4(token, g0, tag, stream, k0, k1, xi);
  dither4(token, g0 + 1, tag, stream, k0, k1, xi + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = -xi[e];
    const float h = bf16_round(x);
    hi[e] = (__bf16)h;
    lo[e] = (__bf16)(x - h);
  }
}

struct TileRegs {
  uint4 k[4];      // FP8: k[0..1] = 32 codes; BF16: k[0..3] = 32 values
  uint4 ke[4];     // exact keys (bf16), 32 values
  uint2 wit;       // 4 witness bands (fp16)
  uint2 v8[4];     // FP8 values: 8 dims of 4 tokens (MFMA B layout)
  uint4 vb[4];     // BF16 values: 16 dims of 2 tokens (vector-ALU layout)
  float ks, vs;    // scales of this lane's compact (token, head) slot
};

// Addressing of one (request, KV head) region range ending at c1, and the
// loads of one 16-token tile.  Dense regions: one uniform base per tensor and
// 32-bit per-lane row offsets (a request holds < 2^24 tokens); paged suffix:
// per-token page lookup with 64-bit rows.  Rows are clamped to the last valid
// token, so a tile past the end re-reads a valid row (its data is unused).
template <int KF, int VF, bool PAGED>
struct TileSrc {
  using RowT = typename std::conditional<PAGED, size_t, uint32_t>::type;
  const uint8_t *kb, *keb, *vbb;
  const uint16_t *wb;
  const float *ksb, *vsb;
  const int32_t *ptab;
  int pshift, page_size, h_kv, kvh, last;

  __device__ __forceinline__ TileSrc(const DecodeLaunch &d, int b, int kvh_, int c1) {
    const RegionDev &R = d.region;
    const size_t sh = R.is_prefix ? (size_t)kvh_ : (size_t)b * d.h_kv + kvh_;
    const size_t row0 = PAGED ? 0 : sh * (size_t)R.length;
    ptab = PAGED ? R.page_table + (size_t)b * R.max_pages : nullptr;
    pshift = R.page_size == 16 ? 4 : 3;      // page sizes 8 or 16
    page_size = R.page_size;
    h_kv = d.h_kv;
    kvh = kvh_;
    last = c1 - 1;
    kb = (const uint8_t *)R.k + row0 * (KF == KVQ_FMT_BF16 ? 2 * D : D);
    keb = (const uint8_t *)R.k_exact + row0 * (2 * D);
    wb = R.witness + row0 * NB;
    ksb = (const float *)R.k_scale + row0;
    vbb = (const uint8_t *)R.v + row0 * (VF == KVQ_FMT_BF16 ? 2 * D : D);
    vsb = (const float *)R.v_scale + row0;
  }

  __device__ __forceinline__ RowT row_of(int t) const {   // row index relative to row0
    t = min(t, last);
    if constexpr (PAGED) {
      const size_t pg = (size_t)ptab[t >> pshift];
      return (pg * h_kv + kvh) * page_size + (t & (page_size - 1));
    } else {
      return (RowT)t;
    }
  }

  __device__ __forceinline__ void load(TileRegs &T, int t0, bool exact, bool wit) const {
    load_keys(T, t0, exact);
    load_rest(T, t0, wit);
  }

  // stored and exact keys with the key scale (what the logits need first)
  __device__ __forceinline__ void load_keys(TileRegs &T, int t0, bool exact) const {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j16 = lane & 15, pp = lane & 3;
    const RowT ra = row_of(t0 + j16), rk = row_of(t0 + 4 * g + pp);
    if constexpr (KF == KVQ_FMT_FP8_E4M3 || KF == KVQ_FMT_INT8_DITHER) {
      const uint4 *p = reinterpret_cast<const uint4 *>(kb + ra * D + 32 * g);
      T.k[0] = p[0];
      T.k[1] = p[1];
      T.ks = KF == KVQ_FMT_FP8_E4M3 ? ksb[rk] : 1.0f;   // INT8: block scales ride on q
    } else {
      const uint4 *p = reinterpret_cast<const uint4 *>(kb + ra * (2 * D) + 64 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) T.k[i] = p[i];
      T.ks = 1.0f;
    }
    if (exact) {
      const uint4 *p = reinterpret_cast<const uint4 *>(keb + ra * (2 * D) + 64 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) T.ke[i] = p[i];
    }
  }

  // witness, values and the value scale
  __device__ __forceinline__ void load_rest(TileRegs &T, int t0, bool wit) const {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j16 = lane & 15, pp = lane & 3;
    const RowT ra = row_of(t0 + j16), rk = row_of(t0 + 4 * g + pp);
    if (wit) T.wit = *reinterpret_cast<const uint2 *>(wb + ra * NB + 4 * g);
    if constexpr (VF == KVQ_FMT_FP8_E4M3 || VF == KVQ_FMT_INT8_DITHER) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        T.v8[e] = *reinterpret_cast<const uint2 *>(vbb + row_of(t0 + 4 * g + e) * D + 8 * j16);
      T.vs = VF == KVQ_FMT_FP8_E4M3 ? vsb[rk] : 1.0f;
    } else if constexpr (VF == KVQ_FMT_BF16) {
      const RowT r0 = row_of(t0 + (lane >> 3)), r1 = row_of(t0 + 8 + (lane >> 3));
      const uint4 *p0 = reinterpret_cast<const uint4 *>(vbb + r0 * (2 * D) + 32 * (lane & 7));
      const uint4 *p1 = reinterpret_cast<const uint4 *>(vbb + r1 * (2 * D) + 32 * (lane & 7));
      T.vb[0] = p0[0]; T.vb[1] = p0[1];
      T.vb[2] = p1[0]; T.vb[3] = p1[1];
      T.vs = 1.0f;
    }
  }
};

// One (request, KV head) chunk [c0, c1) of one region, run by the whole
// work-group (4 wavefronts, tiles of 16 tokens dealt round-robin): leaves each
// wavefront's softmax states and output accumulator in part_s[wv].  The
// (l~, l) pairs go to the spill: SPILL_LDS = the chunk's own LDS buffer
// (entry 64 ((t0 - c0) / 16) + lane), else the group's workspace rows.
//
// FULL: TV and meter requested and this region holds exact bf16 keys and a
// witness (the common quantized case).  Then every load of a tile is issued
// unconditionally, which lets the compiler keep the next tile's loads in
// flight across the current tile's math (no load sits under a runtime branch).
template <int KF, int VF, bool PAGED, bool FULL, bool SPILL_LDS>
__device__ __forceinline__ void mfma_chunk(const DecodeLaunch &d, int b, int kvh, int grp, int c0,
                                           int c1, float2 *spill_s, float (*w_s)[64],
                                           float (*part_s)[4][PART_STRIDE]) {
  constexpr int G = 4;
  const RegionDev &R = d.region;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j16 = lane & 15, hh = j16 >> 2, pp = lane & 3;

  const bool do_tv = FULL || d.has_tv != 0;
  const bool do_meter = FULL || d.has_meter != 0;
  const bool has_exact = FULL || R.exact_fmt == EX_BF16;
  const bool has_wit = FULL || R.witness != nullptr;
  const float qs = d.sm_scale * LOG2E;

  // ---- B operands of the logit contractions, column j16 = 4 hh + pp
  bf16x8_t bq[4];
  f16x4_t bw;
  {
    const float *qp = d.q + ((size_t)b * d.h_q + (size_t)kvh * G + hh) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qp[32 * g + 8 * s + e] * qs;
        const float hi = bf16_round(x);
        const float mid = bf16_round(x - hi);
        const float lo = bf16_round(x - hi - mid);
        const float piece = pp == 0 ? hi : (pp == 1 ? mid : (pp == 2 ? lo : 0.0f));
        bq[s][e] = (__bf16)piece;                   // exact: piece is a bf16 value
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bb = 4 * g + e;
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = qp[4 * bb + i], c = qp[64 + 4 * bb + i];
        ss += a * a + c * c;
      }
      const float qn = sqrtf(ss) * qs;
      const _Float16 h1 = (_Float16)qn;
      const _Float16 h2 = (_Float16)(qn - (float)h1);
      bw[e] = pp == 0 ? h1 : (pp == 1 ? h2 : (_Float16)0.0f);
    }
  }

  // INT8 (subtractive dither): x^ = s_c (code - xi) with s_c per 256-token
  // block and channel.  The logits take the block's scales on the query side:
  // bqs = exact three-way bf16 split of q_c s_c (log2 units), against the
  // codes and the two pieces of -xi.  Values are dequantized to fp16.
  constexpr bool I8K = KF == KVQ_FMT_INT8_DITHER;
  constexpr bool I8V = VF == KVQ_FMT_INT8_DITHER;
  bf16x8_t bqs[4];
  float sv8[8];                                    // value scales of dims 8 j16 + n
  uint32_t i8_stream = 0, i8_ktag = 0, i8_vtag = 0;
  size_t i8_scale_row0 = 0;
  if constexpr (I8K || I8V) {
    const size_t sh = R.is_prefix ? (size_t)kvh : (size_t)b * d.h_kv + kvh;
    i8_scale_row0 = sh * (size_t)((R.length + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK);
    i8_stream = (uint32_t)(R.is_prefix ? R.stream_id : (R.stream_ids ? R.stream_ids[b] : R.stream_id + b));
    i8_ktag = dither_tag(0, R.layer, kvh);
    i8_vtag = dither_tag(1, R.layer, kvh);
  }
  auto set_block = [&](int blk) {
    const size_t srow = (i8_scale_row0 + (size_t)blk) * D;
    if constexpr (I8K) {
      const uint16_t *ks = (const uint16_t *)R.k_scale + srow;
      const float *qp = d.q + ((size_t)b * d.h_q + (size_t)kvh * G + hh) * D;
#pragma unroll
      for (int s8 = 0; s8 < 4; ++s8) {
        const uint4 sc = *reinterpret_cast<const uint4 *>(ks + 32 * g + 8 * s8);
        const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = qp[32 * g + 8 * s8 + e] * qs * fp16_bits_to_f32((sw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          const float hi = bf16_round(x);
          const float mid = bf16_round(x - hi);
          const float lo = bf16_round(x - hi - mid);
          const float piece = pp == 0 ? hi : (pp == 1 ? mid : (pp == 2 ? lo : 0.0f));
          bqs[s8][e] = (__bf16)piece;
        }
      }
    }
    if constexpr (I8V) {
      const uint4 sc = *reinterpret_cast<const uint4 *>((const uint16_t *)R.v_scale + srow + 8 * j16);
      const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
      for (int n = 0; n < 8; ++n) sv8[n] = fp16_bits_to_f32((sw[n >> 1] >> (16 * (n & 1))) & 0xffffu);
    }
  };

  const TileSrc<KF, VF, PAGED> src(d, b, kvh, c1);
  float *spill_g = (do_tv && !SPILL_LDS) ? spill_region<G>(d, grp, R.is_prefix != 0) : nullptr;
  auto load_tile = [&](TileRegs &T, int t0) { src.load(T, t0, do_tv && has_exact, do_meter && has_wit); };

  // per-lane accumulator states (lane = one (token slot, head) pair)
  float mq = NEG_INF, zq = 0.0f;     // attention softmax, maximum uniform per head
  float mm = NEG_INF, zm = 0.0f;     // l~ + c (Theorem 1's A)
  float me = NEG_INF, ze = 0.0f;     // exact logits (TV normalizer)
  // FP8 values: output in MFMA accumulators, N-tile n, lane j16 = dims 8 j16 + n,
  // register r = head r (lanes 0..15).  BF16 values: acc[h][i] per lane.
  f32x4_t ov[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) ov[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int NACC = (VF == KVQ_FMT_BF16) ? G : 1;
  float acc[NACC][16];
#pragma unroll
  for (int h = 0; h < NACC; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;

  auto process = [&](const TileRegs &T, int t0) {
    // ---- logit contractions on the matrix cores
    f32x4_t dq = {0.0f, 0.0f, 0.0f, 0.0f}, de = dq, dc = dq;
    if constexpr (KF == KVQ_FMT_FP8_E4M3) {
      const uint32_t w[8] = {T.k[0].x, T.k[0].y, T.k[0].z, T.k[0].w,
                             T.k[1].x, T.k[1].y, T.k[1].z, T.k[1].w};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w[2 * s], w[2 * s + 1]), bq[s], dq, 0, 0, 0);
    } else if constexpr (I8K) {
      // row j16 = token t0 + j16, slice s = channels 32 g + 8 s .. + 7
      const uint32_t w[8] = {T.k[0].x, T.k[0].y, T.k[0].z, T.k[0].w,
                             T.k[1].x, T.k[1].y, T.k[1].z, T.k[1].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 cw = {i8x2_to_bf16x2(w[2 * s], 0), i8x2_to_bf16x2(w[2 * s], 2),
                          i8x2_to_bf16x2(w[2 * s + 1], 0), i8x2_to_bf16x2(w[2 * s + 1], 2)};
        bf16x8_t xh, xl;
        neg_dither8_bf16((uint32_t)(t0 + j16), (uint32_t)(8 * g + 2 * s), i8_ktag, i8_stream, R.seed_lo,
                         R.seed_hi, xh, xl);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cw), bqs[s], dq, 0, 0, 0);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bqs[s], dq, 0, 0, 0);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bqs[s], dq, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.k[s]), bq[s], dq, 0, 0, 0);
    }
    if (do_tv && has_exact) {
#pragma unroll
      for (int s = 0; s < 4; ++s) de = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.ke[s]), bq[s], de, 0, 0, 0);
    }
    if (do_meter && has_wit)
      dc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, T.wit), bw, dc, 0, 0, 0);

    const int tk = t0 + 4 * g + pp;
    const bool valid = tk < c1;
    float lq = collapse(dq, pp) * T.ks;
    float le = (do_tv && has_exact) ? collapse(de, pp) : lq;
    const float cc = (do_meter && has_wit) ? collapse(dc, pp) : 0.0f;
    if (!valid) {
      lq = NEG_INF;
      le = NEG_INF;
    }
    // spill entry of (tk, hh) is 64 (t0 / 16) + lane: one contiguous 512-byte store
    if constexpr (SPILL_LDS) {
      if (do_tv) spill_s[64 * ((t0 - c0) >> 4) + lane] = make_float2(lq, le);
    } else {
      if (do_tv && valid)
        st_pair(spill_g + 2 * ((size_t)64 * (t0 >> 4) + lane), lq, le, d.total_chunks > 1);
    }

    // ---- attention softmax (maximum uniform per head)
    if (__any(lq > mq + LAZY)) {
      float mx = lq;
      mx = fmaxf(mx, dpp<DPP_QUAD_XOR1>(mx));
      mx = fmaxf(mx, dpp<DPP_QUAD_XOR2>(mx));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = mx > mq + LAZY ? mx : mq;
      const float f = merge_factor(mq, mnew);
      zq *= f;
      float fh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) fh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 4 * h));
      if constexpr (VF == KVQ_FMT_FP8_E4M3 || VF == KVQ_FMT_INT8_DITHER) {   // MFMA accumulators
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[n][r] *= fh[r];
      } else if constexpr (VF == KVQ_FMT_BF16) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[h][i] *= fh[h];
      }
      mq = mnew;
    }
    const float p = valid ? fast_exp2(lq - mq) : 0.0f;
    zq += p;
    if (do_tv) {
      if (le > me + LAZY) {
        ze *= merge_factor(me, le);
        me = le;
      }
      ze += valid ? fast_exp2(le - me) : 0.0f;
    }
    if (do_meter) {
      const float y = lq + cc;
      if (y > mm + LAZY) {
        zm *= merge_factor(mm, y);
        mm = y;
      }
      zm += valid ? fast_exp2(y - mm) : 0.0f;
    }

    // ---- output accumulation
    if constexpr (VF == KVQ_FMT_FP8_E4M3) {
      // weights to the A layout: lane (16 g' + h) needs tokens 4g'..4g'+3 of head h
      w_s[wv][16 * hh + 4 * g + pp] = p * T.vs;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4 wa = *reinterpret_cast<const float4 *>(&w_s[wv][16 * (j16 & 3) + 4 * g]);
      const bool arow = j16 < 4;
      const f16x4_t aw = {(_Float16)(arow ? wa.x : 0.0f), (_Float16)(arow ? wa.y : 0.0f),
                          (_Float16)(arow ? wa.z : 0.0f), (_Float16)(arow ? wa.w : 0.0f)};
      const uint32_t lo[4] = {T.v8[0].x, T.v8[1].x, T.v8[2].x, T.v8[3].x};
      const uint32_t hi[4] = {T.v8[0].y, T.v8[1].y, T.v8[2].y, T.v8[3].y};
      uint32_t tl[4], th[4];
      transpose4x4(lo, tl);
      transpose4x4(hi, th);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        ov[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(aw, fp8x4_to_f16(tl[n]), ov[n], 0, 0, 0);
        ov[n + 4] = __builtin_amdgcn_mfma_f32_16x16x16f16(aw, fp8x4_to_f16(th[n]), ov[n + 4], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    } else if constexpr (I8V) {
      // as FP8, with weights p and values s_c (code - xi) in fp16
      w_s[wv][16 * hh + 4 * g + pp] = p;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4 wa = *reinterpret_cast<const float4 *>(&w_s[wv][16 * (j16 & 3) + 4 * g]);
      const bool arow = j16 < 4;
      const f16x4_t aw = {(_Float16)(arow ? wa.x : 0.0f), (_Float16)(arow ? wa.y : 0.0f),
                          (_Float16)(arow ? wa.z : 0.0f), (_Float16)(arow ? wa.w : 0.0f)};
      f16x4_t vb[8];                               // vb[n][e]: token t0 + 4 g + e, dim 8 j16 + n
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float xi[8];
        const uint32_t tok = (uint32_t)(t0 + 4 * g + e);
        dither4(tok, (uint32_t)(2 * j16), i8_vtag, i8_stream, R.seed_lo, R.seed_hi, xi);
        dither4(tok, (uint32_t)(2 * j16 + 1), i8_vtag, i8_stream, R.seed_lo, R.seed_hi, xi + 4);
        const uint32_t cw[2] = {T.v8[e].x, T.v8[e].y};
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float code = (float)(int)(int8_t)(cw[n >> 2] >> (8 * (n & 3)));
          vb[n][e] = (_Float16)(sv8[n] * (code - xi[n]));
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) ov[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(aw, vb[n], ov[n], 0, 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    } else if constexpr (VF == KVQ_FMT_BF16) {
      w_s[wv][4 * (4 * g + pp) + hh] = p;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4 w0 = *reinterpret_cast<const float4 *>(&w_s[wv][4 * (lane >> 3)]);
      const float4 w1 = *reinterpret_cast<const float4 *>(&w_s[wv][4 * ((lane >> 3) + 8)]);
      const float wa[G] = {w0.x, w0.y, w0.z, w0.w};
      const float wb[G] = {w1.x, w1.y, w1.z, w1.w};
      const uint32_t a[8] = {T.vb[0].x, T.vb[0].y, T.vb[0].z, T.vb[0].w,
                             T.vb[1].x, T.vb[1].y, T.vb[1].z, T.vb[1].w};
      const uint32_t c[8] = {T.vb[2].x, T.vb[2].y, T.vb[2].z, T.vb[2].w,
                             T.vb[3].x, T.vb[3].y, T.vb[3].z, T.vb[3].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * i] = fmaf(wa[h], bf16_lo(a[i]), fmaf(wb[h], bf16_lo(c[i]), acc[h][2 * i]));
          acc[h][2 * i + 1] = fmaf(wa[h], bf16_hi(a[i]), fmaf(wb[h], bf16_hi(c[i]), acc[h][2 * i + 1]));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  };

  // two register sets, no copies: the loads of one tile overlap the other's
  // math.  The next tile is always loaded (rows clamp to the last valid
  // token, so past the end this re-reads a valid row and the data is unused).
  TileRegs ta, tb;
  if constexpr (I8K || I8V) {
    // INT8: wavefront wv takes whole 256-token blocks wv, wv + 4, ... of the
    // chunk, so the block operands change once per 16 tiles
    const int blk0 = c0 / KVQ_INT8_BLOCK;
    for (int blk = blk0 + wv; blk * KVQ_INT8_BLOCK < c1; blk += WAVES) {
      const int tb0 = max(blk * KVQ_INT8_BLOCK, c0), tb1 = min((blk + 1) * KVQ_INT8_BLOCK, c1);
      set_block(blk);
      int t0 = tb0;
      load_tile(ta, t0);
      while (t0 < tb1) {
        load_tile(tb, t0 + 16);
        process(ta, t0);
        t0 += 16;
        if (t0 >= tb1) break;
        load_tile(ta, t0 + 16);
        process(tb, t0);
        t0 += 16;
      }
    }
  } else {
    constexpr int STEP = 16 * WAVES;
    int t0 = c0 + 16 * wv;
    if (t0 < c1) load_tile(ta, t0);
    while (t0 < c1) {
      load_tile(tb, t0 + STEP);
      process(ta, t0);
      t0 += STEP;
      if (t0 >= c1) break;
      load_tile(ta, t0 + STEP);
      process(tb, t0);
      t0 += STEP;
    }
  }

  // ---- wavefront merge: lanes of one head differ in bits 0, 1, 4, 5
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    if (off == 4 || off == 8) continue;
    zq += __shfl_xor(zq, off);
    if (do_meter) {
      const float m2 = __shfl_xor(mm, off), z2 = __shfl_xor(zm, off);
      const float m = fmaxf(mm, m2);
      zm = zm * merge_factor(mm, m) + z2 * merge_factor(m2, m);
      mm = m;
    }
    if (do_tv) {
      const float m2 = __shfl_xor(me, off), z2 = __shfl_xor(ze, off);
      const float m = fmaxf(me, m2);
      ze = ze * merge_factor(me, m) + z2 * merge_factor(m2, m);
      me = m;
    }
  }
  if constexpr (VF == KVQ_FMT_BF16) {
#pragma unroll
    for (int off = 8; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] += __shfl_xor(acc[h][i], off);
  }

  if (lane < 16 && pp == 0) {                      // lane 4h holds head h
    part_s[wv][hh][0] = mq; part_s[wv][hh][1] = zq;
    part_s[wv][hh][2] = mm; part_s[wv][hh][3] = zm;
    part_s[wv][hh][4] = me; part_s[wv][hh][5] = ze;
  }
  if constexpr (VF == KVQ_FMT_FP8_E4M3 || VF == KVQ_FMT_INT8_DITHER) {   // MFMA accumulators
    if (lane < 16) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) part_s[wv][r][8 + 8 * lane + n] = ov[n][r];
    }
  } else if constexpr (VF == KVQ_FMT_BF16) {
    if (lane < 8) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) part_s[wv][h][8 + 16 * lane + i] = acc[h][i];
    }
  } else {
    if (lane < 16) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) part_s[wv][r][8 + 8 * lane + n] = 0.0f;
    }
  }
}

template <int KF, int VF, bool PAGED, bool FULL>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(const DecodeLaunch d) {
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const unsigned n_work = (unsigned)d.batch * d.h_kv * d.n_chunks;
  if (L >= n_work) return;
  const int chunk_idx = (int)(L % (unsigned)d.n_chunks);
  const int grp = (int)(L / (unsigned)d.n_chunks);
  const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;
  const RegionDev &R = d.region;
  const int len = R.is_prefix ? R.length : (R.lengths ? min(max(R.lengths[b], 0), R.length) : R.length);
  const int c0 = chunk_idx * d.chunk;
  const int c1 = min(c0 + d.chunk, len);
  __shared__ __attribute__((aligned(16))) float w_s[WAVES][64];
  __shared__ float part_s[WAVES][4][PART_STRIDE];
  mfma_chunk<KF, VF, PAGED, FULL, false>(d, b, kvh, grp, c0, c1, nullptr, w_s, part_s);
  chunk_epilogue<4>(d, part_s, grp, chunk_idx, b, kvh);
}

// ----------------------------------------------------------------- teams
// A team of T work-groups shares each (request, KV head): member m takes
// tokens [m chunk, (m + 1) chunk) and keeps that chunk's (l~, l) pairs in its
// own LDS, so the TV needs no spill traffic to HBM.  Teams are persistent:
// team t handles groups t, t + n_teams, ... in rounds.
//
// Exchange: each member publishes, per round, its merged softmax states and
// output accumulator into its slot, every word as (tag, value) in one 64-bit
// store; the tag names the launch and round, so a reader polls each word
// until its tag is the expected one.  No store has to be waited for and no
// counter is needed.  Every member derives the exact normalizers of the
// group from all members' states; member h % T writes head h's output, log A,
// bound and meter.  The chunk's TV shares are published in the same slot and
// summed (member order) by member h % T one round later, or at the end of the
// last round.  Slots alternate between two buffers by round parity: a member
// writes round r + 2 only after it has read every member's round r + 1
// states, which each member publishes after it has finished with round r.
// All reductions run in a fixed order (bitwise reproducible).  The grid fits
// the device at once, so all members are resident; a bounded wait leaves NaN
// in the group's results instead of hanging.
constexpr int SLOT_WORDS = 544;    // 24 states (6 per head), 4 TV shares, 4 pad, 512 accumulator words
constexpr int SLOT_TV = 24, SLOT_ACC = 32;

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Words w[i] loaded earlier from addr(i): re-polls any whose tag is not yet
// `tag` and returns the values.  Returns false if a word never arrived.
template <int N, class Addr>
__device__ __forceinline__ bool settle_tagged(Addr addr, uint32_t tag, uint64_t (&w)[N], float (&v)[N],
                                              unsigned limit) {
  bool ok = true;
  unsigned spins = 0;                 // one budget for the whole batch
#pragma unroll
  for (int i = 0; i < N; ++i) {
    while (ok && (uint32_t)(w[i] >> 32) != tag) {
      __builtin_amdgcn_s_sleep(2);
      w[i] = ld_tagged(addr(i));
      if (++spins >= limit) ok = false;            // budget spent: no further waits
    }
    v[i] = __uint_as_float((uint32_t)w[i]);
  }
  return ok;
}

// Reads N tagged words (all loads in flight together), then re-polls any
// whose tag is not yet `tag`.  Returns false if a word never arrived.
template <int N>
__device__ __forceinline__ bool read_tagged(const uint64_t *const (&p)[N], uint32_t tag, float (&v)[N],
                                            unsigned limit) {
  uint64_t w[N];
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = ld_tagged(p[i]);
  return settle_tagged<N>([&](int i) { return p[i]; }, tag, w, v, limit);
}

// (M, Z) merge of two online-softmax states; symmetric in its arguments
__device__ __forceinline__ void mz_merge(float &m, float &z, float m2, float z2) {
  const float mx = fmaxf(m, m2);
  z = z * merge_factor(m, mx) + z2 * merge_factor(m2, mx);
  m = mx;
}

// Sum of the members' TV shares of head h (lanes c < n hold member c's
// share, the others 0): butterfly over the lowest ceil(log2 n) lane bits, so
// lane 0 holds the sum in a fixed order.
__device__ __forceinline__ float wave_sum_fixed(float x, int n) {
  for (int off = 1; off < n; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ void team_epilogue(const DecodeLaunch &d, float (*part_s)[4][PART_STRIDE],
                              const float2 *spill_s, int team, int member, int round,
                              bool last_round, int b, int kvh, int c0, int c1) {
  constexpr int G = 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int T = d.team;
  const bool do_tv = d.has_tv != 0;
  const bool do_meter = d.has_meter != 0;
  const uint32_t tag = d.epoch + (uint32_t)round + 1u;
  uint64_t *slots = reinterpret_cast<uint64_t *>(d.partials) + (size_t)(team * 2 + (round & 1)) * T * SLOT_WORDS;
  uint64_t *mine = slots + (size_t)member * SLOT_WORDS;
  __shared__ float mq_s[G][64];
  __shared__ float unit_s[WAVES][64];
  __shared__ float fin_s[G][4];
  __shared__ float tvw_s[WAVES][G];
  __shared__ int bad_s;
  const float qnan = __builtin_nanf("");

  // 1. publish this member's merged states and accumulator
  if (tid == 0) bad_s = 0;
  __syncthreads();
  for (int idx = tid; idx < G * PART_STRIDE; idx += 256) {
    const int h = idx / PART_STRIDE, k = idx - h * PART_STRIDE;
    if (k == 6 || k == 7) continue;
    const int mk = (k >= 8) ? 0 : (k & ~1);
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
    if (member != d.silent_member)                 // (a test hook silences one member)
      st_tagged(mine + (k < 6 ? 6 * h + k : SLOT_ACC + 128 * h + (k - 8)), tag, r);
  }

  // 2. the group's normalizers: wavefront h reads head h of every member
  //    (lane c = member c), then a butterfly merge over the lowest
  //    ceil(log2 T) lane bits leaves the group's states in lane 0
  const int h = __builtin_amdgcn_readfirstlane(wv);   // uniform: scalar slot bases
  bool ok = true;
  float Mq = NEG_INF, Zq = 0.0f, Mm = NEG_INF, Zm = 0.0f, Me = NEG_INF, Ze = 0.0f;
  if (lane < T) {
    const uint64_t *s = slots + (size_t)lane * SLOT_WORDS + 6 * h;
    const uint64_t *const p[6] = {s, s + 1, s + 2, s + 3, s + 4, s + 5};
    float v[6];
    ok = read_tagged<6>(p, tag, v, d.spin_limit);
    Mq = v[0]; Zq = v[1]; Mm = v[2]; Zm = v[3]; Me = v[4]; Ze = v[5];
  }
  // one member's words missing makes the whole group's states unknown: NaN
  // then flows into every result of the group (never a stale value)
  ok = __all(ok);
  if (!ok) {
    const float qnan_s = __builtin_nanf("");
    Mq = Zq = Mm = Zm = Me = Ze = qnan_s;
    if (lane == 0) bad_s = 1;
  }
  mq_s[h][lane] = Mq;
  for (int off = 1; off < T; off <<= 1) {           // lanes >= T hold empty states
    const float a0 = __shfl_xor(Mq, off), a1 = __shfl_xor(Zq, off);
    const float b0 = __shfl_xor(Mm, off), b1 = __shfl_xor(Zm, off);
    const float e0 = __shfl_xor(Me, off), e1 = __shfl_xor(Ze, off);
    mz_merge(Mq, Zq, a0, a1);
    mz_merge(Mm, Zm, b0, b1);
    mz_merge(Me, Ze, e0, e1);
  }
  if (lane == 0) {
    fin_s[h][0] = Mq;
    fin_s[h][1] = Zq > 0.0f ? 1.0f / Zq : 0.0f;
    fin_s[h][2] = Me;
    fin_s[h][3] = Ze > 0.0f ? 1.0f / Ze : 0.0f;
  }
  __syncthreads();

  // 3. duties, spread so that no member is always the last one out:
  //    - output: 8 units of 64 dims (head u / 2, half u % 2); unit u is
  //      taken by member u % T, wavefront (u / T) % 4 (T < 8) or by member u
  //      (T >= 8, see below), summing the members' accumulators in order;
  //    - log A, bound, meter of head h: member h % T (no loads);
  //    - the previous round's TV of head h: member (h + 4) % T, wavefront h.
  //    The first batch of accumulator words of this wavefront and the
  //    previous round's TV shares are requested first; the TV pass (4.)
  //    runs while they travel.
  const size_t qh = (size_t)b * d.h_q + (size_t)kvh * G + h;
  // T >= 8: unit u = member, its batches of 8 members dealt to the 4
  // wavefronts in turn, partial sums added in wavefront order through LDS
  const bool split = T >= 8;
  const int cb0 = split ? 8 * h : 0;                // this wavefront's first batch
  int pre_u = -1;                                   // unit of the pre-issued batch
  uint64_t pre_w[8];
  if (d.has_out) {
    for (int u = 0; u < 8; ++u) {
      if (split ? u != member : (u % T != member || (u / T) % 4 != h)) continue;
      if (cb0 < T) pre_u = u;
      break;
    }
    if (pre_u >= 0) {
      const uint64_t *ub = slots + SLOT_ACC + 128 * (pre_u >> 1) + 64 * (pre_u & 1) + lane;
#pragma unroll
      for (int i = 0; i < 8; ++i) pre_w[i] = ld_tagged(ub + (size_t)min(cb0 + i, T - 1) * SLOT_WORDS);
    }
  }
  const bool tv_duty = do_tv && d.tv && member == (h + 4) % T;
  // shares of round - 1 sit in the other parity's slots
  const uint64_t *prev_tv = reinterpret_cast<const uint64_t *>(d.partials) +
                            (size_t)(team * 2 + ((round - 1) & 1)) * T * SLOT_WORDS +
                            (size_t)min(lane, T - 1) * SLOT_WORDS + SLOT_TV + h;
  uint64_t pre_tv[1] = {0};
  if (tv_duty && round > 0 && lane < T) pre_tv[0] = ld_tagged(prev_tv);

  // 4. this chunk's TV share: thread tid reads entry pairs (2p, 2p + 1), p =
  //    tid + 256 k, as one float4 (both of head (tid % 8) / 2), into four
  //    independent partial sums; then a butterfly over the lanes of a head
  //    (bits 0, 3, 4, 5) and the wavefronts in order (published below)
  float acc_tv = 0.0f;
  if (do_tv && c1 > c0) {
    const int hm = (lane & 6) >> 1;
    const float Mt = fin_s[hm][0], iZt = fin_s[hm][1];
    const float Mx = fin_s[hm][2], iZe = fin_s[hm][3];
    const int n_pairs = round16(c1 - c0) * G / 2;
    const float4 *sp4 = reinterpret_cast<const float4 *>(spill_s);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = tid; p0 < n_pairs; p0 += 4 * 256) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + 256 * u;
        if (p < n_pairs) {
          const float4 x = sp4[p];
          const int e = 2 * p;
          const int t = c0 + 16 * (e >> 6) + 4 * ((e & 63) >> 4) + (e & 3);
          if (t < c1) tvp_add(a[u], x.x, x.y, Mt, iZt, Mx, iZe);
          if (t + 1 < c1) tvp_add(a[u], x.z, x.w, Mt, iZt, Mx, iZe);
        }
      }
    }
    acc_tv = (a[0] + a[1]) + (a[2] + a[3]);
  }
  acc_tv += __shfl_xor(acc_tv, 1);
  acc_tv += __shfl_xor(acc_tv, 8);
  acc_tv += __shfl_xor(acc_tv, 16);
  acc_tv += __shfl_xor(acc_tv, 32);
  if (lane < 8 && (lane & 1) == 0) tvw_s[wv][lane >> 1] = acc_tv;   // lanes 0, 2, 4, 6: heads 0..3

  // 3 (continued): the output units
  if (d.has_out) {
    for (int u = 0; u < 8; ++u) {
      if (split ? u != member : (u % T != member || (u / T) % 4 != h)) continue;
      const int hu = u >> 1, dim = 64 * (u & 1) + lane;
      const float Mu = fin_s[hu][0];
      const float iZu = fin_s[hu][1];
      const uint64_t *ub = slots + SLOT_ACC + 128 * hu + dim;
      float o = 0.0f;
      bool oku = true;
      for (int cb = cb0; cb < T; cb += split ? 32 : 8) {
        float v[8];
        if (u == pre_u && cb == cb0) {
          oku = settle_tagged<8>([&](int i) { return ub + (size_t)min(cb + i, T - 1) * SLOT_WORDS; },
                                 tag, pre_w, v, d.spin_limit) && oku;
        } else {
          const uint64_t *p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = ub + (size_t)min(cb + i, T - 1) * SLOT_WORDS;
          oku = read_tagged<8>(p, tag, v, d.spin_limit) && oku;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (cb + i < T) o += v[i] * merge_factor(mq_s[hu][cb + i], Mu);
      }
      const size_t qu = (size_t)b * d.h_q + (size_t)kvh * G + hu;
      if (split) {
        unit_s[h][lane] = o;
        if (!oku) bad_s = 1;
      } else {
        d.out[qu * D + dim] = oku ? o * iZu : qnan;
        ok = ok && oku;
      }
    }
    if (split && member < 8) {                     // uniform over the work-group
      __syncthreads();
      if (h == 0) {
        const int hu = member >> 1, dim = 64 * (member & 1) + lane;
        const float o = ((unit_s[0][lane] + unit_s[1][lane]) + unit_s[2][lane]) + unit_s[3][lane];
        const size_t qu = (size_t)b * d.h_q + (size_t)kvh * G + hu;
        d.out[qu * D + dim] = bad_s == 0 ? o * fin_s[hu][1] : qnan;
      }
    }
  }
  if (member == h % T && lane == 0) {
    double log_a = 0.0;
    if (do_meter && Zq > 0.0f && Zm > 0.0f)
      log_a = ((double)Mm - (double)Mq) * 0.69314718055994530942 + log((double)Zm) - log((double)Zq);
    const double bound = 0.5 * expm1(2.0 * log_a);
    const float bf = bound > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)bound;
    if (d.log_a) d.log_a[qh] = ok ? (float)log_a : qnan;
    if (d.bound_raw) d.bound_raw[qh] = ok ? bf : qnan;
    if (d.meter) d.meter[qh] = ok ? fminf(1.0f, bf) : qnan;
  }
  if (tv_duty && round > 0) {
    float sh = 0.0f;
    bool okp = true;
    if (lane < T) {
      float v[1];
      okp = settle_tagged<1>([&](int) { return prev_tv; }, tag - 1u, pre_tv, v, d.spin_limit);
      sh = v[0];
    }
    sh = wave_sum_fixed(sh, T);
    okp = __all(okp);
    const int pg = team + (round - 1) * d.n_teams;
    const int pb = pg / d.h_kv, pk = pg - pb * d.h_kv;
    if (lane == 0) d.tv[(size_t)pb * d.h_q + (size_t)pk * G + h] = okp ? 0.5f * sh : qnan;
  }
  if (!ok) bad_s = 1;
  __syncthreads();
  if (tid < G) {
    const float share = ((tvw_s[0][tid] + tvw_s[1][tid]) + tvw_s[2][tid]) + tvw_s[3][tid];
    if (member != d.silent_member) st_tagged(mine + SLOT_TV + tid, tag, share);
  }

  // 5. last round: member (h + 4) % T also sums this round's shares
  if (last_round && tv_duty) {
    float sh = 0.0f;
    bool okp = true;
    if (lane < T) {
      const uint64_t *const p[1] = {slots + (size_t)lane * SLOT_WORDS + SLOT_TV + h};
      float v[1];
      okp = read_tagged<1>(p, tag, v, d.spin_limit);
      sh = v[0];
    }
    sh = wave_sum_fixed(sh, T);
    okp = __all(okp) && bad_s == 0;
    if (lane == 0) d.tv[qh] = okp ? 0.5f * sh : qnan;
  }
  __syncthreads();                  // LDS buffers are reused by the next round
}

template <int KF, int VF, bool PAGED, bool FULL>
__global__ __launch_bounds__(256, 2) void decode_mfma_team_kernel(const DecodeLaunch d) {
  extern __shared__ __attribute__((aligned(16))) float2 spill_s[];   // d.chunk * 4 entries
  __shared__ __attribute__((aligned(16))) float w_s[WAVES][64];
  __shared__ float part_s[WAVES][4][PART_STRIDE];
  const int T = d.team;
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const int team = (int)(L / (unsigned)T), member = (int)(L % (unsigned)T);
  if (team >= d.n_teams) return;                     // grid padding: member of no team
  const int groups = d.batch * d.h_kv;
  const RegionDev &R = d.region;
  for (int round = 0;; ++round) {
    const int grp = team + round * d.n_teams;
    if (grp >= groups) break;
    const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;
    const int len = R.is_prefix ? R.length : (R.lengths ? min(max(R.lengths[b], 0), R.length) : R.length);
    const int c0 = member * d.chunk;
    const int c1 = min(c0 + d.chunk, len);
    // (the next round's first tile is not loaded ahead: its loads would sit
    // ahead of the exchange's polls in the in-order load counter)
    mfma_chunk<KF, VF, PAGED, FULL, true>(d, b, kvh, grp, c0, c1, spill_s, w_s, part_s);
    team_epilogue(d, part_s, spill_s, team, member, round, grp + d.n_teams >= groups, b, kvh, c0, c1);
  }
}

template <int KF, int VF, bool PAGED>
static void launch_p(const DecodeLaunch &d, hipStream_t stream, dim3 grid) {
  const bool full = d.has_tv && d.has_meter && d.region.exact_fmt == EX_BF16 && d.region.witness;
  if (full)
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, true>), grid, dim3(256), 0, stream, d);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, false>), grid, dim3(256), 0, stream, d);
}

template <int KF, int VF>
static hipError_t launch_m(const DecodeLaunch &d, hipStream_t stream) {
  const long work = (long)d.batch * d.h_kv * d.n_chunks;
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
  if constexpr (KF == KVQ_FMT_INT8_DITHER) {
    launch_p<KF, VF, false>(d, stream, grid);       // INT8 regions are dense
  } else {
    if (d.region.paged)
      launch_p<KF, VF, true>(d, stream, grid);
    else
      launch_p<KF, VF, false>(d, stream, grid);
  }
  return hipGetLastError();
}

template <int KF, int VF, bool PAGED, bool FULL>
static const void *team_fn() {
  return reinterpret_cast<const void *>(&decode_mfma_team_kernel<KF, VF, PAGED, FULL>);
}

template <int KF, int VF>
static const void *team_fn_kv(bool paged, bool full) {
  if (paged) return full ? team_fn<KF, VF, true, true>() : team_fn<KF, VF, true, false>();
  return full ? team_fn<KF, VF, false, true>() : team_fn<KF, VF, false, false>();
}

static const void *team_kernel(int k_format, int v_format, bool paged, bool full) {
  if (k_format == KVQ_FMT_FP8_E4M3) {
    if (v_format == KVQ_FMT_FP8_E4M3) return team_fn_kv<KVQ_FMT_FP8_E4M3, KVQ_FMT_FP8_E4M3>(paged, full);
    if (v_format == KVQ_FMT_BF16) return team_fn_kv<KVQ_FMT_FP8_E4M3, KVQ_FMT_BF16>(paged, full);
    return team_fn_kv<KVQ_FMT_FP8_E4M3, VF_NONE>(paged, full);
  }
  if (v_format == KVQ_FMT_FP8_E4M3) return team_fn_kv<KVQ_FMT_BF16, KVQ_FMT_FP8_E4M3>(paged, full);
  if (v_format == KVQ_FMT_BF16) return team_fn_kv<KVQ_FMT_BF16, KVQ_FMT_BF16>(paged, full);
  return team_fn_kv<KVQ_FMT_BF16, VF_NONE>(paged, full);
}

int team_capacity(int k_format, int v_format, bool paged, bool full) {
  // resident work-groups of the team kernel with the largest LDS chunk;
  // cached per device and kernel instance, 0 when the device cannot tell
  static int cache[16][2][3][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  const int ki = k_format == KVQ_FMT_FP8_E4M3 ? 1 : 0;
  const int vi = v_format == KVQ_FMT_FP8_E4M3 ? 1 : (v_format == KVQ_FMT_BF16 ? 2 : 0);
  int &c = cache[dev][ki][vi][paged ? 1 : 0][full ? 1 : 0];
  if (c > 0) return c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, team_kernel(k_format, v_format, paged, full),
                                                   256, (size_t)TEAM_MAX_CHUNK * 4 * sizeof(float2)) != hipSuccess)
    return 0;
  c = per_cu * cus;
  return c;
}

hipError_t launch_decode_team(const DecodeLaunch &d, int grid, hipStream_t stream) {
  const bool full = d.has_tv && d.has_meter && d.region.exact_fmt == EX_BF16 && d.region.witness;
  const void *fn = team_kernel(d.k_format, d.v_format, d.region.paged != 0, full);
  DecodeLaunch arg = d;
  void *args[] = {&arg};
  // A plain launch: members wait only for members of their own team, and a
  // team's members are consecutive in dispatch order within an XCD's share of
  // the grid, so they become resident together (the grid fits the device at
  // once); a wait that runs out of budget gives NaN, never a hang.
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args,
                         (size_t)d.chunk * 4 * sizeof(float2), stream);
}

bool mfma_path_supports(const DecodeLaunch &d) {
  if (d.group != 4 || d.region.exact_fmt == EX_F32) return false;
  if (d.k_format == KVQ_FMT_INT8_DITHER)           // dense INT8 keys and INT8 (or no) values
    return !d.region.paged && (d.v_format == KVQ_FMT_INT8_DITHER || d.v_format == VF_NONE);
  return (d.k_format == KVQ_FMT_FP8_E4M3 || d.k_format == KVQ_FMT_BF16) &&
         (d.v_format == KVQ_FMT_FP8_E4M3 || d.v_format == KVQ_FMT_BF16 || d.v_format == VF_NONE);
}

hipError_t launch_decode_mfma(const DecodeLaunch &d, hipStream_t s) {
  if (d.k_format == KVQ_FMT_INT8_DITHER) {
    if (d.v_format == KVQ_FMT_INT8_DITHER)
      return launch_m<KVQ_FMT_INT8_DITHER, KVQ_FMT_INT8_DITHER>(d, s);
    return launch_m<KVQ_FMT_INT8_DITHER, VF_NONE>(d, s);
  }
  if (d.k_format == KVQ_FMT_FP8_E4M3) {
    if (d.v_format == KVQ_FMT_FP8_E4M3) return launch_m<KVQ_FMT_FP8_E4M3, KVQ_FMT_FP8_E4M3>(d, s);
    if (d.v_format == KVQ_FMT_BF16) return launch_m<KVQ_FMT_FP8_E4M3, KVQ_FMT_BF16>(d, s);
    return launch_m<KVQ_FMT_FP8_E4M3, VF_NONE>(d, s);
  }
  if (d.v_format == KVQ_FMT_FP8_E4M3) return launch_m<KVQ_FMT_BF16, KVQ_FMT_FP8_E4M3>(d, s);
  if (d.v_format == KVQ_FMT_BF16) return launch_m<KVQ_FMT_BF16, KVQ_FMT_BF16>(d, s);
  return launch_m<KVQ_FMT_BF16, VF_NONE>(d, s);
}

}  // namespace kvq
