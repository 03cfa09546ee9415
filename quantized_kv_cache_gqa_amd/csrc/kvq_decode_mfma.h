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
// of the four heads (lanes 0..15 hold it).  BF16 values take the same layout
// at two bytes a value on v_mfma_f32_16x16x32_bf16, the weights split into
// two bf16 pieces along the contraction (see the tile's P.V).
#pragma once

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

// the same rounding (to nearest, ties to even) by the conversion instruction
__device__ __forceinline__ float bf16_hw_round(float x) { return (float)(__bf16)x; }

// x * y rounded to fp32 by itself (never fused into a following add)
__device__ __forceinline__ float mul_rn(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}

// Piece p of the exact three-way bf16 split x = hi + mid + lo (p = 3: zero).
// All three pieces are formed and one is picked with bit masks: a select
// chain on the lane's p compiles to divergent branches, and a load feeding
// the next element is then not issued before the branches close.
// (No contraction: a product feeding x must not be fused into x - hi, or the
// pieces would split the unrounded product and kernels would differ in the
// last bit depending on how the compiler schedules them.)
__device__ __forceinline__ float split3_piece(float x, int p) {
#pragma clang fp contract(off)
  const float hi = bf16_round(x);
  const float mid = bf16_round(x - hi);
  const float lo = bf16_round(x - hi - mid);
  const uint32_t m0 = 0u - (uint32_t)(p == 0), m1 = 0u - (uint32_t)(p == 1), m2 = 0u - (uint32_t)(p == 2);
  return __uint_as_float((__float_as_uint(hi) & m0) | (__float_as_uint(mid) & m1) | (__float_as_uint(lo) & m2));
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

// The dither of 8 channels: channel groups g0 and g0 + 1 (two generator calls).
__device__ __forceinline__ void dither8(uint32_t token, uint32_t g0, uint32_t tag, uint32_t stream, uint32_t k0,
                                        uint32_t k1, float (&xi)[8]) {
  dither4(token, g0, tag, stream, k0, k1, xi);
  dither4(token, g0 + 1, tag, stream, k0, k1, xi + 4);
}

// -xi split into two exact-sum bf16 pieces: -xi = hi + lo + r, |r| <= 2^-18 |xi|
// (the conversion instruction rounds to nearest even, as bf16_round does for
// finite values, in one instruction per pair).
__device__ __forceinline__ void neg_split8_bf16(const float (&xi)[8], bf16x8_t &hi, bf16x8_t &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = -xi[e];
    const float h = bf16_hw_round(x);
    hi[e] = (__bf16)h;
    lo[e] = (__bf16)(x - h);
  }
}

// Row length (floats) of a wavefront's LDS tile of dithers: 16 tokens x 128
// channels, each row padded by 4 so that the 16 rows start in different banks.
constexpr int XI_ROW = D + 4;

struct TileRegs {
  uint4 k[4];      // FP8: k[0..1] = 32 codes; BF16: k[0..3] = 32 values
  uint4 ke[4];     // exact keys (bf16), 32 values
  uint2 wit;       // 4 witness bands (fp16)
  uint2 v8[4];     // FP8 values: 8 dims of 4 tokens (MFMA B layout)
  uint4 vb[4];     // BF16 values: token 4 g + e, dims 8 j16 .. 8 j16 + 7
  float ks, vs;    // scales of this lane's compact (token, head) slot
  uint32_t vrec;   // value record of this lane's token: fp16 (rho, ||v||)
  uint2 kg[4];     // INT8 group scales: the 4 fp16 key scales of token 4 g + e
  uint32_t vg[4];  // INT8 group scales: value scale of token 4 g + e, dims 8 j16 ..
  uint4 ko;        // outlier values 8 g .. 8 g + 7 of token j16 (bf16, 0 past 2 m)
};

// Tokens between a wavefront's consecutive tiles in the tile loop (the
// work-group's four wavefronts take 16-token tiles in turn).
constexpr int TILE_STEP = 16 * WAVES;

// Page ids of one tile of a paged region: `lo` holds its tokens 0..7, `hi`
// tokens 8..15 (the same page when pages hold 16 tokens).  Unused when dense.
struct TilePages {
  int lo = 0, hi = 0;
};

// Addressing of one (request, KV head) region range [c0, c1), and the loads
// of one 16-token tile.  Dense regions: one uniform base per tensor and 32-bit
// per-lane row offsets (a request holds < 2^24 tokens); paged suffix: 64-bit
// rows from the tile's page ids.  Rows are clamped to the last valid token, so
// a tile past the end re-reads a valid row (its data is unused).
//
// Page ids come from a per-wavefront window: one vector load fetches the
// pages of the wavefront's next 64 tiles (lane i: tile kw + i; tiles are
// TILE_STEP tokens apart from tb = c0 + 16 wv), and each tile reads its two
// ids back with lane reads.  A page lookup per token instead puts a
// dependent load in front of every tile's loads, and its wait drains the
// in-order load counter, so a wavefront keeps about one tile in flight.
// (Tiles start on multiples of 16 tokens: chunk starts are multiples of 64,
// team chunks whole tiles, so a tile never spans more than two 8-token pages
// or one 16-token page.)
template <int KF, int VF, bool PAGED>
struct TileSrc {
  using RowT = typename std::conditional<PAGED, size_t, uint32_t>::type;
  const uint8_t *kb, *keb, *vbb;
  const uint16_t *wb, *vwb;
  const float *ksb, *vsb;
  const uint16_t *ksg, *vsg;   // INT8 group scales: 4 per row
  const uint16_t *kob;         // outlier values of the keys: 2 n_op per row
  int n_op;
  const int32_t *ptab;
  int pshift, page_size, h_kv, kvh, last;
  // paged regions: the page window (empty for dense regions)
  struct Window {
    int tb;                    // first token of this wavefront's tiles
    int kw;                    // first tile index held
    int32_t lo, hi;
  };
  struct NoWindow {};
  using WinT = typename std::conditional<PAGED, Window, NoWindow>::type;
  mutable WinT win;

  __device__ __forceinline__ TileSrc(const DecodeLaunch &d, int b, int kvh_, int c0, int c1) {
    const RegionDev &R = d.region;
    if constexpr (PAGED) {
      win.tb = c0 + 16 * (int)(threadIdx.x >> 6);
      win.kw = -64;            // (the first tile refills)
      win.lo = win.hi = 0;
    }
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
    vwb = R.v_witness + row0 * 2;
    ksb = (const float *)R.k_scale + row0;
    vbb = (const uint8_t *)R.v + row0 * (VF == KVQ_FMT_BF16 ? 2 * D : D);
    vsb = (const float *)R.v_scale + row0;
    ksg = (const uint16_t *)R.k_scale + row0 * 4;
    vsg = (const uint16_t *)R.v_scale + row0 * 4;
    n_op = R.n_op;
    kob = R.kout + row0 * (size_t)(2 * R.n_op);
  }

  // the page ids of tile t0 (a tile of this wavefront, at or after every
  // tile asked for before); refills the window every 64 tiles
  __device__ __forceinline__ TilePages tile_pages(int t0) const {
    TilePages P;
    if constexpr (PAGED) {
      const int k = __builtin_amdgcn_readfirstlane((t0 - win.tb) / TILE_STEP);
      if (k - win.kw >= 64) {
        // t0 <= last here (the loop loads only while a tile of the chunk
        // remains), so every clamped index below is a valid token
        const int t = win.tb + TILE_STEP * (k + (int)(threadIdx.x & 63));
        win.lo = ptab[min(t, last) >> pshift];
        if (page_size == 8) win.hi = ptab[min(t + 8, last) >> 3];
        win.kw = k;
      }
      P.lo = __builtin_amdgcn_readlane(win.lo, k - win.kw);
      P.hi = page_size == 8 ? __builtin_amdgcn_readlane(win.hi, k - win.kw) : P.lo;
    }
    return P;
  }

  // row index (relative to row0) of token t of the tile whose pages are P
  __device__ __forceinline__ RowT row_of(int t, const TilePages &P) const {
    t = min(t, last);
    if constexpr (PAGED) {
      // a token past the end clamps to the last one, whose page is lo or hi
      // by its own position (or both, for a tile wholly past the end).  A
      // mask select: a select of the two fields compiles to an indexed load
      // from a stack copy of P, whose wait would drain the tile's loads.
      const uint32_t m = 0u - ((uint32_t)t >> 3 & 1u);
      const size_t pg = (size_t)(((uint32_t)P.lo & ~m) | ((uint32_t)P.hi & m));
      return (pg * h_kv + kvh) * page_size + (t & (page_size - 1));
    } else {
      return (RowT)t;
    }
  }

  __device__ __forceinline__ void load(TileRegs &T, int t0, bool exact, bool wit, bool vrec) const {
    const TilePages P = tile_pages(t0);
    load_keys(T, t0, exact, P);
    load_rest(T, t0, wit, vrec, P);
  }

  // stored and exact keys with the key scale (what the logits need first)
  __device__ __forceinline__ void load_keys(TileRegs &T, int t0, bool exact, const TilePages &P) const {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j16 = lane & 15, pp = lane & 3;
    const RowT ra = row_of(t0 + j16, P), rk = row_of(t0 + 4 * g + pp, P);
    if constexpr (KF == KVQ_FMT_FP8_E4M3 || KF == KVQ_FMT_INT8_DITHER) {
      const uint4 *p = reinterpret_cast<const uint4 *>(kb + ra * D + 32 * g);
      T.k[0] = p[0];
      T.k[1] = p[1];
      T.ks = KF == KVQ_FMT_FP8_E4M3 ? ksb[rk] : 1.0f;   // INT8: block scales ride on q
    } else if constexpr (KF == KVQ_FMT_INT8_G32) {
      // slice s of this lane: channels 32 s + 8 g .. + 7, so that one
      // contraction covers one scale group
      const uint8_t *p = kb + ra * D + 8 * g;
      const uint2 a0 = *reinterpret_cast<const uint2 *>(p), a1 = *reinterpret_cast<const uint2 *>(p + 32);
      const uint2 a2 = *reinterpret_cast<const uint2 *>(p + 64), a3 = *reinterpret_cast<const uint2 *>(p + 96);
      T.k[0] = uint4{a0.x, a0.y, a1.x, a1.y};
      T.k[1] = uint4{a2.x, a2.y, a3.x, a3.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) T.kg[e] = *reinterpret_cast<const uint2 *>(ksg + row_of(t0 + 4 * g + e, P) * 4);
      T.ks = 1.0f;
      if (n_op > 0) {
        // values 8 g + 2 i, 8 g + 2 i + 1 (a pair's two channels) as one word;
        // rows are 4 n_op bytes, so every word is aligned
        const uint32_t *p = reinterpret_cast<const uint32_t *>(kob + ra * (2 * n_op) + 8 * g);
        const int nw = n_op - 4 * g;                     // words of this lane's 4 that exist
        T.ko.x = nw > 0 ? p[0] : 0u;
        T.ko.y = nw > 1 ? p[1] : 0u;
        T.ko.z = nw > 2 ? p[2] : 0u;
        T.ko.w = nw > 3 ? p[3] : 0u;
      }
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
  __device__ __forceinline__ void load_rest(TileRegs &T, int t0, bool wit, bool vrec, const TilePages &P) const {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j16 = lane & 15, pp = lane & 3;
    const RowT ra = row_of(t0 + j16, P), rk = row_of(t0 + 4 * g + pp, P);
    if (wit) T.wit = *reinterpret_cast<const uint2 *>(wb + ra * NB + 4 * g);
    if (vrec) T.vrec = *reinterpret_cast<const uint32_t *>(vwb + rk * 2);
    if constexpr (VF == KVQ_FMT_FP8_E4M3 || VF == KVQ_FMT_INT8_DITHER || VF == KVQ_FMT_INT8_G32) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const RowT re = row_of(t0 + 4 * g + e, P);
        T.v8[e] = *reinterpret_cast<const uint2 *>(vbb + re * D + 8 * j16);
        if constexpr (VF == KVQ_FMT_INT8_G32) T.vg[e] = vsg[re * 4 + (j16 >> 2)];
      }
      T.vs = VF == KVQ_FMT_FP8_E4M3 ? vsb[rk] : 1.0f;
    } else if constexpr (VF == KVQ_FMT_BF16) {
      // the FP8 layout at two bytes a value: 16 lanes read one 256-byte row
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const RowT re = row_of(t0 + 4 * g + e, P);
        T.vb[e] = *reinterpret_cast<const uint4 *>(vbb + re * (2 * D) + 16 * j16);
      }
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
// EXT: Tier B, the value side, the two-sided form and the block report are
// compiled in (they are tested at run time); without it the tile loop has
// none of their code.
template <int KF, int VF, bool PAGED, bool FULL, bool SPILL_LDS, bool EXT = false>
__device__ __forceinline__ void mfma_chunk(const DecodeLaunch &d, int b, int kvh, int grp, int qh0, int c0,
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
  // Tier B (WitCert Sec. 4.2): zb accumulates p~ e^{u} on the attention's
  // maximum.  tb_l = log(2 S / delta) with S the request's tokens (both
  // regions); eub = e^{u} of this lane's head, constant over a 256-token
  // block of INT8 keys and 1 for keys stored as BF16 (u = 0).
  // (the team launch never takes Tier B or the block report: SPILL_LDS
  // compiles them out of its kernel)
  const bool do_b = EXT && !SPILL_LDS && d.has_tier_b != 0;
  // value side (WitCert Sec. 3 output bound): zv accumulates p~ rho on the
  // attention maximum, vmax the largest ||v|| of the chunk's tokens
  const bool do_v = EXT && d.has_value != 0;
  // two-sided form (WitCert Prop. 1): a running state over l~ - c for A-
  const bool do_n = EXT && d.has_two_sided != 0;
  // block report: spill (l~, l) and c of every token-head, the Tier B radius
  // of every INT8 block
  const bool do_r = EXT && !SPILL_LDS && d.has_report != 0;
  float tb_l = 0.0f, eub = 1.0f;
  if (do_b) {
    const int sl = d.suffix_cap > 0
                       ? (d.suffix_lengths ? min(max(d.suffix_lengths[b], 0), d.suffix_cap) : d.suffix_cap)
                       : 0;
    tb_l = logf(2.0f * (float)(d.prefix_len + sl)) + d.tier_b_log_inv_delta;
  }

  // The wavefront's first tile is requested ahead of the query work below,
  // so that its loads and q's travel together (with INT8 block scales the
  // loop loads its first tile after the block's operands).
  // (A short-lived source serves that load, so that the loop's own source,
  // built below, is not live across the query work.)
  constexpr bool BLOCK_LOOP = KF == KVQ_FMT_INT8_DITHER || VF == KVQ_FMT_INT8_DITHER;
  static_assert(!(PAGED && BLOCK_LOOP), "block-scale INT8 regions are never paged");
  TileRegs ta, tb;
  typename TileSrc<KF, VF, PAGED>::WinT win0{};    // (paged: the page window it fetched)
  if constexpr (!BLOCK_LOOP && !SPILL_LDS) {
    const TileSrc<KF, VF, PAGED> first(d, b, kvh, c0, c1);
    if (c0 + 16 * wv < c1) first.load(ta, c0 + 16 * wv, do_tv && has_exact, do_meter && has_wit, do_v);
    win0 = first.win;
  }

  // ---- B operands of the logit contractions, column j16 = 4 hh + pp (a
  //      group of 1 or 2 query heads pads the tile with copies of its last
  //      head, whose results are not written)
  bf16x8_t bq[4];
  f16x4_t bw;
  const float *qp = d.q + ((size_t)b * d.h_q + (size_t)kvh * d.qg + min(qh0 + hh, d.qg - 1)) * D;
  // Every q value of this lane: dims 32 g .. 32 g + 31 (the split) and the
  // dims of bands 4 g .. 4 g + 3 (the witness factors: 4 k .. 4 k + 3 and
  // 64 + 4 k .. 64 + 4 k + 3 for band k).  A chunk's launch requests them
  // all before any is used (with its first tile, above), so the prologue
  // costs one round trip.
  //
  // The team launch (SPILL_LDS) keeps each q element's load next to its
  // split, where the select of the split's piece makes the loads run one
  // after another, and loads its first tile in the loop: its round prologue
  // then lasts as long as the memory system takes to answer, which keeps
  // the two work-groups of a CU taking turns at streaming (about one
  // streaming work-group per CU, HBM steady near 5.9 TB/s).  Measured on the
  // batch-64 x 12,628-token layer, issuing the loads together lets the
  // teams' rounds fall into step instead: all work-groups stream at once and
  // then all exchange at once, and the launch is 2.5% slower (0.657 against
  // 0.641 ms); a fixed pause in its place is slower still.
  float4 qa[8], qband[8];
  if constexpr (!SPILL_LDS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) qa[i] = reinterpret_cast<const float4 *>(qp + 32 * g)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qband[2 * e] = *reinterpret_cast<const float4 *>(qp + 4 * (4 * g + e));
      qband[2 * e + 1] = *reinterpret_cast<const float4 *>(qp + 64 + 4 * (4 * g + e));
    }
  }
  {
    const float *qf = reinterpret_cast<const float *>(qa);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {                 // exact: each piece is a bf16 value
        if constexpr (SPILL_LDS) {
          const float x = mul_rn(qp[32 * g + 8 * s + e], qs);
          const float hi = bf16_round(x);
          const float mid = bf16_round(x - hi);
          const float lo = bf16_round(x - hi - mid);
          bq[s][e] = (__bf16)(pp == 0 ? hi : (pp == 1 ? mid : (pp == 2 ? lo : 0.0f)));
        } else {
          bq[s][e] = (__bf16)split3_piece(mul_rn(qf[8 * s + e], qs), pp);
        }
      }
    }
    // witness dot: the raised band factors of head hh (bands 4 g .. 4 g + 3
    // in this lane) as two fp16 pieces h1 + h2 >= the factor (h1 to nearest,
    // h2 the fp32-exact remainder rounded up), in columns pp = 0 and 1.  A
    // factor at or beyond 2^15, past what the fp16 operand holds, is an
    // overflow: its piece is +inf, so every c of that head is +inf (or NaN
    // where the band's witness is 0), which the finalize reports as the
    // trivial bound (WitCert Sec. 3 numerics: +inf on overflow, c never
    // truncated).  (Scaling the factors instead would keep a scale factor
    // live through the tile loop, which measurably slows it.)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma clang fp contract(off)                         // (f rounded: r below is exact)
      const float f = SPILL_LDS ? band_factor_up(qp, 4 * g + e, d.c_factor)
                                : band_factor_up(qband[2 * e], qband[2 * e + 1], d.c_factor);
      const bool ok = f < 32768.0f;                  // (inputs are finite)
      const _Float16 h1n = (_Float16)f;
      const float r = f - (float)h1n;                 // exact
      const _Float16 h2n = (_Float16)r;
      const uint16_t u = __builtin_bit_cast(uint16_t, h2n);   // next fp16 toward +inf if below
      const uint16_t up = (u & 0x7fffu) == 0u ? (uint16_t)1u : (uint16_t)((u & 0x8000u) ? u - 1u : u + 1u);
      const _Float16 h1 = ok ? h1n : __builtin_bit_cast(_Float16, (uint16_t)0x7c00u);
      const _Float16 h2 = ok ? __builtin_bit_cast(_Float16, (float)h2n < r ? up : u) : (_Float16)0.0f;
      bw[e] = pp == 0 ? h1 : (pp == 1 ? h2 : (_Float16)0.0f);
    }
  }

  // INT8 (subtractive dither): x^ = s_c (code - xi) with s_c per 256-token
  // block and channel.  The logits take the block's scales on the query side:
  // bqs = exact three-way bf16 split of q_c s_c (log2 units), against the
  // codes and the two pieces of -xi.  Values are dequantized to fp16.
  constexpr bool I8K = KF == KVQ_FMT_INT8_DITHER;
  constexpr bool I8V = VF == KVQ_FMT_INT8_DITHER;
  // INT8 with per-(token, 32-channel group) scales: the logits contract one
  // group per MFMA (bqs = exact three-way split of q_c in log2 units over
  // channels 32 s + 8 g ..) and scale the four partial sums per token; values
  // are dequantized to fp16 with their token's group scale.
  constexpr bool GK = KF == KVQ_FMT_INT8_G32;
  constexpr bool GV = VF == KVQ_FMT_INT8_G32;
  bf16x8_t bqs[4];
  float sv8[8];                                    // value scales of dims 8 j16 + n
  uint32_t i8_stream = 0, i8_tag = 0;
  size_t i8_scale_row0 = 0;
  if constexpr (I8K || I8V || GK || GV) {
    const size_t sh = R.is_prefix ? (size_t)kvh : (size_t)b * d.h_kv + kvh;
    i8_scale_row0 = sh * (size_t)((R.length + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK);
    i8_stream = (uint32_t)(R.is_prefix ? R.stream_id : (R.stream_ids ? R.stream_ids[b] : R.stream_id + b));
    i8_tag = dither_tag(R.layer, kvh);             // (keys and values share a token's dither)
  }
  // Dithered INT8 keys and values: the key phase of a tile computes each
  // generator call once and leaves the tile's 16 x 128 dithers in this
  // wavefront's LDS tile, where the value phase reads its own (token,
  // channel) set (the two phases hold transposed sets per lane).  The per-tile
  // wavefront barriers order the writes before the reads and the reads before
  // the next tile's writes.
  constexpr bool SHARE_XI = I8K && I8V;
  float (*xi_s)[XI_ROW] = nullptr;
  if constexpr (SHARE_XI) {
    __shared__ __attribute__((aligned(16))) float xi_tile[WAVES][16][XI_ROW];
    xi_s = xi_tile[wv];
  }
  auto set_block = [&](int blk) {
    const size_t srow = (i8_scale_row0 + (size_t)blk) * D;
    if constexpr (I8K) {
      const uint16_t *ks = (const uint16_t *)R.k_scale + srow;
      // the block's scales and q (dims 32 g .. 32 g + 31), all loads first
      uint4 sc[4];
      float4 qv[8];
#pragma unroll
      for (int s8 = 0; s8 < 4; ++s8) sc[s8] = *reinterpret_cast<const uint4 *>(ks + 32 * g + 8 * s8);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = reinterpret_cast<const float4 *>(qp + 32 * g)[i];
      const float *qf = reinterpret_cast<const float *>(qv);
      float ss = 0.0f;                             // sum of (q_c s_c)^2 in log2 units
#pragma unroll
      for (int s8 = 0; s8 < 4; ++s8) {
        const uint32_t sw[4] = {sc[s8].x, sc[s8].y, sc[s8].z, sc[s8].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = mul_rn(mul_rn(qf[8 * s8 + e], qs), fp16_bits_to_f32((sw[e >> 1] >> (16 * (e & 1))) & 0xffffu));
          ss = fmaf(x, x, ss);
          bqs[s8][e] = (__bf16)split3_piece(x, pp);
        }
      }
      if (do_b) {
        // lanes 16 g + 4 hh + pp hold channels 32 g .. 32 g + 31 of head hh;
        // u log2(e) = sqrt(2 var log(2S/delta)) log2(e) = sqrt(ss tb_l / 6)
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float ub = sqrtf(ss * tb_l * (1.0f / 6.0f));
        eub = exp2f(ub);
        if (do_r && g == 0 && pp == 0) {
          float *up = d.ublk + ((size_t)grp * d.n_blocks + (R.is_prefix ? 0 : d.pre_blocks) + blk) * G + hh;
          if (d.total_chunks > 1)
            st_dev(up, ub);
          else
            *up = ub;
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

  // fixed outlier pairs (WitCert Sec. 6.2.5): their channels leave the
  // group contractions (q zeroed there) and enter one more contraction
  // against the stored exact values (bqo: q at the channels of values
  // 8 g .. 8 g + 7, three-way split by column)
  float qg2[4] = {0.0f, 0.0f, 0.0f, 0.0f};         // group sums of (q_c qs)^2 of head hh
  bf16x8_t bqo;
  const int n_op = R.n_op;
  if constexpr (GK) {
    uint32_t bm0 = 0, bm1 = 0;                       // bypassed pairs 0..31, 32..63
    if (n_op > 0) {
      const int32_t *opp = R.opairs + (size_t)kvh * n_op;
      for (int i = 0; i < n_op; ++i) {
        const int P = opp[i];
        if (P >= 0 && P < 32) bm0 |= 1u << P;
        if (P >= 32 && P < 64) bm1 |= 1u << (P - 32);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 8 * g + e, slot = k >> 1;
        float x = 0.0f;
        if (k < 2 * n_op) {
          const int P = opp[slot];
          bool act = P >= 0 && P < 64;
          for (int i = 0; i < slot; ++i) act = act && opp[i] != P;
          if (act) x = mul_rn(qp[P + 64 * (k & 1)], qs);
        }
        bqo[e] = (__bf16)split3_piece(x, pp);
      }
    }
    // q at channels 32 s8 + 8 g .. + 7, all loads first
    float4 qv[8];
#pragma unroll
    for (int s8 = 0; s8 < 4; ++s8) {
      qv[2 * s8] = *reinterpret_cast<const float4 *>(qp + 32 * s8 + 8 * g);
      qv[2 * s8 + 1] = *reinterpret_cast<const float4 *>(qp + 32 * s8 + 8 * g + 4);
    }
    const float *qf = reinterpret_cast<const float *>(qv);
#pragma unroll
    for (int s8 = 0; s8 < 4; ++s8) {
      // channels 32 s8 + 8 g + e: pair (32 s8 + 8 g + e) mod 64
      const uint32_t bw_ = (s8 & 1) ? bm1 : bm0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool byp = (bw_ >> (8 * g + e)) & 1u;
        const float x = byp ? 0.0f : mul_rn(qf[8 * s8 + e], qs);
        qg2[s8] = fmaf(x, x, qg2[s8]);
        bqs[s8][e] = (__bf16)split3_piece(x, pp);
      }
      qg2[s8] += __shfl_xor(qg2[s8], 16);
      qg2[s8] += __shfl_xor(qg2[s8], 32);
    }
  }

  const TileSrc<KF, VF, PAGED> src(d, b, kvh, c0, c1);
  if constexpr (!BLOCK_LOOP && !SPILL_LDS) src.win = win0;
  auto load_tile = [&](TileRegs &T, int t0) { src.load(T, t0, do_tv && has_exact, do_meter && has_wit, do_v); };
  float *spill_g = ((do_tv || do_r) && !SPILL_LDS) ? spill_region<G>(d, grp, R.is_prefix != 0) : nullptr;
  float *rspill_g = do_r ? rspill_region<G>(d, grp, R.is_prefix != 0) : nullptr;

  // per-lane accumulator states (lane = one (token slot, head) pair)
  float mq = NEG_INF, zq = 0.0f;     // attention softmax, maximum uniform per head
  float mm = NEG_INF, zm = 0.0f;     // l~ + c (Theorem 1's A)
  float me = NEG_INF, ze = 0.0f;     // exact logits (TV normalizer)
  float zb = 0.0f;                   // Tier B: sum p~ e^u on the attention maximum
  float zv = 0.0f, vmax = 0.0f;      // value side: sum p~ rho, max ||v||
  float mn = NEG_INF, zn = 0.0f;     // l~ - c (Prop. 1's A-)
  float cmax = 0.0f;                 // max c (the tanh shape)
  // Values: output in MFMA accumulators, N-tile n, lane j16 = dims 8 j16 + n,
  // register r = head r (lanes 0..15).
  f32x4_t ov[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) ov[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

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
        float xi[8];
        dither8((uint32_t)(t0 + j16), (uint32_t)(8 * g + 2 * s), i8_tag, i8_stream, R.seed_lo, R.seed_hi, xi);
        if constexpr (SHARE_XI) {
          float4 *dst = reinterpret_cast<float4 *>(&xi_s[j16][32 * g + 8 * s]);
          dst[0] = make_float4(xi[0], xi[1], xi[2], xi[3]);
          dst[1] = make_float4(xi[4], xi[5], xi[6], xi[7]);
        }
        bf16x8_t xh, xl;
        neg_split8_bf16(xi, xh, xl);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cw), bqs[s], dq, 0, 0, 0);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bqs[s], dq, 0, 0, 0);
        dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bqs[s], dq, 0, 0, 0);
      }
    } else if constexpr (GK) {
      // row j16 = token t0 + j16, slice s = scale group s (channels 32 s + 8 g ..)
      const uint32_t w[8] = {T.k[0].x, T.k[0].y, T.k[0].z, T.k[0].w,
                             T.k[1].x, T.k[1].y, T.k[1].z, T.k[1].w};
      f32x4_t ds[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 cw = {i8x2_to_bf16x2(w[2 * s], 0), i8x2_to_bf16x2(w[2 * s], 2),
                          i8x2_to_bf16x2(w[2 * s + 1], 0), i8x2_to_bf16x2(w[2 * s + 1], 2)};
        float xi[8];
        dither8((uint32_t)(t0 + j16), (uint32_t)(8 * s + 2 * g), i8_tag, i8_stream, R.seed_lo, R.seed_hi, xi);
        bf16x8_t xh, xl;
        neg_split8_bf16(xi, xh, xl);
        ds[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cw), bqs[s], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f},
                                                      0, 0, 0);
        ds[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bqs[s], ds[s], 0, 0, 0);
        ds[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bqs[s], ds[s], 0, 0, 0);
      }
      // output row r = token t0 + 4 g + r: its four group scales; Tier B's
      // sum_s s_s^2 qg2_s of the same token
      float ssr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 sw = T.kg[r];
        const float s0 = fp16_bits_to_f32(sw.x & 0xffffu), s1 = fp16_bits_to_f32(sw.x >> 16);
        const float s2 = fp16_bits_to_f32(sw.y & 0xffffu), s3 = fp16_bits_to_f32(sw.y >> 16);
        dq[r] = s0 * ds[0][r];
        dq[r] = fmaf(s1, ds[1][r], dq[r]);
        dq[r] = fmaf(s2, ds[2][r], dq[r]);
        dq[r] = fmaf(s3, ds[3][r], dq[r]);
        float ss = s0 * s0 * qg2[0];
        ss = fmaf(s1 * s1, qg2[1], ss);
        ss = fmaf(s2 * s2, qg2[2], ss);
        ssr[r] = fmaf(s3 * s3, qg2[3], ss);
      }
      if (n_op > 0) {                                // the bypassed channels, exact
        const f32x4_t dov = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.ko), bqo,
                                                                    f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[r] += dov[r];
      }
      if (do_b) {
        // this lane's token t0 + 4 g + pp: u log2(e) = sqrt(sum_s s_s^2 qg2_s tb_l / 6)
        const float a01 = (pp & 1) ? ssr[1] : ssr[0];
        const float a23 = (pp & 1) ? ssr[3] : ssr[2];
        eub = exp2f(sqrtf(((pp & 2) ? a23 : a01) * tb_l * (1.0f / 6.0f)));
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
      if ((do_tv || do_r) && valid)
        st_pair(spill_g + 2 * ((size_t)64 * (t0 >> 4) + lane), lq, le, d.total_chunks > 1);
      if (do_r && valid) {
        float *rp = rspill_g + (size_t)64 * (t0 >> 4) + lane;
        if (d.total_chunks > 1)
          st_dev(rp, cc);
        else
          *rp = cc;
      }
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
      zb *= f;
      zv *= f;
      float fh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) fh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 4 * h));
      if constexpr (VF != VF_NONE) {               // MFMA accumulators
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[n][r] *= fh[r];
      }
      mq = mnew;
    }
    const float p = valid ? fast_exp2(lq - mq) : 0.0f;
    zq += p;
    if (do_b) zb = fmaf(p, eub, zb);
    if (do_v) {
      zv = fmaf(p, fp16_bits_to_f32(T.vrec & 0xffffu), zv);
      if (valid) vmax = fmaxf(vmax, fp16_bits_to_f32(T.vrec >> 16));
    }
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
    if (do_n) {
      const float y = lq - cc;
      if (y > mn + LAZY) {
        zn *= merge_factor(mn, y);
        mn = y;
      }
      zn += valid ? fast_exp2(y - mn) : 0.0f;
      if (valid) cmax = fmaxf(cmax, cc);
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
    } else if constexpr (I8V || GV) {
      // as FP8, with weights p and values s (code - xi) in fp16 (s: the block's
      // scale of the channel, or the token's scale of the channel's group)
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
        if constexpr (SHARE_XI) {                  // left by this tile's key phase
          const float4 *src = reinterpret_cast<const float4 *>(&xi_s[4 * g + e][8 * j16]);
          const float4 a = src[0], c = src[1];
          xi[0] = a.x; xi[1] = a.y; xi[2] = a.z; xi[3] = a.w;
          xi[4] = c.x; xi[5] = c.y; xi[6] = c.z; xi[7] = c.w;
        } else {
          dither8((uint32_t)(t0 + 4 * g + e), (uint32_t)(2 * j16), i8_tag, i8_stream, R.seed_lo, R.seed_hi, xi);
        }
        const uint32_t cw[2] = {T.v8[e].x, T.v8[e].y};
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float code = (float)(int)(int8_t)(cw[n >> 2] >> (8 * (n & 3)));
          const float sc = GV ? fp16_bits_to_f32(T.vg[e]) : sv8[n];
          vb[n][e] = (_Float16)(sc * (code - xi[n]));
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) ov[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(aw, vb[n], ov[n], 0, 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    } else if constexpr (VF == KVQ_FMT_BF16) {
      // weights as for FP8 values, split into two bf16 pieces hi + lo (exact
      // to 2^-16 of p) along the contraction: K element i < 4 pairs piece hi
      // of token 4 g + i with its value, i >= 4 piece lo with the same value,
      // so one 16x16x32 product per N-tile adds (hi + lo) v; the bf16 values
      // enter exactly and the products accumulate in fp32
      w_s[wv][16 * hh + 4 * g + pp] = p;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4 wa = *reinterpret_cast<const float4 *>(&w_s[wv][16 * (j16 & 3) + 4 * g]);
      const bool arow = j16 < 4;
      const float w4[4] = {arow ? wa.x : 0.0f, arow ? wa.y : 0.0f, arow ? wa.z : 0.0f, arow ? wa.w : 0.0f};
      bf16x8_t aw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hi = bf16_hw_round(w4[i]);
        aw[i] = (__bf16)hi;
        aw[4 + i] = (__bf16)(w4[i] - hi);              // (w - hi exact in fp32)
      }
      const uint32_t rw[4][4] = {{T.vb[0].x, T.vb[0].y, T.vb[0].z, T.vb[0].w},
                                 {T.vb[1].x, T.vb[1].y, T.vb[1].z, T.vb[1].w},
                                 {T.vb[2].x, T.vb[2].y, T.vb[2].z, T.vb[2].w},
                                 {T.vb[3].x, T.vb[3].y, T.vb[3].z, T.vb[3].w}};
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        // dim 8 j16 + n of tokens 4 g .. 4 g + 3: half n & 1 of word n >> 1
        const int k = n >> 1;
        const uint32_t v01 = (n & 1) ? ((rw[0][k] >> 16) | (rw[1][k] & 0xffff0000u))
                                     : ((rw[0][k] & 0xffffu) | (rw[1][k] << 16));
        const uint32_t v23 = (n & 1) ? ((rw[2][k] >> 16) | (rw[3][k] & 0xffff0000u))
                                     : ((rw[2][k] & 0xffffu) | (rw[3][k] << 16));
        ov[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, as_bf16x8(uint4{v01, v23, v01, v23}), ov[n], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  };

  // two register sets (ta, tb), no copies: the loads of one tile overlap the
  // other's math.  The next tile is always loaded (rows clamp to the last
  // valid token, so past the end this re-reads a valid row and the data is
  // unused).
  if constexpr (BLOCK_LOOP) {
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
    constexpr int STEP = TILE_STEP;
    int t0 = c0 + 16 * wv;                      // (a chunk's first tile is loaded above)
    if constexpr (SPILL_LDS) {
      if (t0 < c1) load_tile(ta, t0);
    }
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
    if (do_b) zb += __shfl_xor(zb, off);
    if (do_v) {
      zv += __shfl_xor(zv, off);
      vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
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
    if (do_n) {
      const float m2 = __shfl_xor(mn, off), z2 = __shfl_xor(zn, off);
      const float m = fmaxf(mn, m2);
      zn = zn * merge_factor(mn, m) + z2 * merge_factor(m2, m);
      mn = m;
      cmax = fmaxf(cmax, __shfl_xor(cmax, off));
    }
  }
  if (lane < 16 && pp == 0) {                      // lane 4h holds head h
    part_s[wv][hh][0] = mq; part_s[wv][hh][1] = zq;
    part_s[wv][hh][2] = mm; part_s[wv][hh][3] = zm;
    part_s[wv][hh][4] = me; part_s[wv][hh][5] = ze;
    part_s[wv][hh][6] = zb;
    part_s[wv][hh][7] = zv;
    part_s[wv][hh][PART_VMAX] = vmax;
    part_s[wv][hh][PART_MN] = mn;
    part_s[wv][hh][PART_ZN] = zn;
    part_s[wv][hh][PART_CMAX] = cmax;
  }
  if constexpr (VF != VF_NONE) {                  // MFMA accumulators
    if (lane < 16) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) part_s[wv][r][8 + 8 * lane + n] = ov[n][r];
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

// One work-group's share of the per-chunk plan: chunk `chunk_idx` of group
// grp = (request, KV head) in the region d.region, then the chunk epilogue.
template <int KF, int VF, bool PAGED, bool FULL, bool EXT>
__device__ __forceinline__ void chunk_work(const DecodeLaunch &d, int grp, int chunk_idx, float (*w_s)[64],
                                           float (*part_s)[4][PART_STRIDE]) {
  const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;
  const RegionDev &R = d.region;
  const int len = R.is_prefix ? R.length : (R.lengths ? min(max(R.lengths[b], 0), R.length) : R.length);
  const int c0 = chunk_idx * d.chunk;
  const int c1 = min(c0 + d.chunk, len);
  mfma_chunk<KF, VF, PAGED, FULL, false, EXT>(d, b, kvh, grp, d.qh0, c0, c1, nullptr, w_s, part_s);
  chunk_epilogue<4>(d, part_s, grp, chunk_idx, b, kvh);
}

}  // namespace kvq
