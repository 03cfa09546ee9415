// Device helpers shared by the write-path and decode kernels (gfx950).
//
// Number formats, the Philox4x32-10 generator and 8-lane DPP reductions.  The
// formats follow their published definitions; see include/kvq.h for the
// citations of where each enters the method.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int D = 128;          // head dimension
constexpr int NB = 16;          // witness bands (WitCert Sec. 4.1, system value B = 16)
constexpr int BLK = 256;        // INT8 scale block (WitCert Sec. 6.1.1)
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 / fp16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f32_to_fp16_bits_rne(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// Smallest fp16 >= w for finite w >= 0 (+inf above 65504).  Comparisons are
// exact in double; the starting guess only needs to be within one step.
__device__ __forceinline__ uint32_t fp16_round_up_bits(double w) {
  if (!(w > 0.0)) return 0u;
  if (w > 65504.0) return 0x7c00u;
  uint32_t h = f32_to_fp16_bits_rne((float)w);
  if (h > 0x7bffu) h = 0x7bffu;
  // step down while the previous value is still >= w, then up while below w
  while (h > 0u && (double)fp16_bits_to_f32(h - 1u) >= w) --h;
  while ((double)fp16_bits_to_f32(h) < w) ++h;
  return h;
}

// ---------------------------------------------------------------- FP8 E4M3FN

// Encode a finite float already clamped to [-448, 448]: nearest, ties to even
// code, sign bit copied (so -0.0 -> 0x80).  Integer logic, no hardware mode.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  float af = __uint_as_float(a);
  uint32_t mag;
  if (af < 0.015625f) {                        // below 2^-6: multiples of 2^-9
    mag = (uint32_t)rintf(af * 512.0f);        // exact scaling, RNE; 8 -> 2^-6 = code 8
  } else {
    // keep 3 mantissa bits with round-to-nearest-even on the dropped 20 bits;
    // the carry propagates into the exponent field by itself
    mag = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | mag;
}

// Decode one E4M3FN byte in software (exact; NaN codes are never produced).
__device__ __forceinline__ float e4m3_decode_sw(uint32_t c) {
  uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// Hardware decode of bytes 0,1 (hi = false) or 2,3 (hi = true) of a dword.
// gfx950 interprets these conversions as OCP E4M3FN.
template <bool HI>
__device__ __forceinline__ void e4m3x2(uint32_t w, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  a = v[0];
  b = v[1];
}

__device__ __forceinline__ void e4m3x4(uint32_t w, float* f) {
  e4m3x2<false>(w, f[0], f[1]);
  e4m3x2<true>(w, f[2], f[3]);
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
// (SC 2011): two 32x32->64 products per round, key advanced by the Weyl
// constants between rounds, ten rounds.  Each round's two three-input XORs
// are one instruction each (v_bitop3_b32 with truth table 0x96 = a ^ b ^ c).

struct u4 { uint32_t x, y, z, w; };

__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u4 philox4x32_10(u4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    u4 n;
    n.x = xor3((uint32_t)(p1 >> 32), c.y, k0);
    n.y = (uint32_t)p1;
    n.z = xor3((uint32_t)(p0 >> 32), c.w, k1);
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Dither for channels 4g..4g+3 of one token: counter (token, g, tag, stream),
// tag = (layer << 16) | kv_head; xi = (u >> 8) 2^-24 - 1/2.  The counter is
// the pages' five-tuple (request stream, layer, KV head, token, channel),
// which has no key/value component: a token's keys and values share their
// dither (WitCert Sec. 6.3.1, the write kernel's counter).
__device__ __forceinline__ void dither4(uint32_t token, uint32_t g, uint32_t tag, uint32_t stream,
                                        uint32_t k0, uint32_t k1, float* xi) {
  u4 o = philox4x32_10(u4{token, g, tag, stream}, k0, k1);
  xi[0] = (float)(o.x >> 8) * 5.9604644775390625e-08f - 0.5f;
  xi[1] = (float)(o.y >> 8) * 5.9604644775390625e-08f - 0.5f;
  xi[2] = (float)(o.z >> 8) * 5.9604644775390625e-08f - 0.5f;
  xi[3] = (float)(o.w >> 8) * 5.9604644775390625e-08f - 0.5f;
}

__device__ __forceinline__ uint32_t dither_tag(int layer, int kv_head) {
  return ((uint32_t)layer << 16) | (uint32_t)kv_head;
}

// ---------------------------------------------------------------- lane exchange

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8 lanes

// Sum over the 8 lanes of an aligned lane octet; every lane of the octet gets
// the bitwise-identical total (the three steps pair operands symmetrically).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  x += dpp<DPP_QUAD_XOR2>(x);
  x += dpp<DPP_QUAD_XOR1>(x);
  return x;
}

__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_QUAD_XOR2>(x));
  x = fmaxf(x, dpp<DPP_QUAD_XOR1>(x));
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace kvq
