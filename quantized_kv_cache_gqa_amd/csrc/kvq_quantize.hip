// Write path: quantize exact keys / values into the stored formats and store the
// band-norm witness of the keys.
//
// FP8 per-token and BF16 targets: one wavefront per (sequence, KV head, token);
// lane l owns channels l and l + 64, i.e. RoPE pair l under the rotate-half
// pairing, so band b (pairs 4b..4b+3) lives in lanes 4b..4b+3.
// Dithered INT8: one work-group per (sequence, KV head, 256-token block): the
// per-channel block absmax is reduced through LDS, then every (token, channel
// group of 4) draws one Philox4x32-10 block and encodes four channels.
//
// Witness (WitCert Sec. 4.1, Eq. (2)): residuals r = x^ - x are exact in
// float64; each band's squares are summed in coordinate order (4b..4b+3, then
// 64+4b..64+4b+3) with one rounding per operation, square-rooted, multiplied by
// 1 + 2^-48 and rounded up to fp16, so the stored value bounds the exact norm.
//
// Value records (WitCert Sec. 3, the output bound's two norms): per token,
// rho = ||v^ - v|| and ||v||, each summed in float64 over channels 0..127 in
// order, square-rooted, inflated and rounded up the same way.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ float load_in(const void *p, size_t idx, int in_fmt) {
  if (in_fmt == KVQ_FMT_FP32) return reinterpret_cast<const float *>(p)[idx];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[idx] << 16);
}

// Band norm of 8 float64 residuals held in LDS, in the stated order.
__device__ __forceinline__ uint32_t band_witness(const double *r, int b) {
#pragma clang fp contract(off)
  double acc = r[4 * b] * r[4 * b];
  for (int i = 1; i < 4; ++i) {
    double t = r[4 * b + i] * r[4 * b + i];
    acc = acc + t;
  }
  for (int i = 0; i < 4; ++i) {
    double t = r[64 + 4 * b + i] * r[64 + 4 * b + i];
    acc = acc + t;
  }
  double w = sqrt(acc);
  w = w * (1.0 + 0x1p-48);
  return fp16_round_up_bits(w);
}

// Norm of 128 float64 values held in LDS, summed in channel order.
__device__ __forceinline__ uint32_t full_norm_up(const double *x) {
#pragma clang fp contract(off)
  double acc = x[0] * x[0];
  for (int c = 1; c < D; ++c) {
    double t = x[c] * x[c];
    acc = acc + t;
  }
  double w = sqrt(acc);
  w = w * (1.0 + 0x1p-48);
  return fp16_round_up_bits(w);
}

// One wavefront per token; handles FP8 per-token, BF16 and INT8 with
// per-(token, 32-channel group) scales: lanes 0..31 hold group 0 (channels
// 0..31) and group 2 (64..95), lanes 32..63 groups 1 and 3; the dither is the
// block format's (the same Philox counters), so the codes differ from it only
// through the scales.
__global__ __launch_bounds__(256) void quant_token_kernel(
    const void *__restrict__ in, int in_fmt, int target, int n_seq, int h_kv, int capacity,
    int tok_begin, int tok_end, uint8_t *__restrict__ out, void *__restrict__ scale_out,
    uint16_t *__restrict__ wit_out, uint16_t *__restrict__ vrec_out, uint32_t k0, uint32_t k1,
    int layer, int stream_id, const int32_t *__restrict__ stream_ids, const int32_t *__restrict__ opairs,
    int n_op, uint16_t *__restrict__ kout) {
#pragma clang fp contract(off)
  __shared__ double rbuf[4][D];
  __shared__ double xbuf[4][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ntok = tok_end - tok_begin;
  const long gtok = (long)blockIdx.x * 4 + wv;           // over n_seq * h_kv * ntok
  const long total = (long)n_seq * h_kv * ntok;
  if (gtok >= total) return;                             // whole wavefront exits together
  const long sh = gtok / ntok;                           // (seq, kv head)
  const int t = tok_begin + (int)(gtok - sh * ntok);
  const size_t row = (size_t)sh * capacity + t;

  float x0 = load_in(in, row * D + lane, in_fmt);
  float x1 = load_in(in, row * D + lane + 64, in_fmt);
  double h0, h1;                                         // reconstructed values
  if (target == KVQ_FMT_FP8_E4M3) {
    float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    float s = amax / 448.0f;                             // correctly rounded
    if (amax == 0.0f) s = 1.0f;
    float y0 = fminf(fmaxf(x0 / s, -448.0f), 448.0f);
    float y1 = fminf(fmaxf(x1 / s, -448.0f), 448.0f);
    uint32_t c0 = e4m3_encode(y0), c1 = e4m3_encode(y1);
    out[row * D + lane] = (uint8_t)c0;
    out[row * D + lane + 64] = (uint8_t)c1;
    if (lane == 0) reinterpret_cast<float *>(scale_out)[row] = s;
    h0 = (double)e4m3_decode_sw(c0) * (double)s;
    h1 = (double)e4m3_decode_sw(c1) * (double)s;
  } else if (target == KVQ_FMT_INT8_G32) {
    const int seq = (int)(sh / h_kv), kvh = (int)(sh - (long)seq * h_kv);
    // fixed outlier pairs (WitCert Sec. 6.2.5): pair `lane` (channels lane and
    // lane + 64) is bypassed when a slot names it; it keeps its bf16 value,
    // gets code 0 and leaves the group maximum
    int oslot = -1;
    if (n_op > 0) {
      const int32_t *pp = opairs + (size_t)kvh * n_op;
      for (int i = n_op - 1; i >= 0; --i)
        if (pp[i] == lane) oslot = i;                    // the first slot naming the pair
      uint16_t *orow = kout + row * (size_t)(2 * n_op);
      if (lane < n_op) {                                 // slots that bypass nothing hold 0
        const int P = pp[lane];
        bool act = P >= 0 && P < 64;
        for (int i = 0; i < lane; ++i) act = act && pp[i] != P;
        if (!act) {
          orow[2 * lane] = 0;
          orow[2 * lane + 1] = 0;
        }
      }
      if (oslot >= 0) {
        orow[2 * oslot] = (uint16_t)(__float_as_uint(x0) >> 16);   // bf16 input: exact
        orow[2 * oslot + 1] = (uint16_t)(__float_as_uint(x1) >> 16);
      }
    }
    const bool byp = oslot >= 0;
    float a0 = byp ? 0.0f : fabsf(x0), a1 = byp ? 0.0f : fabsf(x1);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {             // maxima over each half-wavefront
      a0 = fmaxf(a0, __shfl_xor(a0, off));
      a1 = fmaxf(a1, __shfl_xor(a1, off));
    }
    const uint32_t s0b = f32_to_fp16_bits_rne(a0 / 126.5f), s1b = f32_to_fp16_bits_rne(a1 / 126.5f);
    const float s0 = fp16_bits_to_f32(s0b), s1 = fp16_bits_to_f32(s1b);
    uint16_t *sc = reinterpret_cast<uint16_t *>(scale_out) + row * 4;
    if ((lane & 31) == 0) {
      sc[lane >> 5] = (uint16_t)s0b;
      sc[2 + (lane >> 5)] = (uint16_t)s1b;
    }
    const uint32_t tag = dither_tag(layer, kvh);
    const uint32_t stream = (uint32_t)(stream_ids ? stream_ids[seq] : stream_id + seq);
    float xa[4], xb[4];
    dither4((uint32_t)t, (uint32_t)(lane >> 2), tag, stream, k0, k1, xa);
    dither4((uint32_t)t, (uint32_t)((lane + 64) >> 2), tag, stream, k0, k1, xb);
    const float xi0 = xa[lane & 3], xi1 = xb[lane & 3];
    float c0 = 0.0f, c1 = 0.0f;
    if (s0 != 0.0f) {
      float y = x0 / s0;                                 // correctly rounded
      float z = y + xi0;
      c0 = fminf(fmaxf(rintf(z), -127.0f), 127.0f);
    }
    if (s1 != 0.0f) {
      float y = x1 / s1;
      float z = y + xi1;
      c1 = fminf(fmaxf(rintf(z), -127.0f), 127.0f);
    }
    if (byp) c0 = c1 = 0.0f;
    out[row * D + lane] = (uint8_t)(int8_t)(int)c0;
    out[row * D + lane + 64] = (uint8_t)(int8_t)(int)c1;
    h0 = s0 != 0.0f ? (double)s0 * ((double)c0 - (double)xi0) : 0.0;
    h1 = s1 != 0.0f ? (double)s1 * ((double)c1 - (double)xi1) : 0.0;
    if (byp) {
      h0 = (double)x0;
      h1 = (double)x1;
    }
  } else {                                               // BF16 target
    uint32_t b0 = in_fmt == KVQ_FMT_FP32 ? f32_to_bf16_bits(x0) : (__float_as_uint(x0) >> 16);
    uint32_t b1 = in_fmt == KVQ_FMT_FP32 ? f32_to_bf16_bits(x1) : (__float_as_uint(x1) >> 16);
    uint16_t *o16 = reinterpret_cast<uint16_t *>(out);
    o16[row * D + lane] = (uint16_t)b0;
    o16[row * D + lane + 64] = (uint16_t)b1;
    h0 = (double)__uint_as_float(b0 << 16);
    h1 = (double)__uint_as_float(b1 << 16);
  }
  if (wit_out) {
    rbuf[wv][lane] = h0 - (double)x0;
    rbuf[wv][lane + 64] = h1 - (double)x1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < NB) wit_out[row * NB + lane] = (uint16_t)band_witness(rbuf[wv], lane);
  }
  if (vrec_out) {                                        // values: (rho, ||v||)
    rbuf[wv][lane] = h0 - (double)x0;
    rbuf[wv][lane + 64] = h1 - (double)x1;
    xbuf[wv][lane] = (double)x0;
    xbuf[wv][lane + 64] = (double)x1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < 2) vrec_out[row * 2 + lane] = (uint16_t)full_norm_up(lane == 0 ? rbuf[wv] : xbuf[wv]);
  }
}

// One work-group per (sequence, KV head, 256-token block): dithered INT8.
__global__ __launch_bounds__(256) void quant_int8_block_kernel(
    const void *__restrict__ in, int in_fmt, int n_seq, int h_kv, int capacity,
    int blk_begin, int n_blk, int tok_end, int8_t *__restrict__ out,
    uint16_t *__restrict__ scale_out, uint16_t *__restrict__ wit_out, uint32_t k0, uint32_t k1,
    int layer, int stream_id, const int32_t *__restrict__ stream_ids, uint16_t *__restrict__ vrec_out) {
#pragma clang fp contract(off)
  __shared__ float amax_s[2][D];
  __shared__ float scale_s[D];
  __shared__ double rbuf[8][D];
  __shared__ double xbuf[8][D];
  const int tid = threadIdx.x;
  const int sh = blockIdx.x / n_blk;                     // (seq, kv head)
  const int blk = blk_begin + (int)(blockIdx.x - sh * n_blk);
  const int seq = sh / h_kv, kvh = sh - (sh / h_kv) * h_kv;
  const int t0 = blk * BLK;
  const int nt = min(BLK, tok_end - t0);
  const size_t base = (size_t)sh * capacity;
  const int nblk_cap = (capacity + BLK - 1) / BLK;

  {  // per-channel absmax over the block
    const int c = tid & (D - 1), half = tid >> 7;
    float m = 0.0f;
    for (int i = half; i < nt; i += 2) m = fmaxf(m, fabsf(load_in(in, (base + t0 + i) * D + c, in_fmt)));
    amax_s[half][c] = m;
  }
  __syncthreads();
  if (tid < D) {
    float amax = fmaxf(amax_s[0][tid], amax_s[1][tid]);
    float s32 = amax / 126.5f;                           // correctly rounded
    uint32_t s16 = f32_to_fp16_bits_rne(s32);
    scale_out[((size_t)sh * nblk_cap + blk) * D + tid] = (uint16_t)s16;
    scale_s[tid] = fp16_bits_to_f32(s16);
  }
  __syncthreads();

  const uint32_t tag = dither_tag(layer, kvh);
  const uint32_t stream = (uint32_t)(stream_ids ? stream_ids[seq] : stream_id + seq);
  const int g = tid & 31;                                // channel group: channels 4g..4g+3
  const int ti = tid >> 5;                               // token within a group of 8
  for (int i0 = 0; i0 < nt; i0 += 8) {
    const int i = i0 + ti;
    if (i < nt) {
      const int t = t0 + i;
      float xi[4];
      dither4((uint32_t)t, (uint32_t)g, tag, stream, k0, k1, xi);
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 4 * g + e;
        float x = load_in(in, (base + t) * D + c, in_fmt);
        float s = scale_s[c];
        float code = 0.0f;
        if (s != 0.0f) {
          float y = x / s;                               // correctly rounded
          float z = y + xi[e];
          code = fminf(fmaxf(rintf(z), -127.0f), 127.0f);
        }
        word |= ((uint32_t)(int)code & 0xffu) << (8 * e);
        if (wit_out || vrec_out) {
          double xh = (s != 0.0f) ? (double)s * ((double)code - (double)xi[e]) : 0.0;
          rbuf[ti][c] = xh - (double)x;
          xbuf[ti][c] = (double)x;
        }
      }
      *reinterpret_cast<uint32_t *>(out + (base + t) * D + 4 * g) = word;
    }
    if (wit_out || vrec_out) {
      __syncthreads();
      if (wit_out && tid < 128) {
        const int tt = tid >> 4, b = tid & 15;
        if (i0 + tt < nt) wit_out[(base + t0 + i0 + tt) * NB + b] = (uint16_t)band_witness(rbuf[tt], b);
      }
      if (vrec_out && tid >= 128 && tid < 144) {
        const int tt = (tid - 128) >> 1, col = tid & 1;
        if (i0 + tt < nt)
          vrec_out[(base + t0 + i0 + tt) * 2 + col] = (uint16_t)full_norm_up(col == 0 ? rbuf[tt] : xbuf[tt]);
      }
      __syncthreads();
    }
  }
}

static hipError_t launch_one(const QuantLaunch &q, int which, hipStream_t stream) {
  const int fmt = which == 0 ? q.k_format : q.v_format;
  const void *in = which == 0 ? q.k_in : q.v_in;
  void *out = which == 0 ? q.k_out : q.v_out;
  void *sc = which == 0 ? q.k_scale_out : q.v_scale_out;
  uint16_t *wit = which == 0 ? q.witness_out : nullptr;
  uint16_t *vrec = which == 1 ? q.v_witness_out : nullptr;
  const int ntok = q.tok_end - q.tok_begin;
  if (ntok <= 0) return hipSuccess;
  if (fmt == KVQ_FMT_INT8_DITHER) {   // block scales (G32 takes the per-token kernel)
    const int blk_begin = q.tok_begin / BLK;
    const int n_blk = (q.tok_end - 1) / BLK - blk_begin + 1;
    const long grid = (long)q.n_seq * q.h_kv * n_blk;
    hipLaunchKernelGGL(quant_int8_block_kernel, dim3((unsigned)grid), dim3(256), 0, stream, in,
                       q.in_format, q.n_seq, q.h_kv, q.capacity, blk_begin, n_blk, q.tok_end,
                       (int8_t *)out, (uint16_t *)sc, wit, (uint32_t)q.seed,
                       (uint32_t)(q.seed >> 32), q.layer, q.stream_id, q.stream_ids, vrec);
  } else {
    const long total = (long)q.n_seq * q.h_kv * ntok;
    const long grid = (total + 3) / 4;
    hipLaunchKernelGGL(quant_token_kernel, dim3((unsigned)grid), dim3(256), 0, stream, in,
                       q.in_format, fmt, q.n_seq, q.h_kv, q.capacity, q.tok_begin, q.tok_end,
                       (uint8_t *)out, sc, wit, vrec, (uint32_t)q.seed, (uint32_t)(q.seed >> 32),
                       q.layer, q.stream_id, q.stream_ids, which == 0 ? q.opairs : nullptr,
                       which == 0 ? q.n_op : 0, which == 0 ? q.k_outliers_out : nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t stream) {
  hipError_t e = launch_one(q, 0, stream);
  if (e != hipSuccess) return e;
  if (q.v_in) e = launch_one(q, 1, stream);
  return e;
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream) {
  size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (uint32_t *)ptr, n);
  return hipGetLastError();
}

}  // namespace kvq
