// Read path, matrix-core kernels for GQA group 4 (the tile loop and its
// operand layouts are described in kvq_decode_mfma.h): the per-chunk kernel of
// one region, and the persistent team kernel of the single-region TV case.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "kvq_decode_mfma.h"

namespace kvq {

template <int KF, int VF, bool PAGED, bool FULL, bool EXT>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(const DecodeLaunch d) {
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const unsigned n_work = (unsigned)d.batch * d.h_kv * d.n_chunks;
  if (L >= n_work) return;
  __shared__ __attribute__((aligned(16))) float w_s[WAVES][64];
  __shared__ float part_s[WAVES][4][PART_STRIDE];
  chunk_work<KF, VF, PAGED, FULL, EXT>(d, (int)(L / (unsigned)d.n_chunks), (int)(L % (unsigned)d.n_chunks), w_s,
                                  part_s);
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
// Slot of one member: per head SLOT_ST words (the six states M~, Z~, M, Z,
// M_e, Z_e; then, with the meter extensions, z_v, max ||v||, M-, Z-, max c),
// 4 TV shares, 512 accumulator words.
constexpr int SLOT_ST = 11;
constexpr int SLOT_TV = 4 * SLOT_ST, SLOT_ACC = SLOT_TV + 4;
constexpr int SLOT_WORDS = SLOT_ACC + 512;
static_assert(SLOT_WORDS * 8 == (int)TEAM_SLOT_BYTES, "team slot size");

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

// EXT: the value side and the two-sided form (with the tanh shape) ride on
// the exchange: z_v merges like Z~, (M-, Z-) like (M, Z), the maxima by max.
template <bool EXT>
__device__ __forceinline__ void team_epilogue(const DecodeLaunch &d, uint32_t epoch, float (*part_s)[4][PART_STRIDE],
                              const float2 *spill_s, int team, int slot_team, int qh0, int member,
                              int round, bool last_round, int b, int kvh, int c0, int c1) {
  constexpr int G = 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int T = d.team;
  const bool do_tv = d.has_tv != 0;
  const bool do_meter = d.has_meter != 0;
  // the exchange is the round's critical path: its waves issue ahead of the
  // co-resident work-group's streaming waves (wave priority only)
  __builtin_amdgcn_s_setprio(1);
  const uint32_t tag = team_tag(epoch + (uint32_t)round + 1u);   // round - 1's is tag - 1
  uint64_t *slots = reinterpret_cast<uint64_t *>(d.partials) + (size_t)(slot_team * 2 + (round & 1)) * T * SLOT_WORDS;
  uint64_t *mine = slots + (size_t)member * SLOT_WORDS;
  __shared__ float mq_s[G][64];
  __shared__ float unit_s[WAVES][64];
  __shared__ float fin_s[G][4];
  __shared__ float tvw_s[WAVES][G];
  __shared__ int bad_s;    // this round's group: a wait ran out, its results are NaN
  __shared__ int late_s;   // any wait of this epilogue ran out (reported in the status word)
  const float qnan = __builtin_nanf("");

  // 1. publish this member's merged states and accumulator
  if (tid == 0) bad_s = late_s = 0;
  __syncthreads();
  for (int idx = tid; idx < G * PART_STRIDE; idx += 256) {
    const int h = idx / PART_STRIDE, k = idx - h * PART_STRIDE;
    int word, mk;                                   // slot word; sum merged on field mk's maximum (-1: a maximum)
    if (k < 6) {
      word = SLOT_ST * h + k;
      mk = (k & 1) ? k - 1 : -1;
    } else if (k >= 8 && k < 8 + D) {
      word = SLOT_ACC + 128 * h + (k - 8);
      mk = 0;
    } else if (EXT && k == 7) {
      word = SLOT_ST * h + 6;
      mk = 0;
    } else if (EXT && k >= PART_VMAX && k <= PART_CMAX) {
      word = SLOT_ST * h + 7 + (k - PART_VMAX);
      mk = k == PART_ZN ? PART_MN : -1;
    } else {
      continue;
    }
    float r;
    if (mk < 0) {
      r = part_s[0][h][k];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) r = fmaxf(r, part_s[w][h][k]);
    } else {
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) M = fmaxf(M, part_s[w][h][mk]);
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) r += part_s[w][h][k] * merge_factor(part_s[w][h][mk], M);
    }
    if (member != d.silent_member)                 // (a test hook silences one member)
      st_tagged(mine + word, tag, r);
  }

  // 2. the group's normalizers: wavefront h reads head h of every member
  //    (lane c = member c), then a butterfly merge over the lowest
  //    ceil(log2 T) lane bits leaves the group's states in lane 0
  const int h = __builtin_amdgcn_readfirstlane(wv);   // uniform: scalar slot bases
  bool ok = true;
  float Mq = NEG_INF, Zq = 0.0f, Mm = NEG_INF, Zm = 0.0f, Me = NEG_INF, Ze = 0.0f;
  float Zv = 0.0f, Vm = 0.0f, Mn = NEG_INF, Zn = 0.0f, Cm = 0.0f;
  if (lane < T) {
    constexpr int NS = EXT ? SLOT_ST : 6;
    const uint64_t *s = slots + (size_t)lane * SLOT_WORDS + SLOT_ST * h;
    const uint64_t *p[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) p[i] = s + i;
    float v[NS];
    ok = read_tagged<NS>(p, tag, v, d.spin_limit);
    Mq = v[0]; Zq = v[1]; Mm = v[2]; Zm = v[3]; Me = v[4]; Ze = v[5];
    if constexpr (EXT) {
      Zv = v[6]; Vm = v[7]; Mn = v[8]; Zn = v[9]; Cm = v[10];
    }
  }
  // one member's words missing makes the whole group's states unknown: NaN
  // then flows into every result of the group (never a stale value)
  ok = __all(ok);
  if (!ok) {
    const float qnan_s = __builtin_nanf("");
    Mq = Zq = Mm = Zm = Me = Ze = qnan_s;
    Zv = Vm = Mn = Zn = Cm = qnan_s;
    if (lane == 0) bad_s = late_s = 1;
  }
  mq_s[h][lane] = Mq;
  for (int off = 1; off < T; off <<= 1) {           // lanes >= T hold empty states
    const float a0 = __shfl_xor(Mq, off), a1 = __shfl_xor(Zq, off);
    const float b0 = __shfl_xor(Mm, off), b1 = __shfl_xor(Zm, off);
    const float e0 = __shfl_xor(Me, off), e1 = __shfl_xor(Ze, off);
    if constexpr (EXT) {
      const float v1 = __shfl_xor(Zv, off), vm = __shfl_xor(Vm, off);
      const float n0 = __shfl_xor(Mn, off), n1 = __shfl_xor(Zn, off), cm = __shfl_xor(Cm, off);
      const float mx = fmaxf(Mq, a0);                // z_v rides on the attention maximum
      Zv = Zv * merge_factor(Mq, mx) + v1 * merge_factor(a0, mx);
      Vm = fmaxf(Vm, vm);
      mz_merge(Mn, Zn, n0, n1);
      Cm = fmaxf(Cm, cm);
    }
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
  const size_t qh = (size_t)b * d.h_q + (size_t)kvh * d.qg + qh0 + h;
  const bool hv = qh0 + h < d.qg;                 // a query head (not a padding head)
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
                            (size_t)(slot_team * 2 + ((round - 1) & 1)) * T * SLOT_WORDS +
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
      const size_t qu = (size_t)b * d.h_q + (size_t)kvh * d.qg + qh0 + hu;
      if (split) {
        unit_s[h][lane] = o;
        if (!oku) bad_s = late_s = 1;
      } else {
        if (qh0 + hu < d.qg) d.out[qu * D + dim] = oku ? o * iZu : qnan;
        ok = ok && oku;
      }
    }
    if (split && member < 8) {                     // uniform over the work-group
      __syncthreads();
      if (h == 0) {
        const int hu = member >> 1, dim = 64 * (member & 1) + lane;
        const float o = ((unit_s[0][lane] + unit_s[1][lane]) + unit_s[2][lane]) + unit_s[3][lane];
        const size_t qu = (size_t)b * d.h_q + (size_t)kvh * d.qg + qh0 + hu;
        if (qh0 + hu < d.qg) d.out[qu * D + dim] = bad_s == 0 ? o * fin_s[hu][1] : qnan;
      }
    }
  }
  if (member == h % T && lane == 0) {
    const double log_a = do_meter ? meter_log_a(Mq, Zq, Mm, Zm) : 0.0;
    const double bound = 0.5 * expm1(2.0 * log_a);
    const float bf = bound > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)bound;
    if (d.log_a && hv) d.log_a[qh] = ok ? (float)log_a : qnan;
    if (d.bound_raw && hv) d.bound_raw[qh] = ok ? bf : qnan;
    if (d.meter && hv) d.meter[qh] = ok ? fminf(1.0f, bf) : qnan;
    if constexpr (EXT) {                             // as the per-chunk finalize
      if (d.has_two_sided) {
        double log_am = 0.0;
        if (Zq > 0.0f && Zn > 0.0f)
          log_am = ((double)Mn - (double)Mq) * 0.69314718055994530942 + log((double)Zn) - log((double)Zq);
        const double two = sinh(log_a - log_am);
        const float tf = two > 3.4028234663852886e38 ? __builtin_huge_valf() : (float)two;
        if (d.log_a_minus && hv) d.log_a_minus[qh] = ok ? (float)log_am : qnan;
        if (d.bound_two_sided && hv) d.bound_two_sided[qh] = ok ? tf : qnan;
        if (d.meter_two_sided && hv) d.meter_two_sided[qh] = ok ? fminf(fminf(1.0f, bf), tf) : qnan;
        if (d.bound_tanh && hv)       // (log A = +inf: an overflowed c, which a maximum skips)
          d.bound_tanh[qh] = ok ? (log_a == __builtin_huge_val() ? 1.0f : (float)tanh((double)Cm * 0.69314718055994530942))
                                : qnan;
      }
      if (d.has_value) {
        const float verr = Zq > 0.0f ? Zv / Zq : 0.0f;
        const float tvb = do_meter ? fminf(1.0f, bf) : 0.0f;
        if (d.value_err && hv) d.value_err[qh] = ok ? verr : qnan;
        if (d.v_norm_max && hv) d.v_norm_max[qh] = ok ? Vm : qnan;
        if (d.out_bound && hv) d.out_bound[qh] = ok ? 2.0f * tvb * Vm + verr : qnan;
      }
    }
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
    if (!okp && lane == 0) late_s = 1;
    const int pg = team + (round - 1) * d.n_teams;
    const int pb = pg / d.h_kv, pk = pg - pb * d.h_kv;
    if (lane == 0 && hv) d.tv[(size_t)pb * d.h_q + (size_t)pk * d.qg + qh0 + h] = okp ? 0.5f * sh : qnan;
  }
  if (!ok) bad_s = late_s = 1;
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
    if (!__all(okp) && lane == 0) late_s = 1;
    okp = __all(okp) && bad_s == 0;
    if (lane == 0 && hv) d.tv[qh] = okp ? 0.5f * sh : qnan;
  }
  __syncthreads();                  // LDS buffers are reused by the next round
  // a wait that ran out is reported to the caller, not only as NaN results
  if (tid == 0 && late_s && d.status)
    __hip_atomic_fetch_or(d.status, (uint32_t)KVQ_DEVSTATUS_TEAM_WAIT, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_setprio(0);
}

template <int KF, int VF, bool PAGED, bool FULL, bool EXT>
__global__ __launch_bounds__(256, 2) void decode_mfma_team_kernel(const DecodeLaunch d) {
  extern __shared__ __attribute__((aligned(16))) float2 spill_s[];   // d.chunk * 4 entries
  __shared__ __attribute__((aligned(16))) float w_s[WAVES][64];
  __shared__ float part_s[WAVES][4][PART_STRIDE];
  const int T = d.team;
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const int rt = (int)(L / (unsigned)T), member = (int)(L % (unsigned)T);
  // A group of 8 query heads: raw teams 2t and 2t + 1 (neighbours in L, so on
  // one XCD) take heads 0-3 and 4-7 of team t's groups in step, and the second
  // read of each tile is served by the caches rather than HBM.
  const bool pairs = d.halves == 2;
  const int team = pairs ? rt >> 1 : rt;
  const int qh0 = d.qh0 + (pairs ? 4 * (rt & 1) : 0);
  const int groups = d.batch * d.h_kv;
  const RegionDev &R = d.region;
  // this launch's epoch, kept in the workspace: round r's tag is epoch + r + 1
  __shared__ uint32_t epoch_s;
  if (threadIdx.x == 0) epoch_s = __hip_atomic_load(d.team_ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t epoch = epoch_s;
  for (int round = 0; team < d.n_teams; ++round) {  // (grid padding: member of no team)
    const int grp = team + round * d.n_teams;
    if (grp >= groups) break;
    const int b = grp / d.h_kv, kvh = grp - b * d.h_kv;
    const int len = R.is_prefix ? R.length : (R.lengths ? min(max(R.lengths[b], 0), R.length) : R.length);
    const int c0 = member * d.chunk;
    const int c1 = min(c0 + d.chunk, len);
    // (the next round's first tile is not loaded ahead: its loads would sit
    // ahead of the exchange's polls in the in-order load counter)
    mfma_chunk<KF, VF, PAGED, FULL, true, EXT>(d, b, kvh, grp, qh0, c0, c1, spill_s, w_s, part_s);
    team_epilogue<EXT>(d, epoch, part_s, spill_s, team, rt, qh0, member, round, grp + d.n_teams >= groups,
                       b, kvh, c0, c1);
  }
  // Every work-group counts itself out after reading the epoch and after its
  // own tagged stores have completed (so nothing of this launch lands after
  // the count); the last one moves the epoch past all of this launch's tags
  // and rearms the count, so the next launch on this workspace (a graph
  // replay included) waits for tags no earlier launch wrote.  When the
  // epoch restarts, that work-group first clears every word a team launch on
  // this workspace can read, so no word from before the restart carries a
  // tag that a later launch waits for.
  __shared__ int last_s;
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(d.team_ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = done == gridDim.x - 1;
  }
  __syncthreads();
  if (!last_s) return;
  const uint32_t rounds = (uint32_t)((groups + d.n_teams - 1) / d.n_teams);
  uint32_t next = epoch + rounds + 1u;
  if (next > TEAM_EPOCH_MAX) {                     // restart: the next launch may use up to 2^18 rounds
    next = 0u;
    uint4 *w = reinterpret_cast<uint4 *>(d.partials);
    const size_t n = d.team_clear_bytes / sizeof(uint4);
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) w[i] = uint4{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(d.team_ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d.team_ctl, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KF, int VF, bool PAGED>
static void launch_p(const DecodeLaunch &d, hipStream_t stream, dim3 grid) {
  const bool full = d.has_tv && d.has_meter && d.region.exact_fmt == EX_BF16 && d.region.witness;
  const bool ext = launch_has_extensions(d);
  if (full && ext)
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, true, true>), grid, dim3(256), 0, stream, d);
  else if (full)
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, true, false>), grid, dim3(256), 0, stream, d);
  else if (ext)
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, false, true>), grid, dim3(256), 0, stream, d);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, PAGED, false, false>), grid, dim3(256), 0, stream, d);
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

template <int KF, int VF, bool PAGED, bool FULL, bool EXT>
static const void *team_fn() {
  return reinterpret_cast<const void *>(&decode_mfma_team_kernel<KF, VF, PAGED, FULL, EXT>);
}

// the meter extensions come with the full meter only (TV, meter, witness)
template <int KF, int VF>
static const void *team_fn_kv(bool paged, bool full, bool ext) {
  if (ext) return paged ? team_fn<KF, VF, true, true, true>() : team_fn<KF, VF, false, true, true>();
  if (paged) return full ? team_fn<KF, VF, true, true, false>() : team_fn<KF, VF, true, false, false>();
  return full ? team_fn<KF, VF, false, true, false>() : team_fn<KF, VF, false, false, false>();
}

static const void *team_kernel(int k_format, int v_format, bool paged, bool full, bool ext) {
  if (k_format == KVQ_FMT_FP8_E4M3) {
    if (v_format == KVQ_FMT_FP8_E4M3) return team_fn_kv<KVQ_FMT_FP8_E4M3, KVQ_FMT_FP8_E4M3>(paged, full, ext);
    if (v_format == KVQ_FMT_BF16) return team_fn_kv<KVQ_FMT_FP8_E4M3, KVQ_FMT_BF16>(paged, full, ext);
    return team_fn_kv<KVQ_FMT_FP8_E4M3, VF_NONE>(paged, full, ext);
  }
  if (v_format == KVQ_FMT_FP8_E4M3) return team_fn_kv<KVQ_FMT_BF16, KVQ_FMT_FP8_E4M3>(paged, full, ext);
  if (v_format == KVQ_FMT_BF16) return team_fn_kv<KVQ_FMT_BF16, KVQ_FMT_BF16>(paged, full, ext);
  return team_fn_kv<KVQ_FMT_BF16, VF_NONE>(paged, full, ext);
}

int team_capacity(int k_format, int v_format, bool paged, bool full, bool ext) {
  // resident work-groups of the team kernel with the largest LDS chunk;
  // cached per device and kernel instance (callers on several host threads
  // may fill an entry at once: they store the same value), 0 when the device
  // cannot tell
  if (ext && !full) return 0;
  static std::atomic<int> cache[16][2][3][2][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  const int ki = k_format == KVQ_FMT_FP8_E4M3 ? 1 : 0;
  const int vi = v_format == KVQ_FMT_FP8_E4M3 ? 1 : (v_format == KVQ_FMT_BF16 ? 2 : 0);
  std::atomic<int> &c = cache[dev][ki][vi][paged ? 1 : 0][full ? 1 : 0][ext ? 1 : 0];
  const int known = c.load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, team_kernel(k_format, v_format, paged, full, ext),
                                                   256, (size_t)TEAM_MAX_CHUNK * 4 * sizeof(float2)) != hipSuccess)
    return 0;
  c.store(per_cu * cus, std::memory_order_relaxed);
  return per_cu * cus;
}

int team_capacity_max() {
  int best = 0;
  const int kfs[2] = {KVQ_FMT_FP8_E4M3, KVQ_FMT_BF16};
  const int vfs[3] = {KVQ_FMT_FP8_E4M3, KVQ_FMT_BF16, VF_NONE};
  for (int kf : kfs)
    for (int vf : vfs)
      for (int paged = 0; paged < 2; ++paged)
        for (int fe = 0; fe < 3; ++fe)                  // (full, ext): plain, full, full + extensions
          best = std::max(best, team_capacity(kf, vf, paged != 0, fe >= 1, fe == 2));
  return best;
}

hipError_t launch_decode_team(const DecodeLaunch &d, int grid, hipStream_t stream) {
  const bool full = d.has_tv && d.has_meter && d.region.exact_fmt == EX_BF16 && d.region.witness;
  const bool ext = d.has_value || d.has_two_sided;   // (Tier B and the report never plan a team)
  if (ext && !full) return hipErrorInvalidValue;
  const void *fn = team_kernel(d.k_format, d.v_format, d.region.paged != 0, full, ext);
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
  if (d.k_format == KVQ_FMT_INT8_G32)              // dense or paged, values alike (or none)
    return d.v_format == KVQ_FMT_INT8_G32 || d.v_format == VF_NONE;
  return (d.k_format == KVQ_FMT_FP8_E4M3 || d.k_format == KVQ_FMT_BF16) &&
         (d.v_format == KVQ_FMT_FP8_E4M3 || d.v_format == KVQ_FMT_BF16 || d.v_format == VF_NONE);
}

hipError_t launch_decode_mfma(const DecodeLaunch &d, hipStream_t s) {
  if (d.k_format == KVQ_FMT_INT8_G32) {
    if (d.v_format == KVQ_FMT_INT8_G32) return launch_m<KVQ_FMT_INT8_G32, KVQ_FMT_INT8_G32>(d, s);
    return launch_m<KVQ_FMT_INT8_G32, VF_NONE>(d, s);
  }
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
