// Read path, one launch over both regions (the cartridge page: one kernel
// spans the shared cartridge and each request's live suffix).  Per (request,
// KV head), chunks [0, n1) walk the prefix and chunks [n1, n1 + n2) the
// suffix, each with its own formats and layout; the last arriving chunk of the
// group merges both regions in chunk order, exactly as when each region has a
// launch of its own, so the results are bitwise the same.
#include <hip/hip_runtime.h>


#include "kvq_decode_mfma.h"

namespace kvq {

template <int KF, int VF1, int VF2, bool PAGED2, bool FULL, bool EXT>
__global__ __launch_bounds__(256, 2) void decode_two_kernel(const DecodeLaunch d1, const DecodeLaunch d2) {
  const unsigned per_xcd = gridDim.x >> 3;
  const unsigned L = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  const unsigned nc = (unsigned)(d1.n_chunks + d2.n_chunks);
  if (L >= (unsigned)d1.batch * d1.h_kv * nc) return;
  __shared__ __attribute__((aligned(16))) float w_s[WAVES][64];
  __shared__ float part_s[WAVES][4][PART_STRIDE];
  // Groups in KV-head-major order: consecutive logical indices, which stay
  // on one XCD, take one KV head across requests, so each XCD's L2 serves
  // its heads' slice of the shared cartridge to every request, and the
  // cartridge is fetched from HBM about once instead of once per XCD.
  const int gi = (int)(L / nc), ci = (int)(L % nc);
  const int grp = (gi % d1.batch) * d1.h_kv + gi / d1.batch;
  if (ci < d1.n_chunks)
    chunk_work<KF, VF1, false, FULL, EXT>(d1, grp, ci, w_s, part_s);
  else
    chunk_work<KF, VF2, PAGED2, FULL, EXT>(d2, grp, ci - d1.n_chunks, w_s, part_s);
}

namespace {

bool full_region(const DecodeLaunch &d) {
  return d.has_tv && d.has_meter && d.region.exact_fmt == EX_BF16 && d.region.witness;
}

template <int KF, int VF1, int VF2, bool PAGED2>
hipError_t launch_2(const DecodeLaunch &d1, const DecodeLaunch &d2, hipStream_t s) {
  const long work = (long)d1.batch * d1.h_kv * (d1.n_chunks + d2.n_chunks);
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
  // FULL = false is exact for every case (it tests the flags at run time)
  constexpr bool F8 = KF == KVQ_FMT_FP8_E4M3;
  const bool full = F8 && full_region(d1) && full_region(d2);
  if (launch_has_extensions(d1)) {
    if (full)
      hipLaunchKernelGGL((decode_two_kernel<KF, VF1, VF2, PAGED2, F8, true>), grid, dim3(256), 0, s, d1, d2);
    else
      hipLaunchKernelGGL((decode_two_kernel<KF, VF1, VF2, PAGED2, false, true>), grid, dim3(256), 0, s, d1, d2);
  } else {
    if (full)
      hipLaunchKernelGGL((decode_two_kernel<KF, VF1, VF2, PAGED2, F8, false>), grid, dim3(256), 0, s, d1, d2);
    else
      hipLaunchKernelGGL((decode_two_kernel<KF, VF1, VF2, PAGED2, false, false>), grid, dim3(256), 0, s, d1, d2);
  }
  return hipGetLastError();
}

template <int KF, int VF1, int VF2>
hipError_t launch_2p(const DecodeLaunch &d1, const DecodeLaunch &d2, hipStream_t s) {
  return d2.region.paged ? launch_2<KF, VF1, VF2, true>(d1, d2, s) : launch_2<KF, VF1, VF2, false>(d1, d2, s);
}

}  // namespace

// The fused launch covers keys of one format (BF16 or FP8) in both regions;
// with BF16 keys any mix of BF16 and FP8 values, with FP8 keys the same value
// format in both; the meter-only call (no values) either way.
bool two_region_supported(const DecodeLaunch &d1, const DecodeLaunch &d2) {
  if (d1.plan_flags & (KVQ_PLAN_LAUNCH_PER_REGION | KVQ_PLAN_VECTOR_ALU)) return false;
  if (!mfma_path_supports(d1) || !mfma_path_supports(d2) || d1.region.paged) return false;
  if (d1.k_format != d2.k_format) return false;
  const int v1 = d1.v_format, v2 = d2.v_format;
  if ((v1 == VF_NONE) != (v2 == VF_NONE)) return false;
  if (d1.k_format == KVQ_FMT_BF16) return true;
  return d1.k_format == KVQ_FMT_FP8_E4M3 && v1 == v2;
}

hipError_t launch_decode_two(const DecodeLaunch &d1, const DecodeLaunch &d2, hipStream_t s) {
  constexpr int B = KVQ_FMT_BF16, F = KVQ_FMT_FP8_E4M3, N = VF_NONE;
  const int v1 = d1.v_format, v2 = d2.v_format;
  if (d1.k_format == B) {
    if (v1 == N) return launch_2p<B, N, N>(d1, d2, s);
    if (v1 == B) return v2 == B ? launch_2p<B, B, B>(d1, d2, s) : launch_2p<B, B, F>(d1, d2, s);
    return v2 == B ? launch_2p<B, F, B>(d1, d2, s) : launch_2p<B, F, F>(d1, d2, s);
  }
  if (v1 == N) return launch_2p<F, N, N>(d1, d2, s);
  return v1 == B ? launch_2p<F, B, B>(d1, d2, s) : launch_2p<F, F, F>(d1, d2, s);
}

}  // namespace kvq
