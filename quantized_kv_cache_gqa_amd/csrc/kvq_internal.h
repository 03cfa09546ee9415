// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// --------------------------------------------------------------- write path

struct QuantLaunch {
  int k_format, v_format, in_format;
  const void *k_in, *v_in;
  int n_seq, h_kv, capacity, tok_begin, tok_end;
  void *k_out, *v_out, *k_scale_out, *v_scale_out;
  uint16_t *witness_out;
  uint64_t seed;
  int layer, stream_id;
  const int32_t *stream_ids;
  uint16_t *v_witness_out;  // value records (rho, ||v||) per token, nullable
  const int32_t *opairs;    // fixed outlier pairs of the keys [h_kv, n_op] (n_op > 0)
  uint16_t *k_outliers_out; // bf16 [.., capacity, 2 n_op]
  int n_op;
};

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t stream);

// --------------------------------------------------------------- read path

// Exact-key format codes seen by the kernels.
enum ExactFmt : int { EX_NONE = 0, EX_BF16 = 1, EX_F32 = 2 };
// Value format code used by the meter-only path.
constexpr int VF_NONE = 4;

struct RegionDev {
  const void *k, *v, *k_scale, *v_scale;
  const uint16_t *witness;
  const void *k_exact;
  int exact_fmt;          // ExactFmt
  int length;             // prefix length, or suffix capacity
  const int32_t *lengths; // suffix per-request lengths (nullable)
  const int32_t *page_table;
  int page_size, max_pages, paged, is_prefix;
  uint32_t seed_lo, seed_hi;
  int layer, stream_id;
  const int32_t *stream_ids;
  const uint16_t *v_witness;    // value records (rho, ||v||) per token (nullable)
  const int32_t *opairs;        // fixed outlier pairs of the keys [h_kv, n_op]
  const uint16_t *kout;         // their exact values, bf16 [.., len, 2 n_op]
  int n_op;                     // outlier pairs per KV head (0: none)
};

struct DecodeLaunch {
  int batch, h_q, h_kv, group;
  // query heads of KV head kvh in q / out / the meter arrays: kvh * qg + qh0 +
  // h for h < group (qg = group, qh0 = 0, unless a group of 8 runs as two
  // launches of 4 heads each)
  int qg, qh0;
  float sm_scale;
  float c_factor;               // sm_scale log2(e) (1 + 2^-19), rounded up to fp32 (see band_factor_up)
  const float *q;
  float *out;
  RegionDev region;
  int k_format, v_format;       // of this region (v_format = VF_NONE for the meter)
  int chunk;                    // tokens per chunk
  int n_chunks;                 // chunks of this region per (request, KV head)
  int chunk_base;               // index of this region's first chunk in the group
  int total_chunks;             // prefix + suffix chunks per (request, KV head)
  int prefix_len;               // tokens before the suffix in the logical order
  int suffix_cap;               // suffix capacity (spill rows per group = prefix_len + suffix_cap)
  const int32_t *suffix_lengths;// for the finalize (nullable: all = suffix_cap)
  int has_tv, has_meter, has_out, has_wit_any;
  float *tv, *bound_raw, *meter, *log_a;
  float *log_a_b, *bound_b_raw, *meter_b;   // Tier B outputs (nullable)
  int has_tier_b;               // Tier B requested: accumulate E_p~[e^u] (partial field 6)
  float tier_b_log_inv_delta;   // log(1 / delta_b)
  float *value_err, *v_norm_max, *out_bound;   // value side outputs (nullable)
  int has_value;                // value side requested: sum p~ rho (field 7), max ||v|| (field 136)
  float *log_a_minus, *bound_two_sided, *meter_two_sided;   // two-sided form (nullable)
  int has_two_sided;            // accumulate E_p~[e^{-c}] (fields 137, 138) and max c (field 139)
  float *bound_tanh;            // tanh(max_t c_t) (nullable)
  float *block_mass, *block_excess, *block_excess_b;   // block report outputs (nullable)
  int32_t *block_order;
  int has_report;               // spill (l~, l) and c per token-head, Tier B radius per block
  int n_blocks, pre_blocks;     // report blocks of both regions, and of the prefix
  int pre_int8, suf_int8;       // the region's keys are dithered INT8 (blocks have a radius)
  float *rspill;                // c per (group, spill entry), log2 units
  float *ublk;                  // Tier B radius per (group, block, head), log2 units
  uint32_t *counters;
  float *partials;
  float *spill;
  int team;                     // > 0: team launch, work-groups per (request, KV head)
  int n_teams;                  // teams in the grid
  int halves;                   // team launch: 2 when a group of 8 runs as pairs of raw teams
                                // (raw team 2t + h takes query heads 4h..4h+3 of team t's groups)
  // deferred finalize (per-chunk plan, several chunks per group): the
  // finalizer publishes the normalizers (M~, 1/Z~, M_e, 1/Z_e per head) and a
  // finish launch runs the TV and the block report over FIN_BLOCKS-block ranges
  int defer_tv;
  float *fin;                   // [groups][G][4]
  float *tvp;                   // [groups][fin_ranges][G] TV partial sums
  float *rkey;                  // [groups][G][n_blocks] page-in keys
  int fin_ranges;               // ranges per group
  int fin_blocks;               // 256-token blocks per group over both regions
  uint32_t *team_ctl;           // team launch: [0] epoch (round r's tag is
                                // team_tag(epoch + r + 1)), [1] work-groups finished (0 at rest)
  unsigned spin_limit;          // team launch: polls per batch of words before giving up
  int silent_member;            // team launch: member that never publishes (test builds; -1: none)
  size_t team_clear_bytes;      // team launch: bytes from `partials` that every team launch on
                                // this workspace may read; cleared when the epoch restarts
  unsigned plan_flags;          // KVQ_PLAN_* bits of the call
  uint32_t *status;             // the call's status word (KVQ_DEVSTATUS_* bits ORed in), or NULL
};

// Team exchange tags: signalling-NaN bit patterns 0x7F800000 | e with e in
// [1, 2^22), which no kernel stores as data (arithmetic yields quiet NaNs).
// A launch uses e = epoch + round + 1 for round < rounds <= 2^18 (groups are
// at most 2^18), so the epoch stays at or below TEAM_EPOCH_MAX and restarts
// from 0 once the next launch could pass 2^22 - 1.
constexpr uint32_t TEAM_TAG_BASE = 0x7F800000u;
constexpr uint32_t TEAM_EPOCH_MAX = (1u << 22) - (1u << 18) - 1u;
__host__ __device__ inline uint32_t team_tag(uint32_t e) { return TEAM_TAG_BASE | e; }

// m~, z~, m', z', m_e, z_e, z_b, z_v, acc[128], max ||v||, m-, z-, max c, 4 pad
constexpr int PART_STRIDE = 144;
constexpr int PART_VMAX = 136;
constexpr int PART_MN = 137, PART_ZN = 138, PART_CMAX = 139;
// Tier B, the value side, the two-sided form, the tanh shape or the block
// report requested: the matrix-core kernels then take their instance with
// that code compiled in
inline bool launch_has_extensions(const DecodeLaunch &d) {
  return d.has_tier_b || d.has_value || d.has_two_sided || d.has_report;
}

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream);
// The finish launch of a deferred finalize (TV and block report).
constexpr int FIN_BLOCKS = 4;
hipError_t launch_finish(const DecodeLaunch &d, hipStream_t stream);
// Matrix-core kernel for GQA group 4 with FP8/BF16 keys and values.
bool mfma_path_supports(const DecodeLaunch &d);
hipError_t launch_decode_mfma(const DecodeLaunch &d, hipStream_t stream);
hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream);
// One launch over both regions (d1: prefix, d2: suffix; same shared fields).
bool two_region_supported(const DecodeLaunch &d1, const DecodeLaunch &d2);
hipError_t launch_decode_two(const DecodeLaunch &d1, const DecodeLaunch &d2, hipStream_t stream);

// Team launch (matrix-core path, one region, TV requested): chunk <=
// TEAM_MAX_CHUNK tokens per member, each kept in LDS; at most TEAM_MAX
// members; TEAM_SLOT_BYTES of workspace per member and round parity.
constexpr int TEAM_MAX_CHUNK = 2048;
constexpr int TEAM_MAX = 64;
constexpr size_t TEAM_SLOT_BYTES = 560 * 8;
// Resident work-groups of the team kernel on the current device (0: no team
// launch possible).
int team_capacity(int k_format, int v_format, bool paged, bool full, bool ext);
// The largest team_capacity over every team kernel instance on the current
// device (bounds the exchange slots any team launch can use).
int team_capacity_max();
hipError_t launch_decode_team(const DecodeLaunch &d, int grid, hipStream_t stream);

}  // namespace kvq
