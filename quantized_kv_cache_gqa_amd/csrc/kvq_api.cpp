// C ABI of the library: host-side argument checks, work planning, workspace
// layout and kernel launches.  Nothing here touches device memory directly.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"

namespace {

using namespace kvq;

constexpr size_t kAlign = 256;
// Workspace layout: the team launch's control words (epoch, finished count)
// in the first 256 bytes, which no plan uses otherwise; the per-chunk plan's
// arrival counters (one per (request, KV head), at most 2^18, zero at rest)
// in the next MiB; then the team plan's exchange slots when a team plan
// exists for the arguments (whatever the plan flags and the status word),
// and after them the per-chunk plan's partials and spill.  So the two plans
// of one set of arguments never share a word, and every team word of any
// shape lies in the first 2 x (resident work-groups) slots after kTeamOff.
constexpr size_t kCtlBytes = 256;
constexpr size_t kCounterBytes = (size_t)1 << 20;
constexpr size_t kTeamOff = kCtlBytes + kCounterBytes;

// Bounded waits of the team exchange: polls per batch of words before a wait
// gives up, and a member that never publishes (none).  Only a test build
// (KVQ_TEST_HOOKS) can change them, through kvq_test_set_team_hooks, to force
// a run-out from the host.
#ifdef KVQ_TEST_HOOKS
unsigned g_spin_limit = 1u << 18;
int g_silent_member = -1;
#else
constexpr unsigned g_spin_limit = 1u << 18;
constexpr int g_silent_member = -1;
#endif

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool is_store_fmt(int f) {
  return f == KVQ_FMT_BF16 || f == KVQ_FMT_FP8_E4M3 || f == KVQ_FMT_INT8_DITHER || f == KVQ_FMT_INT8_G32;
}
inline bool is_int8(int f) { return f == KVQ_FMT_INT8_DITHER || f == KVQ_FMT_INT8_G32; }
// keys and values of a region share the per-token group layout, or neither does
inline bool g32_paired(int kf, int vf) {
  return (kf == KVQ_FMT_INT8_G32) == (vf == KVQ_FMT_INT8_G32);
}

struct Plan {
  int group = 0, chunk = 0, pre_chunks = 0, suf_chunks = 0, total_chunks = 0;
  int kgroup = 0;               // query heads per tile of the kernels: group, or 4 padding a group of 1 or 2
  int prefix_len = 0, suffix_cap = 0;
  bool tv = false, meter = false, wit_any = false, tier_b = false, value = false, two_sided = false;
  bool report = false;          // per-block risk report
  int n_blocks = 0, pre_blocks = 0;
  bool defer = false;           // per-chunk plan: TV and report in a finish launch
  int fin_blocks = 0, fin_ranges = 0;
  size_t off_fin = 0, off_tvp = 0, off_rkey = 0;
  int team = 0, n_teams = 0, grid = 0, rounds = 0;   // team launch (team > 0)
  int halves = 1;               // team launch of a group of 8: 2 = pairs of raw teams in one launch
  unsigned flags = 0;           // KVQ_PLAN_* bits of the call
  size_t team_res = 0;          // bytes of the team region (0: no team plan for these arguments)
  size_t off_counters = 0, off_partials = 0, off_spill = 0, off_rspill = 0, off_ublk = 0, bytes = 0;
};

// Team plan for a one-region launch with the TV on the matrix-core path:
// T members per (request, KV head), chunks of <= TEAM_MAX_CHUNK tokens (whole
// 16-token tiles), persistent teams over the groups.  Picks the T with the
// least work per member over all rounds (a round's fixed cost is counted as
// 256 tokens).  Returns false when the arguments admit no team launch (the
// plan flags and the status word are the caller's business).  hv = 2: a group
// of 8 as one launch of paired raw teams of 4 query heads each; hv = 1: one
// launch per 4 heads, each reading the cache.
bool plan_team(const kvq_attn_args *a, bool meter_only, int groups, Plan &p, int hv) {
  // (the kernel-group test below uses the padded group of the matrix-core
  // kernels: a group of 1 or 2 is a tile of 4)
  if (!p.tv || p.tier_b || p.report || a->split_tokens != 0 || (p.kgroup != 4 && p.group != 8)) return false;
  if ((p.prefix_len > 0) == (p.suffix_cap > 0)) return false;   // exactly one region
  const kvq_region &r = p.prefix_len > 0 ? a->prefix : a->suffix;
  if (r.k_format != KVQ_FMT_BF16 && r.k_format != KVQ_FMT_FP8_E4M3) return false;
  const int vf = meter_only ? VF_NONE : r.v_format;
  if (!meter_only && vf != KVQ_FMT_BF16 && vf != KVQ_FMT_FP8_E4M3) return false;
  if (!r.k_exact || r.k_exact_format != KVQ_FMT_BF16) return false;
  const bool full = p.tv && p.meter && r.witness;
  // the value side and the two-sided form ride on the exchange (full meter only)
  const bool ext = p.value || p.two_sided;
  if (ext && !full) return false;
  // one plan for the decode and the meter call on the same arguments (so
  // kvq_workspace_bytes fits both): the smaller capacity of the two kernels
  const bool paged = p.prefix_len == 0 && r.page_table;
  const int vf_dec = (r.v_format == KVQ_FMT_BF16 || r.v_format == KVQ_FMT_FP8_E4M3) ? r.v_format : VF_NONE;
  const int cap = std::min(team_capacity(r.k_format, VF_NONE, paged, full, ext),
                           team_capacity(r.k_format, vf_dec, paged, full, ext));
  (void)vf;
  if (cap <= 0) return false;
  if (p.group != 8) hv = 1;
  const int capg = cap / hv;                       // resident work-groups per logical team slot
  if (capg <= 0) return false;
  const int64_t len = r.length;
  const int64_t tmin = (len + TEAM_MAX_CHUNK - 1) / TEAM_MAX_CHUNK;
  const int64_t tmax = std::min<int64_t>(std::min<int64_t>(capg, TEAM_MAX), (len + 63) / 64);
  int64_t best_cost = -1;
  for (int64_t T = tmin; T <= tmax; ++T) {
    const int64_t n_teams = std::min<int64_t>(capg / T, groups);
    if (n_teams <= 0) break;
    const int64_t rounds = (groups + n_teams - 1) / n_teams;
    const int64_t chunk = ((len + T - 1) / T + 15) / 16 * 16;      // whole tiles
    const int64_t cost = rounds * (chunk + 256);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      p.team = (int)T;
      p.n_teams = (int)n_teams;
      p.chunk = (int)chunk;
    }
  }
  if (p.team <= 0) return false;
  // the grid is padded to whole XCD slices (8) and must stay resident
  while (p.n_teams > 1 && (int64_t)round_up((size_t)p.n_teams * hv * p.team, 8) > cap) --p.n_teams;
  p.grid = (int)round_up((size_t)p.n_teams * hv * p.team, 8);
  p.halves = hv;
  if (p.grid > cap) {
    p.team = 0;
    return false;
  }
  p.pre_chunks = p.prefix_len > 0 ? p.team : 0;
  p.suf_chunks = p.suffix_cap > 0 ? p.team : 0;
  p.total_chunks = p.team;
  p.rounds = (groups + p.n_teams - 1) / p.n_teams;
  p.off_counters = kCtlBytes;
  p.off_partials = kTeamOff;
  p.off_spill = p.off_partials + round_up((size_t)p.n_teams * hv * 2 * p.team * TEAM_SLOT_BYTES, kAlign);
  p.bytes = p.off_spill;
  return true;
}

kvq_status check_region(const kvq_region &r, bool is_prefix, bool need_v, int batch, int h_kv) {
  if (r.length < 0) return KVQ_ERR_SHAPE;
  if (r.length == 0) return KVQ_OK;                          // region absent
  if (r.length > (1 << 24)) return KVQ_ERR_SHAPE;           // < 2^24 tokens per request
  if (!is_store_fmt(r.k_format)) return KVQ_ERR_FORMAT;
  if (need_v && !is_store_fmt(r.v_format)) return KVQ_ERR_FORMAT;
  if (!r.k || (need_v && !r.v)) return KVQ_ERR_NULL;
  if (r.k_format != KVQ_FMT_BF16 && !r.k_scale) return KVQ_ERR_NULL;
  if (need_v && r.v_format != KVQ_FMT_BF16 && !r.v_scale) return KVQ_ERR_NULL;
  if (r.k_exact && r.k_exact_format != KVQ_FMT_BF16 && r.k_exact_format != KVQ_FMT_FP32)
    return KVQ_ERR_FORMAT;
  // fixed outlier pairs (WitCert Sec. 6.2.5): group-scale keys only
  if (r.n_outlier_pairs < 0 || r.n_outlier_pairs > 16) return KVQ_ERR_SHAPE;
  const bool op = r.n_outlier_pairs > 0;
  if (op && r.k_format != KVQ_FMT_INT8_G32) return KVQ_ERR_UNSUPPORTED;
  if (op && (!r.outlier_pairs || !r.k_outliers)) return KVQ_ERR_NULL;
  const void *ptrs[] = {r.k, need_v ? r.v : nullptr, r.k_scale, need_v ? r.v_scale : nullptr,
                        r.witness, r.k_exact, r.lengths, r.page_table, r.stream_ids, r.v_witness,
                        op ? r.outlier_pairs : nullptr, op ? r.k_outliers : nullptr};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KVQ_ERR_ALIGN;
  const bool int8 = r.k_format == KVQ_FMT_INT8_DITHER || (need_v && r.v_format == KVQ_FMT_INT8_DITHER);   // block scales
  const bool any_int8 = is_int8(r.k_format) || (need_v && is_int8(r.v_format));
  if (any_int8 && (r.layer < 0 || r.layer >= (1 << 15) || h_kv > (1 << 16))) return KVQ_ERR_SHAPE;
  if (need_v && !g32_paired(r.k_format, r.v_format)) return KVQ_ERR_UNSUPPORTED;
  if (is_prefix) {
    if (r.lengths || r.page_table || r.stream_ids) return KVQ_ERR_UNSUPPORTED;
  } else if (r.page_table) {
    if (int8) return KVQ_ERR_UNSUPPORTED;                    // 256-token blocks would span pages
    if (r.page_size != 8 && r.page_size != 16) return KVQ_ERR_UNSUPPORTED;
    if (r.max_pages <= 0 || (int64_t)r.max_pages * r.page_size != r.length) return KVQ_ERR_SHAPE;
  }
  (void)batch;
  return KVQ_OK;
}

RegionDev region_dev(const kvq_region &r, bool is_prefix);

// allow_team = false: the per-chunk plan even where a team launch applies
kvq_status make_plan(const kvq_attn_args *a, const kvq_meter_out *m, bool meter_only, Plan &p,
                     bool allow_team = true) {
  if (!a) return KVQ_ERR_NULL;
  if (a->head_dim != KVQ_HEAD_DIM) return KVQ_ERR_UNSUPPORTED;
  if (a->batch <= 0 || a->num_kv_heads <= 0 || a->num_q_heads <= 0) return KVQ_ERR_SHAPE;
  if (a->batch > (1 << 20) || a->num_q_heads > 4096) return KVQ_ERR_SHAPE;
  if (a->num_q_heads % a->num_kv_heads) return KVQ_ERR_SHAPE;
  p.group = a->num_q_heads / a->num_kv_heads;
  if (p.group != 1 && p.group != 2 && p.group != 4 && p.group != 8) return KVQ_ERR_UNSUPPORTED;
  p.kgroup = p.group;
  if (a->plan_flags & ~(uint32_t)KVQ_PLAN_ALL_FLAGS) return KVQ_ERR_UNSUPPORTED;
  p.flags = a->plan_flags;
  if (!a->q) return KVQ_ERR_NULL;
  if (!aligned16(a->q)) return KVQ_ERR_ALIGN;
  if (a->status && !aligned16(a->status)) return KVQ_ERR_ALIGN;
  if (!meter_only) {
    if (!a->out) return KVQ_ERR_NULL;
    if (!aligned16(a->out)) return KVQ_ERR_ALIGN;
  }
  if (!(a->sm_scale > 0.0f) || a->sm_scale > 1e6f) return KVQ_ERR_SHAPE;
  kvq_status s = check_region(a->prefix, true, !meter_only, a->batch, a->num_kv_heads);
  if (s != KVQ_OK) return s;
  s = check_region(a->suffix, false, !meter_only, a->batch, a->num_kv_heads);
  if (s != KVQ_OK) return s;
  p.prefix_len = a->prefix.length;
  p.suffix_cap = a->suffix.length;
  // a group of 1 or 2 query heads runs on the matrix-core kernels as a tile of
  // 4 heads (the rest copies of the last, never written) where they apply
  if ((p.group == 1 || p.group == 2) && !(p.flags & KVQ_PLAN_VECTOR_ALU)) {
    bool ok = true;
    for (int pre = 0; pre < 2; ++pre) {
      const kvq_region &r = pre ? a->prefix : a->suffix;
      if (r.length <= 0) continue;
      DecodeLaunch t;
      memset(&t, 0, sizeof(t));
      t.group = 4;
      t.region = region_dev(r, pre != 0);
      t.k_format = r.k_format;
      t.v_format = meter_only ? VF_NONE : r.v_format;
      ok = ok && mfma_path_supports(t);
    }
    if (ok) p.kgroup = 4;
  }
  if (p.prefix_len + (int64_t)p.suffix_cap <= 0) return KVQ_ERR_SHAPE;
  if (a->split_tokens < 0 || (a->split_tokens % 64) != 0) return KVQ_ERR_SHAPE;

  if ((int64_t)a->batch * a->num_kv_heads > (1 << 18)) return KVQ_ERR_SHAPE;  // counters fit 1 MiB
  const int groups = a->batch * a->num_kv_heads;
  const int smax = p.prefix_len + p.suffix_cap;
  int chunk = a->split_tokens;
  if (chunk == 0) {
    // about two resident work-groups per CU (256 CUs): as many chunks per group
    // as fill 512 work-groups, each a multiple of 64 tokens, but at least 640
    // tokens: below that the partials' merge and the short work-groups cost
    // more than the parallelism gives (measured: a 1,656-token cartridge +
    // suffix step 46.6 us with 640-token chunks, 57.9 us with 448)
    //
    // A step that would then have fewer work-groups than CUs takes chunks of
    // at least 256 tokens instead: with few work-groups each one's chain of
    // tiles sets the step's time, and more, shorter chains finish sooner
    // than the extra partials cost (measured: the single-request 696-token
    // step 15.6 us as 4 chunks, 17.6 us as 2).
    const int64_t target = 512;
    const int64_t per_group = groups >= target ? 1 : (target + groups - 1) / groups;
    int64_t c = (smax + per_group - 1) / per_group;
    c = (c + 63) / 64 * 64;
    // (Not with block-scale INT8 regions: their wavefronts take whole
    // 256-token blocks, so a 256-token chunk would keep one of four busy.)
    // (the values count for the meter call too: both calls plan one chunk)
    const bool blocks = (p.prefix_len > 0 && (a->prefix.k_format == KVQ_FMT_INT8_DITHER ||
                                              a->prefix.v_format == KVQ_FMT_INT8_DITHER)) ||
                        (p.suffix_cap > 0 && (a->suffix.k_format == KVQ_FMT_INT8_DITHER ||
                                              a->suffix.v_format == KVQ_FMT_INT8_DITHER));
    const int64_t min_chunk = (!blocks && (int64_t)groups * ((smax + 639) / 640) < 256) ? 256 : 640;
    chunk = (int)(c < min_chunk ? min_chunk : c);
  }
  p.chunk = chunk;
  p.pre_chunks = (p.prefix_len + chunk - 1) / chunk;
  p.suf_chunks = (p.suffix_cap + chunk - 1) / chunk;
  p.total_chunks = p.pre_chunks + p.suf_chunks;

  const bool any_exact = (p.prefix_len > 0 && a->prefix.k_exact) || (p.suffix_cap > 0 && a->suffix.k_exact);
  p.wit_any = (p.prefix_len > 0 && a->prefix.witness) || (p.suffix_cap > 0 && a->suffix.witness);
  if (m) {
    const void *mp[] = {m->tv, m->bound_raw, m->meter, m->log_a};
    for (const void *x : mp)
      if (x && !aligned16(x)) return KVQ_ERR_ALIGN;
    p.tv = m->tv && any_exact;
    const void *mv[] = {m->value_err, m->v_norm_max, m->out_bound};
    for (const void *x : mv)
      if (x && !aligned16(x)) return KVQ_ERR_ALIGN;
    p.value = m->value_err || m->v_norm_max || m->out_bound;
    // every region's value records for the value side
    if (p.value && p.prefix_len > 0 && !a->prefix.v_witness) return KVQ_ERR_NULL;
    if (p.value && p.suffix_cap > 0 && !a->suffix.v_witness) return KVQ_ERR_NULL;
    // Tier A (and the joint bound, which uses it): a region without a witness
    // counts as holding the exact keys (c = 0), which only keys stored as BF16
    // can; quantized keys without a witness are rejected, never metered as exact
    const void *mn[] = {m->log_a_minus, m->bound_two_sided, m->meter_two_sided, m->bound_tanh};
    for (const void *x : mn)
      if (x && !aligned16(x)) return KVQ_ERR_ALIGN;
    const bool wants_two = m->log_a_minus || m->bound_two_sided || m->meter_two_sided || m->bound_tanh;
    const bool tier_b_req = m->log_a_b || m->bound_b_raw || m->meter_b;
    // the block report (WitCert Sec. 6.3.5): Tier A's contributions need c,
    // Tier B's need the Tier B request; the order ranks Tier B when requested
    const void *mr[] = {m->block_mass, m->block_excess, m->block_excess_b, m->block_order};
    for (const void *x : mr)
      if (x && !aligned16(x)) return KVQ_ERR_ALIGN;
    p.report = m->block_mass || m->block_excess || m->block_excess_b || m->block_order;
    p.pre_blocks = (p.prefix_len + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK;
    p.n_blocks = p.pre_blocks + (p.suffix_cap + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK;
    if (m->block_excess_b && !tier_b_req) return KVQ_ERR_UNSUPPORTED;
    // Tier B's block contributions need a radius shared by the block
    const bool g32_keys = (p.prefix_len > 0 && a->prefix.k_format == KVQ_FMT_INT8_G32) ||
                          (p.suffix_cap > 0 && a->suffix.k_format == KVQ_FMT_INT8_G32);
    if (g32_keys && (m->block_excess_b || (m->block_order && tier_b_req))) return KVQ_ERR_UNSUPPORTED;
    if (m->block_order && p.n_blocks > 512) return KVQ_ERR_UNSUPPORTED;
    const bool rep_a = m->block_excess || (m->block_order && !tier_b_req);
    const bool wants_a = m->bound_raw || m->meter || m->log_a || m->out_bound || wants_two || rep_a;
    if (wants_a) {
      if (p.prefix_len > 0 && a->prefix.k_format != KVQ_FMT_BF16 && !a->prefix.witness)
        return KVQ_ERR_UNSUPPORTED;
      if (p.suffix_cap > 0 && a->suffix.k_format != KVQ_FMT_BF16 && !a->suffix.witness)
        return KVQ_ERR_UNSUPPORTED;
    }
    p.meter = wants_a && p.wit_any;
    p.two_sided = wants_two && p.wit_any;
    const void *mb[] = {m->log_a_b, m->bound_b_raw, m->meter_b};
    for (const void *x : mb)
      if (x && !aligned16(x)) return KVQ_ERR_ALIGN;
    p.tier_b = m->log_a_b || m->bound_b_raw || m->meter_b;
    if (p.tier_b) {
      // WitCert Sec. 4.2: a probability, and keys whose residual is the
      // uniform dither residual (INT8) or zero (BF16)
      if (!(m->delta_b > 0.0 && m->delta_b < 1.0)) return KVQ_ERR_SHAPE;
      if (p.prefix_len > 0 && !is_int8(a->prefix.k_format) && a->prefix.k_format != KVQ_FMT_BF16)
        return KVQ_ERR_UNSUPPORTED;
      if (p.suffix_cap > 0 && !is_int8(a->suffix.k_format) && a->suffix.k_format != KVQ_FMT_BF16)
        return KVQ_ERR_UNSUPPORTED;
    }
  }
  // The team region these arguments would use (reserved whatever the flags
  // and the status word, so that per-chunk words of these arguments never
  // land on it); the team plan itself is taken only with a status word, to
  // which a wait that runs out is reported, and when the flags allow it.
  {
    Plan t = p;
    if (plan_team(a, meter_only, groups, t, 2)) p.team_res = t.bytes - kTeamOff;
    Plan t1 = p;
    if (p.group == 8 && plan_team(a, meter_only, groups, t1, 1))
      p.team_res = std::max(p.team_res, t1.bytes - kTeamOff);
    const bool want = allow_team && a->status && !(p.flags & (KVQ_PLAN_NO_TEAM | KVQ_PLAN_VECTOR_ALU));
    Plan tp = p;
    if (want && p.team_res > 0 &&
        plan_team(a, meter_only, groups, tp, (p.flags & KVQ_PLAN_GROUP8_SEPARATE) ? 1 : 2)) {
      p = tp;
      return KVQ_OK;
    }
  }
  const int wg = std::max(p.group, p.kgroup);      // heads per group in the workspace
  p.off_counters = kCtlBytes;
  p.off_partials = round_up(kTeamOff + p.team_res, kAlign);
  p.off_spill = p.off_partials +
                round_up((size_t)groups * p.total_chunks * wg * PART_STRIDE * sizeof(float), kAlign);
  p.bytes = p.off_spill;
  // spill: each region padded to whole 16-token tiles
  const size_t spill_rows = round_up((size_t)p.prefix_len, 16) + round_up((size_t)p.suffix_cap, 16);
  if (p.tv || p.report) p.bytes += round_up((size_t)groups * spill_rows * wg * 2 * sizeof(float), kAlign);
  if (p.report) {
    // c of every token-head, and the Tier B radius of every block and head
    p.off_rspill = p.bytes;
    p.bytes += round_up((size_t)groups * spill_rows * wg * sizeof(float), kAlign);
    p.off_ublk = p.bytes;
    p.bytes += round_up((size_t)groups * p.n_blocks * wg * sizeof(float), kAlign);
  }
  // Several chunks per group: the last work-group of a group would stream the
  // whole group's spill alone for the TV and the report; a finish launch
  // spreads that over FIN_BLOCKS-block ranges instead (KVQ_PLAN_FINALIZE_IN_PLACE
  // keeps it in the decode launch).
  p.defer = p.total_chunks > 1 && (p.tv || p.report) && !(p.flags & KVQ_PLAN_FINALIZE_IN_PLACE);
  if (p.defer) {
    p.fin_blocks = (p.prefix_len + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK +
                   (p.suffix_cap + KVQ_INT8_BLOCK - 1) / KVQ_INT8_BLOCK;
    p.fin_ranges = (p.fin_blocks + FIN_BLOCKS - 1) / FIN_BLOCKS;
    if ((int64_t)groups * p.fin_ranges > ((int64_t)1 << 30)) {   // grid too large: keep the passes in place
      p.defer = false;
      p.fin_blocks = p.fin_ranges = 0;
      return KVQ_OK;
    }
    p.off_fin = p.bytes;
    p.bytes += round_up((size_t)groups * wg * 4 * sizeof(float), kAlign);
    p.off_tvp = p.bytes;
    p.bytes += round_up((size_t)groups * p.fin_ranges * wg * sizeof(float), kAlign);
    if (p.report) {
      p.off_rkey = p.bytes;
      p.bytes += round_up((size_t)groups * wg * p.fin_blocks * sizeof(float), kAlign);
    }
  }
  return KVQ_OK;
}

// The scratch of kvq_decode_attn_noalloc: one array per device, brought in
// by the code object (no allocation call).  Host code never uses the name as
// an address: it looks up the device address once per device
// (hipGetSymbolAddress, with that device current) and passes that pointer.
__device__ __align__(256) unsigned char scratch[KVQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];       // device address of `scratch`, per device

// The current device's scratch; the first call on a device looks it up and
// enqueues one fill kernel on `stream` that clears it.
kvq_status device_scratch(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_LAUNCH;
    if (launch_fill_zero(p, KVQ_SCRATCH_BYTES, stream) != hipSuccess) return KVQ_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

RegionDev region_dev(const kvq_region &r, bool is_prefix) {
  RegionDev d;
  memset(&d, 0, sizeof(d));
  d.k = r.k; d.v = r.v; d.k_scale = r.k_scale; d.v_scale = r.v_scale;
  d.witness = r.witness;
  d.k_exact = r.k_exact;
  d.exact_fmt = r.k_exact ? (r.k_exact_format == KVQ_FMT_FP32 ? EX_F32 : EX_BF16) : EX_NONE;
  d.length = r.length;
  d.lengths = is_prefix ? nullptr : r.lengths;
  d.page_table = is_prefix ? nullptr : r.page_table;
  d.page_size = r.page_size > 0 ? r.page_size : 1;
  d.max_pages = r.max_pages;
  d.paged = (!is_prefix && r.page_table) ? 1 : 0;
  d.is_prefix = is_prefix ? 1 : 0;
  d.seed_lo = (uint32_t)r.seed;
  d.seed_hi = (uint32_t)(r.seed >> 32);
  d.layer = r.layer;
  d.stream_id = r.stream_id;
  d.stream_ids = is_prefix ? nullptr : r.stream_ids;
  d.v_witness = r.v_witness;
  d.n_op = r.n_outlier_pairs > 0 ? r.n_outlier_pairs : 0;
  d.opairs = d.n_op ? r.outlier_pairs : nullptr;
  d.kout = d.n_op ? r.k_outliers : nullptr;
  return d;
}

// The per-chunk plan's launch arguments: the fields every launch shares, and
// one copy per region (dp: prefix, ds: suffix).  ws may be NULL (planning
// only: the workspace pointers are then NULL).
void chunk_launches(const kvq_attn_args *a, const kvq_meter_out *m, const Plan &p, bool meter_only,
                    void *ws, DecodeLaunch &d, DecodeLaunch &dp, DecodeLaunch &ds) {
  memset(&d, 0, sizeof(d));
  d.batch = a->batch;
  d.h_q = a->num_q_heads;
  d.h_kv = a->num_kv_heads;
  d.group = p.kgroup;
  d.qg = p.group;
  d.qh0 = 0;
  d.sm_scale = a->sm_scale;
  {
    // the factor of the witness dot's band norms, raised by 2^-19 and rounded
    // up to fp32 (its own rounding then only lifts it further)
    const double cf = (double)a->sm_scale * 1.4426950408889634074 * (1.0 + 0x1p-19);
    float f = (float)cf;
    if ((double)f < cf) f = nextafterf(f, INFINITY);
    d.c_factor = f;
  }
  d.q = a->q;
  d.out = meter_only ? nullptr : a->out;
  d.plan_flags = p.flags;
  d.status = a->status;
  d.chunk = p.chunk;
  d.total_chunks = p.total_chunks;
  d.prefix_len = p.prefix_len;
  d.suffix_cap = p.suffix_cap;
  d.suffix_lengths = p.suffix_cap > 0 ? a->suffix.lengths : nullptr;
  d.has_tv = p.tv;
  d.has_meter = p.meter;
  d.has_out = meter_only ? 0 : 1;
  d.has_wit_any = p.wit_any;
  if (m) {
    d.tv = m->tv; d.bound_raw = m->bound_raw; d.meter = m->meter; d.log_a = m->log_a;
    d.log_a_b = m->log_a_b; d.bound_b_raw = m->bound_b_raw; d.meter_b = m->meter_b;
  }
  d.has_tier_b = p.tier_b;
  if (m) {
    d.value_err = m->value_err; d.v_norm_max = m->v_norm_max; d.out_bound = m->out_bound;
  }
  d.has_value = p.value;
  if (m) {
    d.log_a_minus = m->log_a_minus; d.bound_two_sided = m->bound_two_sided;
    d.meter_two_sided = m->meter_two_sided;
    d.bound_tanh = m->bound_tanh;
  }
  d.has_two_sided = p.two_sided;
  if (m) {
    d.block_mass = m->block_mass; d.block_excess = m->block_excess;
    d.block_excess_b = m->block_excess_b; d.block_order = m->block_order;
  }
  d.has_report = p.report;
  d.n_blocks = p.n_blocks;
  d.pre_blocks = p.pre_blocks;
  d.pre_int8 = p.prefix_len > 0 && a->prefix.k_format == KVQ_FMT_INT8_DITHER;
  d.suf_int8 = p.suffix_cap > 0 && a->suffix.k_format == KVQ_FMT_INT8_DITHER;
  d.tier_b_log_inv_delta = p.tier_b ? (float)-log(m->delta_b) : 0.0f;
  if (ws) {
    char *w = static_cast<char *>(ws);
    d.counters = reinterpret_cast<uint32_t *>(w + p.off_counters);
    d.partials = reinterpret_cast<float *>(w + p.off_partials);
    d.spill = ((p.tv || p.report) && !p.team) ? reinterpret_cast<float *>(w + p.off_spill) : nullptr;
    d.rspill = p.report ? reinterpret_cast<float *>(w + p.off_rspill) : nullptr;
    d.ublk = p.report ? reinterpret_cast<float *>(w + p.off_ublk) : nullptr;
    if (p.defer) {
      d.fin = reinterpret_cast<float *>(w + p.off_fin);
      d.tvp = reinterpret_cast<float *>(w + p.off_tvp);
      d.rkey = p.report ? reinterpret_cast<float *>(w + p.off_rkey) : nullptr;
    }
  }
  d.defer_tv = p.defer ? 1 : 0;
  d.fin_blocks = p.fin_blocks;
  d.fin_ranges = p.fin_ranges;
  dp = d;
  ds = d;
  if (p.pre_chunks > 0) {
    dp.region = region_dev(a->prefix, true);
    dp.k_format = a->prefix.k_format;
    dp.v_format = meter_only ? VF_NONE : a->prefix.v_format;
    dp.n_chunks = p.pre_chunks;
    dp.chunk_base = 0;
  }
  if (p.suf_chunks > 0) {
    ds.region = region_dev(a->suffix, false);
    ds.k_format = a->suffix.k_format;
    ds.v_format = meter_only ? VF_NONE : a->suffix.v_format;
    ds.n_chunks = p.suf_chunks;
    ds.chunk_base = p.pre_chunks;
  }
}

// Launches the per-chunk plan makes: one for both regions where the kernels
// allow it (the cartridge page's one kernel over cartridge and live suffix),
// else one per region.
int chunk_launch_count(const Plan &p, const DecodeLaunch &dp, const DecodeLaunch &ds) {
  if (p.pre_chunks > 0 && p.suf_chunks > 0) return two_region_supported(dp, ds) ? 1 : 2;
  return 1;
}

// A GQA group of 8 whose regions all take the matrix-core kernels runs as two
// launch sets of 4 query heads each (the group-4 kernels; each reads the
// cache once), instead of the vector-ALU kernel.
bool split_halves(const Plan &p, const DecodeLaunch &dp, const DecodeLaunch &ds) {
  if (p.group != 8 || (p.flags & KVQ_PLAN_VECTOR_ALU)) return false;
  DecodeLaunch hp = dp, hs = ds;
  hp.group = hs.group = 4;
  if (p.pre_chunks > 0 && !mfma_path_supports(hp)) return false;
  if (p.suf_chunks > 0 && !mfma_path_supports(hs)) return false;
  return true;
}

void make_half(DecodeLaunch &x, int half) {
  x.group = 4;
  x.qh0 = 4 * half;
}

// The per-chunk plan's launches: both regions in one launch where the kernels
// allow it, else one per region; then the finish launch when deferred.
hipError_t launch_chunks(const Plan &p, const DecodeLaunch &d, const DecodeLaunch &dp, const DecodeLaunch &ds,
                         hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (chunk_launch_count(p, dp, ds) == 1 && p.pre_chunks > 0 && p.suf_chunks > 0) {
    e = launch_decode_two(dp, ds, stream);
    if (e != hipSuccess) return e;
  } else {
    if (p.pre_chunks > 0 && (e = launch_decode(dp, stream)) != hipSuccess) return e;
    if (p.suf_chunks > 0 && (e = launch_decode(ds, stream)) != hipSuccess) return e;
  }
  if (p.defer) e = launch_finish(d, stream);
  return e;
}

kvq_status run_decode(const kvq_attn_args *a, const kvq_meter_out *m, void *ws, size_t ws_bytes,
                      hipStream_t stream, bool meter_only) {
  Plan p;
  kvq_status s = make_plan(a, m, meter_only, p);
  if (s != KVQ_OK) return s;
  if (!ws) return KVQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVQ_ERR_ALIGN;
  if (ws_bytes < p.bytes) return KVQ_ERR_WORKSPACE;

  DecodeLaunch d, dp, ds;
  chunk_launches(a, m, p, meter_only, ws, d, dp, ds);
  hipError_t e = hipSuccess;
  if (p.team) {
    const bool pre = p.prefix_len > 0;
    d.region = region_dev(pre ? a->prefix : a->suffix, pre);
    d.k_format = pre ? a->prefix.k_format : a->suffix.k_format;
    d.v_format = meter_only ? VF_NONE : (pre ? a->prefix.v_format : a->suffix.v_format);
    d.n_chunks = p.team;
    d.chunk_base = 0;
    d.team = p.team;
    d.n_teams = p.n_teams;
    d.team_ctl = reinterpret_cast<uint32_t *>(ws);
    d.spin_limit = g_spin_limit;
    d.silent_member = g_silent_member;
    // every word a team launch of any shape on this workspace can read: at
    // most 2 slots per resident work-group, from the team region's start
    const size_t reach = (size_t)2 * std::max(team_capacity_max(), p.grid) * TEAM_SLOT_BYTES;
    d.team_clear_bytes = std::min(reach, ws_bytes - kTeamOff) & ~(size_t)15;
    if (p.group == 8 && p.halves == 2) {           // one launch, paired raw teams of 4 heads
      make_half(d, 0);
      d.halves = 2;
      e = launch_decode_team(d, p.grid, stream);
    } else if (p.group == 8) {                      // two launches of 4 query heads
      for (int half = 0; half < 2 && e == hipSuccess; ++half) {
        DecodeLaunch hd = d;
        make_half(hd, half);
        e = launch_decode_team(hd, p.grid, stream);
      }
    } else {
      e = launch_decode_team(d, p.grid, stream);
    }
    return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
  }
  if (split_halves(p, dp, ds)) {
    for (int half = 0; half < 2 && e == hipSuccess; ++half) {
      DecodeLaunch hd = d, hp = dp, hs = ds;
      make_half(hd, half);
      make_half(hp, half);
      make_half(hs, half);
      e = launch_chunks(p, hd, hp, hs, stream);
    }
  } else {
    e = launch_chunks(p, d, dp, ds, stream);
  }
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char *kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "required pointer is NULL";
    case KVQ_ERR_SHAPE: return "size out of range or inconsistent";
    case KVQ_ERR_FORMAT: return "unknown or disallowed format";
    case KVQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KVQ_ERR_UNSUPPORTED: return "unsupported combination";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

kvq_status kvq_quantize(const kvq_quant_args *a, kvq_stream stream) {
  if (!a) return KVQ_ERR_NULL;
  if (a->head_dim != KVQ_HEAD_DIM) return KVQ_ERR_UNSUPPORTED;
  if (a->in_format != KVQ_FMT_BF16 && a->in_format != KVQ_FMT_FP32) return KVQ_ERR_FORMAT;
  if (!is_store_fmt(a->k_format)) return KVQ_ERR_FORMAT;
  if (a->v_in && !is_store_fmt(a->v_format)) return KVQ_ERR_FORMAT;
  if (a->n_seq <= 0 || a->num_kv_heads <= 0 || a->capacity <= 0) return KVQ_ERR_SHAPE;
  if (a->capacity > (1 << 24) || (int64_t)a->n_seq * a->num_kv_heads > (1 << 24)) return KVQ_ERR_SHAPE;
  if (a->tok_begin < 0 || a->tok_end > a->capacity || a->tok_begin >= a->tok_end) return KVQ_ERR_SHAPE;
  if (!a->k_in || !a->k_out) return KVQ_ERR_NULL;
  if (a->v_in && !a->v_out) return KVQ_ERR_NULL;
  if (a->k_format != KVQ_FMT_BF16 && !a->k_scale_out) return KVQ_ERR_NULL;
  if (a->v_in && a->v_format != KVQ_FMT_BF16 && !a->v_scale_out) return KVQ_ERR_NULL;
  if (a->n_outlier_pairs < 0 || a->n_outlier_pairs > 16) return KVQ_ERR_SHAPE;
  const bool op = a->n_outlier_pairs > 0;
  // the bypassed channels are stored as the inputs' own bf16 values
  if (op && (a->k_format != KVQ_FMT_INT8_G32 || a->in_format != KVQ_FMT_BF16)) return KVQ_ERR_UNSUPPORTED;
  if (op && (!a->outlier_pairs || !a->k_outliers_out)) return KVQ_ERR_NULL;
  const void *ptrs[] = {a->k_in, a->v_in, a->k_out, a->v_out, a->k_scale_out, a->v_scale_out,
                        a->witness_out, a->stream_ids, a->v_witness_out,
                        op ? a->outlier_pairs : nullptr, op ? a->k_outliers_out : nullptr};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KVQ_ERR_ALIGN;
  const bool int8 = a->k_format == KVQ_FMT_INT8_DITHER || (a->v_in && a->v_format == KVQ_FMT_INT8_DITHER);
  const bool any_int8 = is_int8(a->k_format) || (a->v_in && is_int8(a->v_format));
  if (a->v_in && !g32_paired(a->k_format, a->v_format)) return KVQ_ERR_UNSUPPORTED;
  if (int8 && a->tok_begin % KVQ_INT8_BLOCK) return KVQ_ERR_UNSUPPORTED;   // whole 256-token blocks
  if (any_int8) {
    if (a->layer < 0 || a->layer >= (1 << 15) || a->num_kv_heads > (1 << 16)) return KVQ_ERR_SHAPE;
  }
  QuantLaunch q;
  q.k_format = a->k_format; q.v_format = a->v_format; q.in_format = a->in_format;
  q.k_in = a->k_in; q.v_in = a->v_in;
  q.n_seq = a->n_seq; q.h_kv = a->num_kv_heads; q.capacity = a->capacity;
  q.tok_begin = a->tok_begin; q.tok_end = a->tok_end;
  q.k_out = a->k_out; q.v_out = a->v_out; q.k_scale_out = a->k_scale_out; q.v_scale_out = a->v_scale_out;
  q.witness_out = a->witness_out;
  q.seed = a->seed; q.layer = a->layer; q.stream_id = a->stream_id; q.stream_ids = a->stream_ids;
  q.v_witness_out = a->v_in ? a->v_witness_out : nullptr;
  q.n_op = op ? a->n_outlier_pairs : 0;
  q.opairs = op ? a->outlier_pairs : nullptr;
  q.k_outliers_out = op ? a->k_outliers_out : nullptr;
  return launch_quantize(q, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

size_t kvq_workspace_bytes(const kvq_attn_args *a, const kvq_meter_out *m) {
  // the size does not depend on out/v; the per-chunk plan's region lies after
  // the team region of the same arguments, so its end covers both plans
  Plan p, q;
  if (make_plan(a, m, true, p) != KVQ_OK) return 0;
  if (make_plan(a, m, true, q, false) != KVQ_OK) return 0;
  return std::max(p.bytes, q.bytes);
}

kvq_status kvq_decode_plan(const kvq_attn_args *a, const kvq_meter_out *m, int meter_only,
                           kvq_plan_info *info) {
  if (!info) return KVQ_ERR_NULL;
  Plan p;
  const kvq_status s = make_plan(a, m, meter_only != 0, p);
  if (s != KVQ_OK) return s;
  info->team = p.team;
  info->n_teams = p.n_teams;
  info->rounds = p.rounds;
  info->grid = p.grid;
  info->chunk = p.chunk;
  info->chunks = p.total_chunks;
  info->workspace_bytes = p.bytes;
  if (p.team) {
    info->launches = (p.group == 8 && p.halves != 2) ? 2 : 1;
  } else {
    DecodeLaunch d, dp, ds;
    chunk_launches(a, m, p, meter_only != 0, nullptr, d, dp, ds);
    if (split_halves(p, dp, ds)) {
      DecodeLaunch hp = dp, hs = ds;
      make_half(hp, 0);
      make_half(hs, 0);
      info->launches = 2 * (chunk_launch_count(p, hp, hs) + (p.defer ? 1 : 0));
    } else {
      info->launches = chunk_launch_count(p, dp, ds) + (p.defer ? 1 : 0);
    }
  }
  info->reserved = 0;
  return KVQ_OK;
}

kvq_status kvq_workspace_init(void *ws, size_t bytes, kvq_stream stream) {
  if (!ws) return KVQ_ERR_NULL;
  if (!aligned16(ws)) return KVQ_ERR_ALIGN;
  // the whole workspace: the counters, and tagged team words of earlier calls
  return launch_fill_zero(ws, bytes & ~(size_t)3, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

kvq_status kvq_decode_attn(const kvq_attn_args *a, const kvq_meter_out *m, void *ws, size_t ws_bytes,
                           kvq_stream stream) {
  return run_decode(a, m, ws, ws_bytes, (hipStream_t)stream, false);
}

kvq_status kvq_meter(const kvq_attn_args *a, const kvq_meter_out *m, void *ws, size_t ws_bytes,
                     kvq_stream stream) {
  return run_decode(a, m, ws, ws_bytes, (hipStream_t)stream, true);
}

kvq_status kvq_decode_attn_noalloc(const kvq_attn_args *a, const kvq_meter_out *m, kvq_stream stream) {
  Plan p;
  const kvq_status s = make_plan(a, m, false, p);
  if (s != KVQ_OK) return s;
  if (p.bytes > KVQ_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;     // beyond the static scratch
  void *ws = nullptr;
  const kvq_status t = device_scratch((hipStream_t)stream, &ws);
  if (t != KVQ_OK) return t;
  return run_decode(a, m, ws, KVQ_SCRATCH_BYTES, (hipStream_t)stream, false);
}

#ifdef KVQ_TEST_HOOKS
// Test builds only: a smaller wait budget and a member that never publishes,
// so a GPU test can force a team wait to run out (the results turn to NaN
// and the status word reports it).  spin_limit 0 restores the default.
void kvq_test_set_team_hooks(unsigned spin_limit, int silent_member) {
  g_spin_limit = spin_limit ? spin_limit : (1u << 18);
  g_silent_member = silent_member;
}
#endif

}  // extern "C"
