/*
 * kvq.h - C ABI of the quantized-KV grouped-query decode attention library
 * with its fused quantization-risk meter (gfx950 / MI355X).
 *
 * The method comes from two public pages:
 *  - "WitCert: Sound Runtime Risk Observability and Gating for KV-Cache
 *    Quantization" (arXiv 2607.28699v1): the total-variation target (Sec. 3),
 *    Theorem 1 (e-form bound), the band-norm witness and Theorem 2 (Sec. 4.1),
 *    the subtractively dithered INT8 quantizer (Sec. 4.2, 6.2.1), the split-KV
 *    merge of the meter (Sec. 6.2.2) and its numerics (Sec. 3, 4.3, 6.2.4).
 *  - "Compress the shared cartridge. Keep the keys." (knlp.io): BF16/FP8 key
 *    and value layouts, the shared cartridge read with each request's live
 *    suffix in one online softmax ("One kernel spans cartridge and live KV").
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device unless
 *    stated; the caller owns every buffer.  The library never allocates,
 *    frees, copies to or from the host, or synchronizes; work is enqueued on
 *    `stream` (a hipStream_t; NULL is the null stream) in call order.
 *  - Argument checks run on the host before anything is enqueued and return a
 *    status; nothing aborts or throws across the ABI.  A launch failure
 *    reported by the runtime returns KVQ_ERR_LAUNCH.
 *  - Unsupported combinations are rejected with a status, never degraded.
 *  - head_dim is 128; the witness has 16 bands (2 bytes each, 32 B per token
 *    and head); INT8 scales cover blocks of 256 tokens.
 *  - Tensor element layouts are row-major with the listed shapes; every base
 *    pointer must be 16-byte aligned.
 *  - Results are bitwise reproducible for a given shape on a given device:
 *    the split of the sequence and every reduction order depend only on the
 *    shapes and on how many work-groups the device keeps resident.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 11
#define KVQ_HEAD_DIM 128
#define KVQ_N_BANDS 16
#define KVQ_INT8_BLOCK 256
#define KVQ_MAX_GROUP 8

typedef void *kvq_stream; /* hipStream_t */

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL */
  KVQ_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  KVQ_ERR_FORMAT = 3,      /* unknown format code, or a format not allowed here */
  KVQ_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  KVQ_ERR_UNSUPPORTED = 5, /* a valid combination this library does not implement */
  KVQ_ERR_WORKSPACE = 6,   /* workspace missing or smaller than kvq_workspace_bytes() */
  KVQ_ERR_LAUNCH = 7       /* the HIP runtime reported an error at launch */
} kvq_status;

/* Storage formats.  Scale layouts follow the format:
 *  KVQ_FMT_BF16         values stored as bf16, no scale.
 *  KVQ_FMT_FP8_E4M3     OCP E4M3FN codes (1 byte) with one fp32 scale per (token, KV
 *                       head): s = amax/448, code = nearest-even E4M3(x/s) (cartridge
 *                       page, "What fake quantization does"; WitCert Sec. 6.2.1 for
 *                       encoding with the stored scale).
 *  KVQ_FMT_INT8_DITHER  int8 codes with subtractive dither and one fp16 scale per
 *                       (256-token block, KV head, channel): s = fp16(amax/126.5),
 *                       code = rint(x/s + xi), x^ = s (code - xi), xi regenerated from
 *                       Philox4x32-10 (WitCert Sec. 4.2, 6.1.1, 6.2.1).
 *  KVQ_FMT_FP32         exact keys / write-path input only.
 *  KVQ_FMT_INT8_G32     int8 codes with the same subtractive dither and one fp16
 *                       scale per (token, KV head, 32-channel group), 4 per row:
 *                       scales [.., L, 4] laid out like the codes' rows (WitCert
 *                       Sec. 6.2.3, Table 4: token x G_c-channel groups, G_c = 32,
 *                       paging-safe).  Keys and values of a region use it together
 *                       (or keys alone for kvq_meter).  Decoded on the matrix cores
 *                       (one contraction per 32-channel group, scaled per token
 *                       after it), or on the vector ALUs where those do not apply. */
typedef enum kvq_format {
  KVQ_FMT_BF16 = 0,
  KVQ_FMT_FP8_E4M3 = 1,
  KVQ_FMT_INT8_DITHER = 2,
  KVQ_FMT_FP32 = 3,
  KVQ_FMT_INT8_G32 = 5
} kvq_format;

/* One KV region: the shared prefix ("cartridge", no batch dimension) or the
 * per-request suffix.  Shapes, with L = length, Hk = num_kv_heads, D = 128:
 *   dense prefix   codes [Hk, L, D]        fp8 scale [Hk, L]     int8 scale [Hk, ceil(L/256), D]
 *                  witness [Hk, L, 16]     exact keys [Hk, L, D]
 *   dense suffix   the same with a leading [batch] (L = capacity per request)
 *   paged suffix   codes [n_pages, Hk, P, D], fp8 scale [n_pages, Hk, P], witness
 *                  [n_pages, Hk, P, 16], exact keys [n_pages, Hk, P, D]; token i of
 *                  request b sits in page page_table[b * max_pages + i / P], row i % P.
 *                  Paged INT8 is rejected (its 256-token blocks would span pages).
 * Values in device memory are the caller's to keep in range, since the host
 * checks cannot read them without a synchronization: page ids in [0, n_pages)
 * for the pages a request's tokens use, suffix lengths (clamped to [0, length]
 * by the kernels) and finite inputs.
 * Semantics:
 *   witness NULL  -> the stored keys are claimed exact for the meter (c_t = 0).
 *   k_exact NULL  -> the stored keys are claimed exact for the TV (l_t = l~_t).
 * Logical token order is prefix tokens 0..P-1, then suffix tokens 0..n_b-1; the
 * dither stream of a token uses its index inside its own region. */
typedef struct kvq_region {
  int32_t k_format;         /* KVQ_FMT_BF16 | KVQ_FMT_FP8_E4M3 | KVQ_FMT_INT8_DITHER |
                               KVQ_FMT_INT8_G32 */
  int32_t v_format;         /* same set; INT8_G32 keys and values go together */
  const void *k;            /* stored key codes */
  const void *v;            /* stored value codes (may be NULL for kvq_meter) */
  const void *k_scale;      /* float (FP8) or fp16 bits (INT8); NULL for BF16 */
  const void *v_scale;
  const uint16_t *witness;  /* fp16 bits, or NULL */
  const void *k_exact;      /* exact keys for the TV, or NULL */
  int32_t k_exact_format;   /* KVQ_FMT_BF16 or KVQ_FMT_FP32 */
  int32_t length;           /* prefix: tokens (0 = no prefix); suffix: capacity per request */
  const int32_t *lengths;   /* suffix: device int32 [batch] tokens per request (<= length),
                               NULL = every request has `length` tokens; prefix: NULL */
  const int32_t *page_table;/* suffix only: device int32 [batch, max_pages], NULL = dense */
  int32_t page_size;        /* paged: 8 or 16 */
  int32_t max_pages;        /* paged: row length of page_table; capacity = max_pages * page_size */
  uint64_t seed;            /* INT8 dither: Philox key */
  int32_t layer;            /* INT8 dither: layer index, < 32768 */
  int32_t stream_id;        /* INT8 dither: prefix stream id; suffix: request b uses stream_id + b */
  const int32_t *stream_ids;/* suffix: optional device int32 [batch] stream ids (overrides) */
  const uint16_t *v_witness;/* value records, fp16 bits [.., len, 2] laid out like the witness:
                               (rho_t = ||v^_t - v_t||, ||v_t||), each rounded up; or NULL */
  /* Fixed outlier RoPE pairs of the keys (WitCert Sec. 6.2.5: one channel set
   * per (layer, KV head), kept exactly and left out of the group maximum),
   * KVQ_FMT_INT8_G32 keys only.  Slot i of KV head h names pair
   * P = outlier_pairs[h * n_outlier_pairs + i], i.e. channels P and P + 64;
   * a slot is active when 0 <= P < 64 and no earlier slot of that head names
   * P (others bypass nothing).  A bypassed channel's code is 0 and its value
   * is k_outliers[.., t, 2 i] (channel P) and [.., 2 i + 1] (channel P + 64),
   * the key's own bf16 value; inactive slots hold 0. */
  const int32_t *outlier_pairs; /* device int32 [num_kv_heads, n_outlier_pairs], or NULL */
  const uint16_t *k_outliers;   /* bf16 bits [.., len, 2 n_outlier_pairs] laid out like the codes */
  int32_t n_outlier_pairs;      /* m in [0, 16]; 0: no bypass */
} kvq_region;

/* Plan flags (kvq_attn_args.plan_flags).  0 is the library's choice; a flag
 * only narrows that choice, never enables a plan the arguments do not allow.
 * Unknown bits return KVQ_ERR_UNSUPPORTED.  Results of every plan meet the
 * same accuracy; they are bitwise equal only within one plan. */
#define KVQ_PLAN_NO_TEAM           0x01u /* never the team launch (the TV pairs go
                                            through the workspace instead of LDS) */
#define KVQ_PLAN_VECTOR_ALU        0x02u /* the vector-ALU kernel for every region
                                            (no matrix cores, no team, one launch
                                            per region) */
#define KVQ_PLAN_GROUP8_SEPARATE   0x04u /* a group of 8 on the team plan: two
                                            launches of 4 query heads, each
                                            reading the cache, not one paired launch */
#define KVQ_PLAN_FINALIZE_IN_PLACE 0x08u /* per-chunk plan: the TV and the block
                                            report in the decode launch's last
                                            work-group, no finish launch */
#define KVQ_PLAN_LAUNCH_PER_REGION 0x10u /* per-chunk plan: one launch per region,
                                            not one over cartridge and suffix */
#define KVQ_PLAN_ALL_FLAGS         0x1Fu

/* Bits a decode or meter call ORs into its status word (kvq_attn_args.status). */
#define KVQ_DEVSTATUS_TEAM_WAIT    0x1u  /* a team launch's bounded wait ran out (the
                                            device was shared with other work longer
                                            than the wait budget, about 10 ms): the
                                            results of the affected (request, KV
                                            head) pairs are NaN, none is stale */

/* Decode-step attention over prefix ++ suffix for every (request, query head).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  sm_scale is the
 * logit scale (1/sqrt(128) for the workloads here). */
typedef struct kvq_attn_args {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;     /* num_q_heads / num_kv_heads must be 1, 2, 4 or 8 */
  int32_t head_dim;         /* must be 128 */
  float sm_scale;           /* in (0, 1e6] */
  int32_t split_tokens;     /* tokens per work chunk; 0 = library choice; else a multiple of 64 */
  uint32_t plan_flags;      /* KVQ_PLAN_* bits, 0 = library choice */
  uint32_t *status;         /* device uint32 the call ORs KVQ_DEVSTATUS_* bits into, in
                               stream order (the caller clears it), or NULL.  The team
                               plan is taken only with a status word: it is the one plan
                               whose waits can run out.  16-byte aligned. */
  const float *q;           /* device fp32 [batch, num_q_heads, 128], post-RoPE, finite */
  kvq_region prefix;        /* prefix.length == 0: no shared prefix */
  kvq_region suffix;
  float *out;               /* device fp32 [batch, num_q_heads, 128] = sum_t p~_t v^_t */
} kvq_attn_args;

/* Per-(request, query head) meter outputs, device fp32 [batch, num_q_heads] each;
 * any may be NULL.  (WitCert Sec. 3, Thm. 1, Thm. 2, Sec. 4.3, 6.2.4)
 *   tv        = 1/2 sum_t |p_t - p~_t|, p from exact keys, p~ from stored keys
 *   log_a     = log E_p~[e^{c_t}],  c_t = sm_scale * sum_b ||q_b|| w_{t,b}
 *   bound_raw = 1/2 (A^2 - 1), +inf when beyond the float range
 *   meter     = min(1, bound_raw)
 * A is evaluated in the log domain and c is never truncated: when a term of
 * the log-domain sum overflows (or a band factor sm_scale ||q_b|| log2(e)
 * reaches 2^15, beyond the fp16 operand of the matrix-core witness dot),
 * log_a and bound_raw are +inf and meter is 1, the trivial bound (WitCert
 * Sec. 3 numerics, Sec. 6.2.4); bound_tanh is then 1.  c_t is rounded
 * upward: each band factor is raised by 2^-19 relative (a constant rounded
 * up) and enters as fp16 pieces whose sum is not below it, which covers the
 * fp32 roundings of the band norm and of the sum over the 16 bands, so the
 * computed c_t is not below c_t of the stored witness.
 * Tier B (WitCert Sec. 4.2, Lemma 2; Sec. 6.2.3): the sub-Gaussian certificate
 * of subtractively dithered INT8 keys, from the stored scales and the query
 * alone (no witness).  Requesting any of its outputs needs delta_b in (0, 1)
 * and, in every region present, INT8-dithered keys (either scale layout) or
 * keys stored as BF16 (radius 0); other key formats return KVQ_ERR_UNSUPPORTED.
 *   u_t         = sqrt(2 var_t log(2 S / delta_b)),
 *                 var_t = sm_scale^2 / 12 * sum_c q_c^2 s_{c,t}^2 (s: the key's
 *                 scale of channel c at token t), S = the request's tokens
 *   log_a_b     = log E_p~[e^{u_t}]
 *   bound_b_raw = 1/2 (A_B^2 - 1), +inf when beyond the float range
 *   meter_b     = min(1, bound_b_raw)
 * TV <= bound_b_raw holds with probability >= 1 - delta_b jointly over the S
 * tokens for a query that does not depend on the stored dither (a
 * non-adaptive query); delta_b is the per-(layer, head, step) share of a
 * request's budget, delta_req / (layers * heads * steps).
 * Value side and the joint output bound (WitCert Sec. 3; Sec. 4.2 "Value side
 * and the joint event"), from the regions' value records (every region present
 * must have v_witness, else KVQ_ERR_NULL; keys stored as BF16 or with a
 * witness, else KVQ_ERR_UNSUPPORTED):
 *   value_err  = sum_t p~_t rho_t
 *   v_norm_max = max_t ||v_t|| over the request's tokens
 *   out_bound  = 2 meter v_norm_max + value_err, an upper bound of
 *                ||y - out||, y the attention output with exact keys and values
 *                (meter as above; 0 when every region's keys are stored exactly).
 * Two-sided form (WitCert Sec. 4.3, Proposition 1), same needs as Tier A:
 *   log_a_minus     = log E_p~[e^{-c_t}]
 *   bound_two_sided = 1/2 (A/A- - A-/A), +inf when beyond the float range
 *   meter_two_sided = min(1, bound_raw, bound_two_sided)
 * Block-decomposable risk report (WitCert Sec. 6.3.5), device arrays
 * [batch, num_q_heads, n_blocks] with n_blocks = ceil(prefix.length / 256) +
 * ceil(suffix.length / 256): 256-token blocks aligned at the start of each
 * region, prefix first; blocks past a request's tokens read 0.
 *   block_mass     = sum_{t in j} p~_t
 *   block_excess   = sum_{t in j} p~_t (e^{c_t} - 1)   (they add up to A - 1;
 *                    same needs as Tier A)
 *   block_excess_b = block_mass (e^{u_j} - 1), u_j the block's Tier B radius
 *                    (needs the Tier B request and block-scale keys, whose
 *                    radius a block shares; they add up to A_B - 1)
 *   block_order    = int32 block indices by decreasing block_excess_b when
 *                    Tier B is requested (block-scale keys only), else
 *                    block_excess; ties by lower
 *                    index (the page-in order); needs n_blocks <= 512.
 * Deterministic tanh shape (WitCert Sec. 6.4.2, the compared system's
 * tanh(max_t Delta_t) with the same witness, Delta_t = c_t), same needs as
 * Tier A:
 *   bound_tanh = tanh(max_t c_t) */
typedef struct kvq_meter_out {
  float *tv;
  float *bound_raw;
  float *meter;
  float *log_a;
  float *log_a_b;
  float *bound_b_raw;
  float *meter_b;
  double delta_b;
  float *value_err;
  float *v_norm_max;
  float *out_bound;
  float *log_a_minus;
  float *bound_two_sided;
  float *meter_two_sided;
  float *block_mass;
  float *block_excess;
  float *block_excess_b;
  int32_t *block_order;
  float *bound_tanh;
} kvq_meter_out;

/* Write path: quantize tokens [tok_begin, tok_end) of every sequence and store
 * codes, scales and (optionally) the witness of the keys (WitCert Sec. 4.1,
 * Eq. (2): w_{t,b} = ||k^_t - k_t|| over band b, stored as fp16 rounded up).
 * Inputs are dense [n_seq, num_kv_heads, capacity, 128] in in_format (BF16 or
 * FP32); outputs use the dense region layouts above (a prefix is n_seq = 1).
 * For INT8 a call covers whole 256-token blocks: tok_begin must be a multiple of
 * 256 and the last block ends at tok_end.  A target format equal to the input
 * format copies the values.  The witness is computed in float64 and rounded
 * up to fp16, so it bounds the true residual norm. */
typedef struct kvq_quant_args {
  int32_t k_format;         /* target formats */
  int32_t v_format;
  int32_t in_format;        /* KVQ_FMT_BF16 or KVQ_FMT_FP32 */
  const void *k_in;         /* exact keys */
  const void *v_in;         /* exact values (NULL: values not written) */
  int32_t n_seq;
  int32_t num_kv_heads;
  int32_t head_dim;         /* must be 128 */
  int32_t capacity;
  int32_t tok_begin;
  int32_t tok_end;
  void *k_out;
  void *v_out;
  void *k_scale_out;        /* float [n_seq, Hk, capacity] or fp16 [n_seq, Hk, ceil(capacity/256), 128] */
  void *v_scale_out;
  uint16_t *witness_out;    /* fp16 bits [n_seq, Hk, capacity, 16], or NULL */
  uint64_t seed;            /* INT8 dither parameters, as in kvq_region */
  int32_t layer;
  int32_t stream_id;
  const int32_t *stream_ids;
  uint16_t *v_witness_out;  /* value records fp16 bits [n_seq, Hk, capacity, 2] =
                               (||v^_t - v_t||, ||v_t||): norms in float64 summed over
                               channels 0..127 in order, times 1 + 2^-48, rounded up
                               to fp16; or NULL.  Needs v_in. */
  const int32_t *outlier_pairs; /* fixed outlier pairs of the keys, as in kvq_region: their
                                   channels leave the group maximum, get code 0 and are
                                   stored exactly in k_outliers_out.  KVQ_FMT_INT8_G32 keys
                                   and BF16 input only (the stored values are the inputs). */
  uint16_t *k_outliers_out;     /* bf16 bits [n_seq, Hk, capacity, 2 n_outlier_pairs] */
  int32_t n_outlier_pairs;      /* m in [0, 16] */
} kvq_quant_args;

/* Library ABI version (KVQ_ABI_VERSION of the build). */
int kvq_abi_version(void);

/* Static English name of a status code. */
const char *kvq_status_string(kvq_status status);

/* Write path (see kvq_quant_args). */
kvq_status kvq_quantize(const kvq_quant_args *args, kvq_stream stream);

/* Bytes of device workspace kvq_decode_attn / kvq_meter need for these
 * arguments, captured into a graph or not.  Host-only: reads the current
 * device's properties, never its memory.  The decode and the meter call on
 * the same arguments need the same size.  Returns 0 on invalid arguments. */
size_t kvq_workspace_bytes(const kvq_attn_args *args, const kvq_meter_out *meter);

/* How kvq_decode_attn (meter_only = 0) or kvq_meter (meter_only != 0) will
 * run for these arguments on the current device, captured into a graph or not
 * (host-only, as above).
 *  - team > 0: one launch of at most as many work-groups as the device holds
 *    at once; `team` work-groups share each
 *    (request, KV head), each keeping its chunk's logit pairs in LDS for the
 *    TV (WitCert Sec. 3 target), `n_teams` teams take the (request, KV head)
 *    pairs in `rounds` rounds.  Chosen when the TV is requested for a single
 *    region of at most 131,072 tokens with GQA group 4 or 8, FP8/BF16 keys
 *    and values and bf16 exact keys, split_tokens 0, and neither Tier B nor
 *    the block report.  A group of 8 runs in one launch whose teams come in
 *    pairs, one raw team per 4 query heads (grid = 2 * n_teams * team,
 *    rounded up to a multiple of 8), so each tile is fetched from HBM about
 *    once; the per-chunk plan runs it as two launches of 4 query heads each
 *    where its kernels allow, each reading the cache.  Members wait only
 *    for members of their own team, with a bounded wait: a wait that runs
 *    out (another kernel holding the device for longer) leaves NaN in that
 *    (request, KV head)'s results, never a hang, and sets
 *    KVQ_DEVSTATUS_TEAM_WAIT in the call's status word.  Taken only when
 *    args->status is non-NULL and plan_flags allow it.
 *  - team == 0: `chunks` chunks of each (request, KV head) over both regions,
 *    one work-group each, in one launch (cartridge page: one kernel spans the
 *    shared cartridge and the live suffix) when both regions have keys of one
 *    format and, with FP8 keys, values of one format; else one launch per
 *    region.  The TV's logit pairs go through the workspace.
 * Both plans may be captured into a HIP graph: a team launch takes its tags
 * from an epoch kept in the workspace, which the launch's last work-group
 * moves past every tag it used, so each replay waits for fresh tags.
 * workspace_bytes is what this plan needs; kvq_workspace_bytes may return
 * more (it covers the other plan of the same arguments too). */
typedef struct kvq_plan_info {
  int32_t team;             /* work-groups per (request, KV head); 0: no team launch */
  int32_t n_teams;          /* teams; a group of 8 runs two raw teams (4 query heads each) per team */
  int32_t rounds;           /* (request, KV head) pairs each team takes in turn */
  int32_t grid;             /* work-groups of the team launch */
  int32_t chunk;            /* tokens per chunk */
  int32_t chunks;           /* chunks per (request, KV head), both regions */
  int32_t launches;         /* kernel launches of the call: 1, or 2 when the
                               two regions' formats need separate kernels; one
                               more when a per-chunk plan with several chunks
                               per (request, KV head) runs the TV and the block
                               report in a finish launch over many work-groups;
                               a per-chunk plan of a group of 8 doubles all that */
  int32_t reserved;         /* 0 */
  uint64_t workspace_bytes;
} kvq_plan_info;
kvq_status kvq_decode_plan(const kvq_attn_args *args, const kvq_meter_out *meter, int meter_only,
                           kvq_plan_info *info);

/* Prepare a workspace for first use: clears all of it (one fill kernel on
 * `stream`).  A workspace stays ready after every successful kvq_decode_attn /
 * kvq_meter call, of any shape and either plan, so calls of different shapes
 * may share one workspace (not at the same time: calls that share a
 * workspace must not overlap).  Layout, from the start:
 *  - 256 bytes of control words: the team epoch and the count of finished
 *    team work-groups (0 at rest);
 *  - 1 MiB of per-chunk arrival counters, one per (request, KV head), each
 *    reset to 0 by the group's last work-group;
 *  - the team plan's exchange slots, when a team plan exists for the
 *    arguments;
 *  - the per-chunk plan's partial states and TV spill.
 * So the two plans of the same arguments never share a word.  Team words are
 * 64-bit (tag, value) pairs.  A tag is a signalling-NaN bit pattern that no
 * kernel stores as data (arithmetic never produces one, and no input is
 * copied into the workspace), so no partial state or spill word of any call
 * can pass for a team word.  A launch waits only for tags above every tag
 * used on the workspace since the epoch last restarted.  The epoch restarts
 * after 2^22 - 2^18 tags (about 430,000 launches of the batch-64 step); the
 * launch that restarts it clears every word any team launch on the workspace
 * can read (at most 2 x resident work-groups x 4,480 bytes, 4.6 MB here), so
 * no word from before the restart carries a tag being waited for. */
kvq_status kvq_workspace_init(void *workspace, size_t workspace_bytes, kvq_stream stream);

/* Decode attention with the fused meter (WitCert Sec. 6 meter loop, read path;
 * cartridge page, one online softmax over cartridge and suffix).  meter may be
 * NULL (attention only).  args->out must be non-NULL. */
kvq_status kvq_decode_attn(const kvq_attn_args *args, const kvq_meter_out *meter,
                           void *workspace, size_t workspace_bytes, kvq_stream stream);

/* Meter only ("observatory" role, WitCert Fig. 2): the same pass without the
 * values and the output; args->out and the regions' v pointers are ignored. */
kvq_status kvq_meter(const kvq_attn_args *args, const kvq_meter_out *meter,
                     void *workspace, size_t workspace_bytes, kvq_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * kvq_decode_attn with the library's own scratch instead of a caller
 * workspace.  The scratch is one static device array of KVQ_SCRATCH_BYTES per
 * device, held until the process ends; the call allocates nothing.  The
 * caller still passes the inputs, outputs and (for the team plan) the status
 * word.  The first call on a device looks the array up and enqueues one fill
 * kernel on `stream` that clears it (make that first call outside graph
 * capture if the capture must not contain it); later calls rely on the
 * workspace protocol, which leaves the scratch ready after every call.
 * Returns KVQ_ERR_WORKSPACE, before anything is enqueued, when the plan for
 * these arguments needs more than KVQ_SCRATCH_BYTES (kvq_decode_plan's
 * workspace_bytes); the per-chunk plan's TV spill is the large part (32
 * bytes per cached token and KV head).  Every call on one device shares its
 * array: calls that overlap in time on one device (other streams, other
 * threads) race and must not be made. */
#define KVQ_SCRATCH_BYTES ((size_t)96 << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_attn_args *args, const kvq_meter_out *meter,
                                   kvq_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
