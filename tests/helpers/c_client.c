/* A plain C99 client of the C ABI (include/kvq.h): host-only calls, no
 * device memory.  It plans the batch-64 x 12,628-token decode step (FP8 keys
 * and values, bf16 exact keys, witness) and prints what the planner reports,
 * so a test can check that the header is valid C and the library links and
 * answers from C without any Python. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

int main(void) {
  static char dummy[64] __attribute__((aligned(256)));   /* never dereferenced by the host calls */
  void *p = dummy;
  kvq_attn_args a;
  kvq_meter_out m;
  kvq_plan_info info;
  memset(&a, 0, sizeof a);
  memset(&m, 0, sizeof m);
  memset(&info, 0, sizeof info);
  a.batch = 64;
  a.num_q_heads = 32;
  a.num_kv_heads = 8;
  a.head_dim = KVQ_HEAD_DIM;
  a.sm_scale = 0.08838834764831845f;
  a.q = (const float *)p;
  a.out = (float *)p;
  a.suffix.k_format = KVQ_FMT_FP8_E4M3;
  a.suffix.v_format = KVQ_FMT_FP8_E4M3;
  a.suffix.k = p;
  a.suffix.v = p;
  a.suffix.k_scale = p;
  a.suffix.v_scale = p;
  a.suffix.witness = (const uint16_t *)p;
  a.suffix.k_exact = p;
  a.suffix.k_exact_format = KVQ_FMT_BF16;
  a.suffix.length = 12628;
  a.plan_flags = KVQ_PLAN_NO_TEAM;
  m.tv = (float *)p;
  m.bound_raw = (float *)p;
  m.meter = (float *)p;
  m.log_a = (float *)p;
  const kvq_status s = kvq_decode_plan(&a, &m, 0, &info);
  const size_t ws = kvq_workspace_bytes(&a, &m);
  printf("abi %d\n", kvq_abi_version());
  printf("status %d %s\n", (int)s, kvq_status_string(s));
  printf("plan chunk %d chunks %d launches %d team %d\n", info.chunk, info.chunks, info.launches, info.team);
  printf("workspace %llu %llu\n", (unsigned long long)info.workspace_bytes, (unsigned long long)ws);
  a.head_dim = 64;                                        /* rejected before anything is enqueued */
  printf("bad head_dim %d\n", (int)kvq_decode_attn(&a, &m, p, ws, NULL));
  return s == KVQ_OK ? 0 : 1;
}
