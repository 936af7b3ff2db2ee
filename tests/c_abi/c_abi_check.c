/* Plain C (C99) use of the library's C ABI, without Python or C++: includes
 * include/wt.h, links libwt.so and drives the host-only entry points (plan
 * validation and shape, the replay schedule, the static schedule builder,
 * status texts, the host-side progress wait). No GPU call is made. Exit code
 * 0 and "c abi ok" on success; the first failed check is printed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "wt.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("check failed at line %d: %s\n", __LINE__, #cond);      \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  /* options */
  wt_plan_options o;
  wt_plan_options_init(&o);
  CHECK(o.watermark_bytes == 512ull << 20 && o.dst_write_mode == WT_DST_ZERO_COPY && o.device == -1);

  /* one fused output [q; k] of 256 x 256 from two tasks with 2 shards each
     (made-up, aligned device addresses: nothing is dereferenced) */
  wt_shard q_sh[2] = {{(const void *)(uintptr_t)0x7f0000000000ull, 64}, {(const void *)(uintptr_t)0x7f0000010000ull, 64}};
  wt_shard k_sh[2] = {{(const void *)(uintptr_t)0x7f0000020000ull, 64}, {(const void *)(uintptr_t)0x7f0000030000ull, 64}};
  wt_task t[2];
  memset(t, 0, sizeof t);
  t[0].shards = q_sh;
  t[0].n_shards = 2;
  t[0].shard_mem = WT_MEM_DEVICE;
  t[0].cols = 256;
  t[0].dtype = WT_FP8_E4M3FN_B128;
  t[0].fusion_group = 7;
  t[0].dst_offset = 0;
  t[0].scale_offset = 65536;
  t[1] = t[0];
  t[1].shards = k_sh;
  wt_plan_info info;
  CHECK(wt_plan_check(t, 2, 65536 + 256, WT_MEM_DEVICE, &o, &info) == WT_OK);
  CHECK(info.n_outputs == 1 && info.n_tiles == 4 && info.input_bytes == 2 * 256 * 256);
  CHECK(info.output_bytes == 256 * 256 + 16 && info.n_launches == 1 && info.n_chunks == 0 && info.n_units == 1);

  /* errors carry a status and a message */
  CHECK(wt_plan_check(t, 2, 1000, WT_MEM_DEVICE, &o, &info) == WT_E_RANGE);
  CHECK(strlen(wt_plan_last_error(NULL)) > 0);
  CHECK(strncmp(wt_status_str(WT_E_RANGE), "WT_E_RANGE", 10) == 0);

  /* pinned-host shards: a replay schedule of H2D copy and prepare per chunk */
  t[0].shard_mem = t[1].shard_mem = WT_MEM_PINNED_HOST;
  size_t n_ops = 0;
  CHECK(wt_plan_schedule(t, 2, 65536 + 256, WT_MEM_DEVICE, &o, NULL, 0, &n_ops) == WT_OK && n_ops >= 2);
  wt_sched_op ops[16];
  CHECK(n_ops <= 16);
  CHECK(wt_plan_schedule(t, 2, 65536 + 256, WT_MEM_DEVICE, &o, ops, n_ops, &n_ops) == WT_OK);
  CHECK(ops[0].stage == 0 && ops[1].stage == 1 && ops[0].chunk == 0);

  /* static schedule: two training parameters fused into one inference tensor */
  const char *comps[2] = {"q", "k"};
  wt_param_meta pm[3] = {{"q", 128, 256, 2, WT_MEM_DEVICE, NULL},
                         {"k", 128, 256, 2, WT_MEM_DEVICE, NULL},
                         {"unused", 4, 4, 1, WT_MEM_DEVICE, NULL}};
  wt_dst_meta dm[1] = {{"qk", comps, 2, WT_FP8_E4M3FN_B128}};
  wt_schedule *sch = NULL;
  CHECK(wt_schedule_build(pm, 3, dm, 1, NULL, &sch) == WT_OK && sch != NULL);
  size_t nt = 0, ns = 0, nu = 0;
  uint64_t db = 0;
  CHECK(wt_schedule_info(sch, &nt, &ns, &db, &nu) == WT_OK);
  CHECK(nt == 2 && ns == 4 && nu == 1 && db == 65536 + 256);
  uint64_t dofs = 1, sofs = 0, ib = 0;
  int32_t src = -2;
  CHECK(wt_schedule_output(sch, 0, &dofs, &sofs, &src, &ib) == WT_OK);
  CHECK(dofs == 0 && sofs == 65536 && src == 0 && ib == 2 * 256 * 256);
  wt_task st[2];
  wt_shard ssh[4];
  CHECK(wt_schedule_tasks(sch, -1, st, 1, ssh, 4, &nt, &ns) == WT_E_RANGE && nt == 2);
  CHECK(wt_schedule_tasks(sch, -1, st, 2, ssh, 4, &nt, &ns) == WT_OK);
  CHECK(st[0].fusion_group == 0 && st[1].fusion_group == 0 && st[1].shards[1].rows == 64);
  wt_schedule_destroy(sch);
  const char *bad[1] = {"nope"};
  wt_dst_meta dbad[1] = {{"x", bad, 1, WT_FP8_E4M3FN_B128}};
  CHECK(wt_schedule_build(pm, 3, dbad, 1, NULL, &sch) == WT_E_INVAL && sch == NULL);
  CHECK(strstr(wt_plan_last_error(NULL), "nope") != NULL);

  /* host-side progress wait */
  uint64_t word = 3;
  CHECK(wt_progress_wait(&word, 3, 0) == WT_OK);
  CHECK(wt_progress_wait(&word, 4, 1000000) == WT_E_TIMEOUT);
  CHECK(wt_progress_wait(NULL, 1, 0) == WT_E_INVAL);

  printf("c abi ok\n");
  return 0;
}
