/* Plain C (C99) use of the whole GPU path through the library's C ABI, with
 * the HIP runtime for memory and a stream and nothing else (no Python, no
 * C++): reads a task table and the shards' BF16 bytes from a file, puts every
 * shard in its own device allocation, creates a plan over a device
 * destination region filled with 0xA5, replays it twice on a stream of its
 * own, and writes the destination region to a second file.
 *
 * Input file, little-endian: "WTC1", uint32 n_tasks, uint64 dst_bytes; per
 * task: int32 n_shards, int32 dtype, int32 fusion_group, int32 0, int64 cols,
 * uint64 dst_offset, uint64 scale_offset, int64 rows[n_shards]; then the
 * shards' bytes (2 rows cols each), task by task, shard by shard.
 *
 * Usage: c_gpu_prepare IN OUT [REPLAYS]. REPLAYS (default 2, at least 2)
 * replays are made; from the second on they are issued back to back and
 * timed, on the stream (HIP events) and on the host (the wt_prepare calls),
 * and the times per replay are printed. Exit code 0 and "c gpu prepare ok"
 * on success; otherwise the failing call and its status text are printed. */
#define _POSIX_C_SOURCE 199309L
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "wt.h"

#define FAIL(...)                      \
  do {                                 \
    fprintf(stderr, __VA_ARGS__);      \
    fputc('\n', stderr);               \
    return 1;                          \
  } while (0)

#define HIP_CHECK(call)                                                      \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));     \
  } while (0)

static int read_exact(FILE *f, void *p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char **argv) {
  if (argc != 3 && argc != 4) FAIL("usage: %s IN OUT [REPLAYS]", argv[0]);
  const long replays = argc == 4 ? strtol(argv[3], NULL, 10) : 2;
  if (replays < 2 || replays > 1000000) FAIL("REPLAYS must be in [2, 1000000]");
  FILE *in = fopen(argv[1], "rb");
  if (!in) FAIL("cannot open %s", argv[1]);

  char magic[4];
  uint32_t n_tasks = 0;
  uint64_t dst_bytes = 0;
  if (!read_exact(in, magic, 4) || memcmp(magic, "WTC1", 4) != 0 || !read_exact(in, &n_tasks, 4) ||
      !read_exact(in, &dst_bytes, 8) || n_tasks == 0 || dst_bytes == 0)
    FAIL("bad header in %s", argv[1]);

  wt_task *tasks = calloc(n_tasks, sizeof *tasks);
  wt_shard **shards = calloc(n_tasks, sizeof *shards);
  if (!tasks || !shards) FAIL("out of host memory");
  for (uint32_t i = 0; i < n_tasks; ++i) {
    int32_t h[4];
    int64_t cols;
    uint64_t offs[2];
    if (!read_exact(in, h, sizeof h) || !read_exact(in, &cols, 8) || !read_exact(in, offs, sizeof offs))
      FAIL("truncated task %u", i);
    if (h[0] < 1) FAIL("task %u: no shards", i);
    shards[i] = calloc((size_t)h[0], sizeof **shards);
    if (!shards[i]) FAIL("out of host memory");
    for (int32_t k = 0; k < h[0]; ++k) {
      int64_t rows;
      if (!read_exact(in, &rows, 8)) FAIL("truncated task %u", i);
      shards[i][k].rows = rows;
    }
    tasks[i].shards = shards[i];
    tasks[i].n_shards = h[0];
    tasks[i].shard_mem = WT_MEM_DEVICE;
    tasks[i].cols = cols;
    tasks[i].dtype = h[1];
    tasks[i].fusion_group = h[2];
    tasks[i].dst_offset = offs[0];
    tasks[i].scale_offset = offs[1];
  }
  /* shard bytes into device memory, one allocation per shard */
  for (uint32_t i = 0; i < n_tasks; ++i)
    for (int32_t k = 0; k < tasks[i].n_shards; ++k) {
      const size_t bytes = 2u * (size_t)shards[i][k].rows * (size_t)tasks[i].cols;
      if (bytes == 0) continue;
      void *host = malloc(bytes), *dev = NULL;
      if (!host) FAIL("out of host memory");
      if (!read_exact(in, host, bytes)) FAIL("truncated shard data (task %u shard %d)", i, (int)k);
      HIP_CHECK(hipMalloc(&dev, bytes));
      HIP_CHECK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
      free(host);
      shards[i][k].ptr = dev;
    }
  fclose(in);

  void *dst = NULL;
  HIP_CHECK(hipMalloc(&dst, (size_t)dst_bytes));
  HIP_CHECK(hipMemset(dst, 0xA5, (size_t)dst_bytes));
  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));

  wt_plan *plan = NULL;
  wt_status st = wt_plan_create(tasks, n_tasks, dst, (size_t)dst_bytes, WT_MEM_DEVICE, NULL, &plan);
  if (st != WT_OK) FAIL("wt_plan_create: %s: %s", wt_status_str(st), wt_plan_last_error(NULL));
  wt_plan_info info;
  st = wt_plan_get_info(plan, &info);
  if (st != WT_OK) FAIL("wt_plan_get_info: %s", wt_status_str(st));
  /* the first replay, then the others back to back, timed */
  st = wt_prepare(plan, (void *)stream);
  if (st != WT_OK) FAIL("wt_prepare: %s: %s", wt_status_str(st), wt_plan_last_error(plan));
  HIP_CHECK(hipStreamSynchronize(stream));
  hipEvent_t e0, e1;
  HIP_CHECK(hipEventCreate(&e0));
  HIP_CHECK(hipEventCreate(&e1));
  struct timespec h0, h1;
  clock_gettime(CLOCK_MONOTONIC, &h0);
  HIP_CHECK(hipEventRecord(e0, stream));
  for (long r = 1; r < replays; ++r) {
    st = wt_prepare(plan, (void *)stream);
    if (st != WT_OK) FAIL("wt_prepare: %s: %s", wt_status_str(st), wt_plan_last_error(plan));
  }
  clock_gettime(CLOCK_MONOTONIC, &h1);
  HIP_CHECK(hipEventRecord(e1, stream));
  HIP_CHECK(hipEventSynchronize(e1));
  float ms = 0.0f;
  HIP_CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double host_us = (double)(h1.tv_sec - h0.tv_sec) * 1e6 + (double)(h1.tv_nsec - h0.tv_nsec) * 1e-3;
  printf("%ld replays back to back: %.2f us per replay on the stream, %.2f us per wt_prepare call on the host\n",
         replays - 1, 1000.0 * ms / (double)(replays - 1), host_us / (double)(replays - 1));
  HIP_CHECK(hipEventDestroy(e0));
  HIP_CHECK(hipEventDestroy(e1));
  wt_plan_destroy(plan);

  unsigned char *out = malloc((size_t)dst_bytes);
  if (!out) FAIL("out of host memory");
  HIP_CHECK(hipMemcpy(out, dst, (size_t)dst_bytes, hipMemcpyDeviceToHost));
  FILE *fo = fopen(argv[2], "wb");
  if (!fo || fwrite(out, 1, (size_t)dst_bytes, fo) != (size_t)dst_bytes || fclose(fo) != 0)
    FAIL("cannot write %s", argv[2]);
  free(out);

  HIP_CHECK(hipStreamDestroy(stream));
  HIP_CHECK(hipFree(dst));
  for (uint32_t i = 0; i < n_tasks; ++i) {
    for (int32_t k = 0; k < tasks[i].n_shards; ++k)
      if (shards[i][k].ptr) HIP_CHECK(hipFree((void *)shards[i][k].ptr));
    free(shards[i]);
  }
  free(shards);
  free(tasks);
  printf("c gpu prepare ok: %u tasks, %lld tiles, %llu bytes\n", n_tasks, (long long)info.n_tiles,
         (unsigned long long)dst_bytes);
  return 0;
}
