// plan.h -- host-only plan building for libwt.so: validation of the task
// table, the output/segment model, pipeline chunks with their staging ring
// placement, and the device descriptor tables of each launch. Nothing here
// calls the HIP runtime, so it runs (and is tested) without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "wt.h"
#include "wt_internal.h"

namespace wt {

// Rows [row0, row0 + nrows) of an output come from the shard at `src`.
struct HostSeg {
  const void *src;
  int64_t row0;
  int64_t nrows;
};

struct HostOutput {
  int32_t dtype = 0;  // WT_FP8_E4M3FN_B128 or WT_BF16_COPY
  int32_t mem = 0;    // WT_MEM_DEVICE or WT_MEM_PINNED_HOST
  int32_t first_task = 0;
  int64_t rows = 0, cols = 0;
  uint64_t dst_off = 0, scale_off = 0;
  int64_t tiles_r = 0, tiles_c = 0;
  int64_t in_bytes = 0, data_bytes = 0, scale_bytes = 0;
  std::vector<HostSeg> segs;  // non-empty shards only, in assembly order
};

// A host-to-device copy of a pinned-host run into staging.
struct H2DCopy {
  const void *src;
  int64_t stage_off;  // relative to the chunk's slot
  int64_t bytes;
};

// A staging-to-destination copy (WT_DST_STAGED).
struct DstCopy {
  int64_t stage_off;  // relative to the chunk's slot
  uint64_t dst_off;
  int64_t bytes;
};

// Outputs moved through the pipeline stages together.
struct Chunk {
  std::vector<int32_t> outputs;
  bool h2d = false;                   // inputs come from pinned host memory
  int64_t slot_off = 0, slot_bytes = 0;  // staging slot in the ring
  int32_t wait_for = -1;              // chunk whose release must precede our H2D
  int64_t in_bytes = 0;               // BF16 bytes prepared
  // staging placement (offsets relative to the slot):
  std::vector<std::vector<int64_t>> seg_stage;  // [k][s]: input segment s of outputs[k]
  std::vector<int64_t> data_stage;              // [k]: output data (staged mode), -1 otherwise
  std::vector<int64_t> scale_stage;             // [k]: output scales (staged mode)
  std::vector<H2DCopy> h2d_copies;
  std::vector<DstCopy> dst_copies;
};

struct Layout {
  std::vector<HostOutput> outs;
  std::vector<int32_t> direct;  // device-resident outputs prepared by one launch on the caller's stream
  std::vector<Chunk> chunks;
  int64_t staging_bytes = 0;
  int32_t dst_mode = WT_DST_ZERO_COPY;
  uint32_t load_hint = WT_LOAD_AUTO;
  uint32_t max_replays_in_flight = 1;  // resolved host-side backpressure depth (pipelined plans)
  uint32_t tile_group = WT_GROUP_AUTO;
  std::vector<int32_t> task_unit;  // completion unit of each task (direct launch, then chunks)
  wt_plan_info info{};
};

// Validates the table and builds the layout. err receives a message on failure.
wt_status build_layout(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                       const wt_plan_options &opts, Layout *layout, std::string *err);

// Host images of the device tables of one launch batch.
struct HostTables {
  std::vector<DevOut> outs;
  std::vector<DevSeg> segs;
  std::vector<RegDesc> fast;
  std::vector<TileItem> edge;
  std::vector<GenDesc> general;
  std::vector<CopyItem> copies;
  bool xcd_order = false;  // some aligned-path output's rows share 128-byte lines with a neighbour tile's
};

// Address resolver for one batch: where output k's inputs and outputs are.
struct BatchAddr {
  // segment source address (segment s of output o)
  virtual uint64_t seg_src(int32_t k, int32_t o, int32_t s) const = 0;
  virtual uint64_t data_dst(int32_t k, int32_t o) const = 0;
  virtual uint64_t scale_dst(int32_t k, int32_t o) const = 0;
  virtual ~BatchAddr() = default;
};

void build_tables(const Layout &L, const std::vector<int32_t> &outputs, const BatchAddr &addr, HostTables *t);

// Number of kernel launches a batch needs (aligned tiles + copies, general tiles).
int launches_for(const HostTables &t);

// Splits one byte-range copy into CopyItems (alignment-aware, <= kCopyItemMax bytes each).
void add_copy_items(std::vector<CopyItem> &v, uint64_t src, uint64_t dst, uint64_t bytes);

// Records of the schedule one wt_prepare replays, in enqueue order.
void schedule_ops(const Layout &L, std::vector<wt_sched_op> *ops);

// Options with defaults filled in (host_api.cpp).
wt_plan_options resolve_opts(const wt_plan_options *o);
// The calling thread's last error text (host_api.cpp).
void set_thread_error(const std::string &msg);
// Text of the last error recorded on a plan (runtime.cpp).
const char *plan_error_text(const wt_plan *plan);

}  // namespace wt
