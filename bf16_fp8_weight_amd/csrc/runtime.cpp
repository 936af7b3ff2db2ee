// runtime.cpp -- C ABI of libwt.so: plan creation (device tables, staging,
// streams), replay, teardown, and the element-function check entry points.
//
// Replay follows "Weight transfer for RL post-training in under 2 seconds",
// section "Task pipeline": each stage keeps a FIFO of tasks and a task moves
// to the next stage's queue when it finishes the current one. Here each stage
// is an in-order HIP stream (host-to-device copy, prepare, destination copy);
// a chunk of tasks enters the next stage's stream behind an event recorded
// when it left the previous one, and a chunk's host-to-device copy waits for
// the release of the earlier chunk whose staging slot it reuses, which keeps
// in-flight staging under the watermark (section "GPU memory usage control").
// Everything is enqueued asynchronously; the host never polls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "plan.h"
#include "wt.h"

namespace wt {
hipError_t launch_batch(const LaunchTables &T, hipStream_t stream, int device);
hipError_t launch_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, uint8_t *out, int variant,
                                  hipStream_t stream);
hipError_t launch_cast_range(uint32_t first, uint64_t count, uint8_t *out, hipStream_t stream);
hipError_t launch_act_quant(const ActArgs &a, bool fast, hipStream_t stream);
hipError_t launch_progress_mark(uint64_t *epoch, uint64_t *word, bool first, hipStream_t stream);
}  // namespace wt

using namespace wt;

struct wt_plan {
  Layout L;
  int device = 0;
  uint8_t *dst = nullptr;
  size_t dst_bytes = 0;
  int32_t dst_kind = WT_MEM_DEVICE;
  bool pipeline = false;

  uint8_t *tables = nullptr;  // every batch's device tables, one allocation
  uint64_t *epoch = nullptr;  // replay counter (device, inside the tables allocation)
  uint64_t *progress = nullptr;  // caller's completion words (pinned host), or null
  uint8_t *staging = nullptr;
  std::vector<LaunchTables> batches;  // [0] = direct batch when present, then one per chunk
  int direct_batch = -1;
  int first_chunk_batch = 0;

  hipStream_t s_h2d = nullptr, s_prep = nullptr, s_out = nullptr;
  std::vector<hipEvent_t> ev_h2d, ev_prep, ev_rel;
  hipEvent_t ev_start = nullptr, ev_out_end = nullptr;
  hipEvent_t ev_last = nullptr;  // after the latest launch on the caller's stream (plans without a pipeline)
  std::vector<hipEvent_t> ev_done;  // end of pipelined replay r at [r % size]: replays in flight
  uint64_t replays = 0;             // pipelined replays enqueued so far

  std::vector<char> rel_waited;  // per chunk: some later chunk waits for its release
  // no-allocation plan (wt_plan_create_noalloc): its device tables live in
  // the device's static scratch array and ev_last is that device's event;
  // neither is freed by the plan
  struct NoAllocDev *noalloc = nullptr;
  std::atomic<bool> busy{false};
  mutable std::mutex err_mu;
  std::string last_error;
};

namespace {

void set_err(wt_plan *p, const std::string &m) {
  if (p) {
    std::lock_guard<std::mutex> g(p->err_mu);
    p->last_error = m;
  } else {
    set_thread_error(m);
  }
}

}  // namespace

namespace wt {
// Text of the last error recorded on a plan (wt_plan_last_error).
const char *plan_error_text(const wt_plan *plan) {
  std::lock_guard<std::mutex> g(plan->err_mu);
  // the string lives in the plan; valid until the next error on it or destroy
  return plan->last_error.c_str();
}
}  // namespace wt

namespace {

std::string hip_msg(const char *what, hipError_t e) {
  return std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
}

#define HIP_OR(plan, expr)                               \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) {                              \
      set_err((plan), hip_msg(#expr, e_));               \
      return WT_E_HIP;                                   \
    }                                                    \
  } while (0)

// Makes `dev` current for the scope and restores the caller's device on
// exit; a no-op (one hipGetDevice) when `dev` is current already.
struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      (void)hipGetLastError();
      prev = -1;
    }
    if (dev >= 0 && dev != prev && hipSetDevice(dev) == hipSuccess) switched = prev >= 0;
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

}  // namespace

// ---- device tables without allocation (wt_plan_create_noalloc)
// One static array per GPU holds the descriptor tables of that GPU's one
// no-allocation plan. On the host, `scratch` names a host-side stand-in,
// not device memory: host code uses only the device address that
// hipGetSymbolAddress returns for it (per device, at the first
// no-allocation call on that device).
static __device__ __align__(256) uint8_t scratch[WT_NOALLOC_TABLE_BYTES];

// Flags of the event a replay of a plan without a pipeline records behind
// its launch when the destination is device memory. The event only tells
// wt_plan_destroy that every replay has run (the kernels read the device
// tables; nothing the host reads depends on it), so it carries no
// system-scope fence: with the fence (a cache write-back and invalidation) a
// replay of a one-layer plan (720 tiles) took 9.75 us on the stream and
// 5.6 us on the host back to back, without it 7.9 and 4.5 us, on MI355X.
// Plans that write host memory keep the fenced event, the last command of
// their replay, so that synchronizing with the stream still publishes the
// bytes to the host as before.
constexpr unsigned kReplayEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

struct NoAllocDev {
  std::once_flag once;
  hipError_t err = hipSuccess;
  uint8_t *ptr = nullptr;   // this device's copy of `scratch`
  hipEvent_t ev = nullptr;  // after the latest replay of the device's no-allocation plan
  std::atomic<bool> in_use{false};
};

namespace {

constexpr int kMaxNoAllocDevices = 64;
NoAllocDev g_noalloc[kMaxNoAllocDevices];

// Set-up of device `dev` (which must be current): the address of its scratch
// array and its event, made once per device and kept until the process ends.
NoAllocDev *noalloc_device(int dev, std::string *err) {
  if (dev < 0 || dev >= kMaxNoAllocDevices) {
    *err = "device ordinal out of range for the no-allocation path";
    return nullptr;
  }
  NoAllocDev &d = g_noalloc[dev];
  std::call_once(d.once, [&d] {
    void *a = nullptr;
    d.err = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess && !a) d.err = hipErrorInvalidSymbol;
    if (d.err == hipSuccess) {
      d.ptr = (uint8_t *)a;
      d.err = hipEventCreateWithFlags(&d.ev, hipEventDisableTiming);
    }
    if (d.err != hipSuccess) (void)hipGetLastError();
  });
  if (d.err != hipSuccess) {
    *err = hip_msg("no-allocation set-up (hipGetSymbolAddress / hipEventCreate)", d.err);
    return nullptr;
  }
  return &d;
}

// Checks that [p, p + bytes) lies in one allocation of the expected kind.
wt_status check_memory(const void *p, uint64_t bytes, int32_t kind, int device, const std::string &what,
                       std::string *err) {
  if (bytes == 0) return WT_OK;
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof a);
  hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *err = what + ": pointer is not HIP device or pinned host memory";
    return WT_E_INVAL;
  }
  if (kind == WT_MEM_DEVICE) {
    if (a.type != hipMemoryTypeDevice) {
      *err = what + ": expected device memory";
      return WT_E_INVAL;
    }
    if (a.device != device) {
      *err = what + ": device memory of another GPU";
      return WT_E_INVAL;
    }
  } else {
    if (a.type != hipMemoryTypeHost) {
      *err = what + ": expected pinned host memory";
      return WT_E_INVAL;
    }
  }
  // extent: the allocation that holds p must also hold p + bytes - 1 (device
  // allocations and pinned host allocations alike are tracked by the runtime)
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess && base) {
    const uint64_t lo = (uint64_t)(uintptr_t)base, hi = lo + size;
    if ((uint64_t)(uintptr_t)p < lo || (uint64_t)(uintptr_t)p + bytes > hi) {
      *err = what + ": range runs past the end of its allocation";
      return WT_E_RANGE;
    }
  } else {
    (void)hipGetLastError();
  }
  return WT_OK;
}

struct RealAddr : BatchAddr {
  const Layout *L;
  const Chunk *C;  // null for the direct batch
  uint64_t dst, staging;
  uint64_t seg_src(int32_t k, int32_t o, int32_t s) const override {
    if (C && C->h2d) return staging + (uint64_t)C->slot_off + (uint64_t)C->seg_stage[k][s];
    return (uint64_t)(uintptr_t)L->outs[o].segs[s].src;
  }
  uint64_t data_dst(int32_t k, int32_t o) const override {
    if (C && C->data_stage[k] >= 0) return staging + (uint64_t)C->slot_off + (uint64_t)C->data_stage[k];
    return dst + L->outs[o].dst_off;
  }
  uint64_t scale_dst(int32_t k, int32_t o) const override {
    if (C && C->scale_stage[k] >= 0) return staging + (uint64_t)C->slot_off + (uint64_t)C->scale_stage[k];
    return dst + L->outs[o].scale_off;
  }
};

size_t pad256(size_t x) { return (x + 255) & ~size_t(255); }

template <class T>
size_t blob_bytes(const std::vector<T> &v) {
  return pad256(v.size() * sizeof(T));
}

void destroy_resources(wt_plan *p) {
  if (p->ev_last) (void)hipEventSynchronize(p->ev_last);  // the tables are in use until then
  if (p->noalloc) {
    // the event and the scratch array belong to the device, not the plan
    p->ev_last = nullptr;
    p->noalloc->in_use.store(false);
    p->noalloc = nullptr;
  }
  if (p->s_prep) (void)hipStreamSynchronize(p->s_prep);
  if (p->s_out) (void)hipStreamSynchronize(p->s_out);
  if (p->s_h2d) (void)hipStreamSynchronize(p->s_h2d);
  for (auto *v : {&p->ev_h2d, &p->ev_prep, &p->ev_rel, &p->ev_done})
    for (hipEvent_t e : *v)
      if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : {p->ev_start, p->ev_out_end, p->ev_last})
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t s : {p->s_h2d, p->s_prep, p->s_out})
    if (s) (void)hipStreamDestroy(s);
  if (p->tables) (void)hipFree(p->tables);
  if (p->staging) (void)hipFree(p->staging);
}

wt_status create_impl(wt_plan *p, const wt_task *tasks, size_t n_tasks, const wt_plan_options &opts) {
  std::string err;
  // memory of every shard and of the destination region
  {
    wt_status st = check_memory(p->dst, p->dst_bytes, p->dst_kind, p->device, "destination region", &err);
    if (st != WT_OK) {
      set_err(p, err);
      return st;
    }
    if ((uintptr_t)p->dst % 16) {
      set_err(p, "destination region base not 16-byte aligned");
      return WT_E_ALIGN;
    }
    for (size_t i = 0; i < n_tasks; ++i)
      for (int32_t k = 0; k < tasks[i].n_shards; ++k) {
        const wt_shard &s = tasks[i].shards[k];
        st = check_memory(s.ptr, 2ull * (uint64_t)s.rows * (uint64_t)tasks[i].cols, tasks[i].shard_mem, p->device,
                          "task " + std::to_string(i) + " shard " + std::to_string(k), &err);
        if (st != WT_OK) {
          set_err(p, err);
          return st;
        }
      }
  }
  const Layout &L = p->L;
  p->pipeline = !L.chunks.empty();
  if (p->noalloc && (p->pipeline || L.staging_bytes > 0)) {
    set_err(p, "pinned-host shards and staged writes need staging memory, which a plan without allocation "
               "cannot have");
    return WT_E_INVAL;
  }

  if (L.staging_bytes > 0) HIP_OR(p, hipMalloc((void **)&p->staging, (size_t)L.staging_bytes));

  // host tables of every batch
  std::vector<HostTables> hts;
  RealAddr ra;
  ra.L = &L;
  ra.dst = (uint64_t)(uintptr_t)p->dst;
  ra.staging = (uint64_t)(uintptr_t)p->staging;
  if (!L.direct.empty()) {
    ra.C = nullptr;
    hts.emplace_back();
    build_tables(L, L.direct, ra, &hts.back());
    p->direct_batch = 0;
  }
  p->first_chunk_batch = (int)hts.size();
  for (const Chunk &C : L.chunks) {
    ra.C = &C;
    hts.emplace_back();
    build_tables(L, C.outputs, ra, &hts.back());
  }
  size_t total = 0;
  for (const HostTables &t : hts)
    total += blob_bytes(t.outs) + blob_bytes(t.segs) + blob_bytes(t.fast) + blob_bytes(t.edge) +
             blob_bytes(t.general) + blob_bytes(t.copies);
  const size_t epoch_off = total;
  total += 256;
  std::vector<uint8_t> blob(total, 0);  // zero-filled: the replay counter starts at 0
  uint8_t *base = nullptr;
  if (p->noalloc) {
    if (total > (size_t)WT_NOALLOC_TABLE_BYTES) {
      set_err(p, "device tables need " + std::to_string(total) + " bytes, above the " +
                     std::to_string((size_t)WT_NOALLOC_TABLE_BYTES) + " bytes a plan without allocation can hold");
      return WT_E_NOMEM;
    }
    base = p->noalloc->ptr;
  } else {
    HIP_OR(p, hipMalloc((void **)&p->tables, total));
    base = p->tables;
  }
  size_t off = 0;
  for (const HostTables &t : hts) {
    LaunchTables T{};
    auto put = [&](const auto &v) -> uint64_t {
      using E = typename std::decay_t<decltype(v)>::value_type;
      const uint64_t dev = (uint64_t)(uintptr_t)(base + off);
      if (!v.empty()) std::memcpy(blob.data() + off, v.data(), v.size() * sizeof(E));
      off += blob_bytes(v);
      return dev;
    };
    T.outs = (const DevOut *)(uintptr_t)put(t.outs);
    T.segs = (const DevSeg *)(uintptr_t)put(t.segs);
    T.fast_tiles = (const RegDesc *)(uintptr_t)put(t.fast);
    T.edge_tiles = (const TileItem *)(uintptr_t)put(t.edge);
    T.general_tiles = (const GenDesc *)(uintptr_t)put(t.general);
    T.copies = (const CopyItem *)(uintptr_t)put(t.copies);
    if (t.fast.size() > UINT32_MAX / 2 || t.edge.size() > UINT32_MAX / 2 || t.general.size() > UINT32_MAX / 2 ||
        t.copies.size() > UINT32_MAX / 2) {
      set_err(p, "work list too large for one launch");
      return WT_E_INVAL;
    }
    T.n_fast = (uint32_t)t.fast.size();
    T.n_edge = (uint32_t)t.edge.size();
    T.n_general = (uint32_t)t.general.size();
    T.n_copies = (uint32_t)t.copies.size();
    T.xcd_order = t.xcd_order ? 1u : 0u;
    p->batches.push_back(T);
  }
  p->epoch = (uint64_t *)(base + epoch_off);
  HIP_OR(p, hipMemcpy(base, blob.data(), total, hipMemcpyHostToDevice));

  if (p->noalloc)
    p->ev_last = p->noalloc->ev;
  else if (!p->pipeline)
    HIP_OR(p, hipEventCreateWithFlags(&p->ev_last, p->dst_kind == WT_MEM_DEVICE ? kReplayEventFlags
                                                                             : hipEventDisableTiming));
  if (p->pipeline) {
    HIP_OR(p, hipStreamCreateWithFlags(&p->s_h2d, hipStreamNonBlocking));
    HIP_OR(p, hipStreamCreateWithFlags(&p->s_prep, hipStreamNonBlocking));
    HIP_OR(p, hipStreamCreateWithFlags(&p->s_out, hipStreamNonBlocking));
    const size_t nc = L.chunks.size();
    p->ev_h2d.assign(nc, nullptr);
    p->ev_prep.assign(nc, nullptr);
    p->ev_rel.assign(nc, nullptr);
    for (size_t c = 0; c < nc; ++c) {
      HIP_OR(p, hipEventCreateWithFlags(&p->ev_h2d[c], hipEventDisableTiming));
      HIP_OR(p, hipEventCreateWithFlags(&p->ev_prep[c], hipEventDisableTiming));
      HIP_OR(p, hipEventCreateWithFlags(&p->ev_rel[c], hipEventDisableTiming));
    }
    HIP_OR(p, hipEventCreateWithFlags(&p->ev_start, hipEventDisableTiming));
    HIP_OR(p, hipEventCreateWithFlags(&p->ev_out_end, hipEventDisableTiming));
    p->ev_done.assign(L.max_replays_in_flight, nullptr);
    for (hipEvent_t &e : p->ev_done) HIP_OR(p, hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  return WT_OK;
}

wt_status prepare_impl(wt_plan *p, hipStream_t user) {
  const Layout &L = p->L;
  const bool progress = p->progress != nullptr;
  if (p->pipeline) {
    // a pipelined replay waits on the host (backpressure): not possible inside stream capture
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_OR(p, hipStreamIsCapturing(user, &cs));
    if (cs != hipStreamCaptureStatusNone) {
      set_err(p, "a pipelined plan cannot be replayed under stream capture");
      return WT_E_STATE;
    }
  }
  if (!p->pipeline) {
    HIP_OR(p, launch_batch(p->batches[p->direct_batch], user, p->device));
    if (progress) HIP_OR(p, launch_progress_mark(p->epoch, p->progress, true, user));
    HIP_OR(p, hipEventRecord(p->ev_last, user));
    return WT_OK;
  }
  const int unit_base = p->direct_batch >= 0 ? 1 : 0;
  // a chunk's release is recorded only when a later chunk waits for it
  std::vector<char> &waited = p->rel_waited;
  if (waited.size() != L.chunks.size()) {
    waited.assign(L.chunks.size(), 0);
    for (const Chunk &C : L.chunks)
      if (C.wait_for >= 0) waited[C.wait_for] = 1;
  }
  const bool staged = L.dst_mode == WT_DST_STAGED;
  const hipMemcpyKind out_kind = p->dst_kind == WT_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost;

  // Backpressure: before enqueueing replay r the host waits for replay
  // r - D to finish (D = max_replays_in_flight, default 1). The runtime
  // otherwise throttles deep queues of copies by blocking single
  // hipMemcpyAsync calls for milliseconds, in lockstep with the GPU, which
  // left the copy engine idle between chunks. Measured on MI355X with the
  // pinned-host MLA stack: with D = 2, 17 chunks per replay ran back to back
  // at the speed of a replay from idle but 33 chunks took 58 ms per replay
  // instead of 33.5 (one call held for 121 ms); waiting for each chunk
  // instead of each replay was slower still.
  const uint64_t r = p->replays;
  const size_t D = p->ev_done.size();
  if (r >= D) HIP_OR(p, hipEventSynchronize(p->ev_done[r % D]));
  // Order after the caller's prior work and after this plan's previous replay.
  HIP_OR(p, hipEventRecord(p->ev_start, user));
  for (hipStream_t s : {p->s_h2d, p->s_prep, p->s_out}) {
    HIP_OR(p, hipStreamWaitEvent(s, p->ev_start, 0));
    if (r > 0) HIP_OR(p, hipStreamWaitEvent(s, p->ev_done[(r - 1) % D], 0));
  }
  if (p->direct_batch >= 0) {
    HIP_OR(p, launch_batch(p->batches[p->direct_batch], p->s_prep, p->device));
    if (progress) HIP_OR(p, launch_progress_mark(p->epoch, p->progress, true, p->s_prep));
  }

  for (size_t c = 0; c < L.chunks.size(); ++c) {
    const Chunk &C = L.chunks[c];
    if (C.h2d) {
      // stage 1: host-to-device copy, admitted once the slot it reuses is released
      if (C.wait_for >= 0) HIP_OR(p, hipStreamWaitEvent(p->s_h2d, p->ev_rel[C.wait_for], 0));
      for (const H2DCopy &h : C.h2d_copies)
        HIP_OR(p, hipMemcpyAsync(p->staging + C.slot_off + h.stage_off, h.src, (size_t)h.bytes,
                                 hipMemcpyHostToDevice, p->s_h2d));
      HIP_OR(p, hipEventRecord(p->ev_h2d[c], p->s_h2d));
      HIP_OR(p, hipStreamWaitEvent(p->s_prep, p->ev_h2d[c], 0));
    } else if (C.wait_for >= 0) {
      HIP_OR(p, hipStreamWaitEvent(p->s_prep, p->ev_rel[C.wait_for], 0));
    }
    // stage 2: preparation (one launch over the chunk's work list)
    HIP_OR(p, launch_batch(p->batches[p->first_chunk_batch + c], p->s_prep, p->device));
    HIP_OR(p, hipEventRecord(p->ev_prep[c], p->s_prep));
    if (staged) {
      // stage 3: staging -> destination region (the emulated one-sided write)
      HIP_OR(p, hipStreamWaitEvent(p->s_out, p->ev_prep[c], 0));
      for (const DstCopy &d : C.dst_copies)
        HIP_OR(p, hipMemcpyAsync(p->dst + d.dst_off, p->staging + C.slot_off + d.stage_off, (size_t)d.bytes,
                                 out_kind, p->s_out));
      if (progress) HIP_OR(p, launch_progress_mark(p->epoch, p->progress + unit_base + c, unit_base + c == 0, p->s_out));
      if (waited[c]) HIP_OR(p, hipEventRecord(p->ev_rel[c], p->s_out));
    } else {
      if (progress) HIP_OR(p, launch_progress_mark(p->epoch, p->progress + unit_base + c, unit_base + c == 0, p->s_prep));
      if (waited[c]) HIP_OR(p, hipEventRecord(p->ev_rel[c], p->s_prep));
    }
  }
  // join: everything done -> ev_done on s_prep -> the caller's stream
  HIP_OR(p, hipEventRecord(p->ev_out_end, p->s_out));
  HIP_OR(p, hipStreamWaitEvent(p->s_prep, p->ev_out_end, 0));
  HIP_OR(p, hipEventRecord(p->ev_done[r % D], p->s_prep));
  HIP_OR(p, hipStreamWaitEvent(user, p->ev_done[r % D], 0));
  p->replays = r + 1;
  return WT_OK;
}

}  // namespace

extern "C" {

static wt_status plan_create(const wt_task *tasks, size_t n_tasks, void *dst, size_t dst_bytes, int32_t dst_kind,
                             const wt_plan_options *opts, bool noalloc, wt_plan **out) {
  if (!out) return WT_E_INVAL;
  *out = nullptr;
  wt_plan *p = nullptr;
  try {
    const wt_plan_options o = resolve_opts(opts);
    if (!dst || dst_bytes == 0) {
      set_err(nullptr, "destination region is empty");
      return WT_E_INVAL;
    }
    p = new wt_plan();
    std::string err;
    wt_status st = build_layout(tasks, n_tasks, dst_bytes, dst_kind, o, &p->L, &err);
    if (st != WT_OK) {
      set_err(nullptr, err);
      delete p;
      return st;
    }
    int dev = o.device;
    if (dev < 0) {
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) {
        set_err(nullptr, hip_msg("hipGetDevice", e));
        delete p;
        return WT_E_HIP;
      }
    }
    p->device = dev;
    p->dst = (uint8_t *)dst;
    p->dst_bytes = dst_bytes;
    p->dst_kind = dst_kind;
    DeviceGuard guard(dev);
    if (noalloc) {
      NoAllocDev *d = noalloc_device(dev, &err);
      if (!d) {
        set_err(nullptr, err);
        delete p;
        return WT_E_HIP;
      }
      bool expected = false;
      if (!d->in_use.compare_exchange_strong(expected, true)) {
        set_err(nullptr, "another plan without allocation is live on device " + std::to_string(dev) +
                             " (one per device: its tables occupy the device's scratch array)");
        delete p;
        return WT_E_STATE;
      }
      p->noalloc = d;
    }
    st = create_impl(p, tasks, n_tasks, o);
    if (st != WT_OK) {
      set_err(nullptr, p->last_error);
      destroy_resources(p);
      delete p;
      return st;
    }
    *out = p;
    return WT_OK;
  } catch (const std::bad_alloc &) {
    set_err(nullptr, "host allocation failed");
    if (p) {
      destroy_resources(p);
      delete p;
    }
    return WT_E_NOMEM;
  } catch (...) {
    set_err(nullptr, "internal error");
    if (p) {
      destroy_resources(p);
      delete p;
    }
    return WT_E_INVAL;
  }
}

wt_status wt_plan_create(const wt_task *tasks, size_t n_tasks, void *dst, size_t dst_bytes, int32_t dst_kind,
                         const wt_plan_options *opts, wt_plan **out) {
  return plan_create(tasks, n_tasks, dst, dst_bytes, dst_kind, opts, false, out);
}

wt_status wt_plan_create_noalloc(const wt_task *tasks, size_t n_tasks, void *dst, size_t dst_bytes, int32_t dst_kind,
                                 const wt_plan_options *opts, wt_plan **out) {
  return plan_create(tasks, n_tasks, dst, dst_bytes, dst_kind, opts, true, out);
}

wt_status wt_prepare(wt_plan *plan, void *stream) {
  if (!plan) return WT_E_INVAL;
  bool expected = false;
  if (!plan->busy.compare_exchange_strong(expected, true)) {
    set_err(plan, "wt_prepare already running on this plan");
    return WT_E_STATE;
  }
  wt_status st;
  try {
    DeviceGuard guard(plan->device);
    st = prepare_impl(plan, (hipStream_t)stream);
  } catch (...) {
    set_err(plan, "internal error");
    st = WT_E_INVAL;
  }
  plan->busy.store(false);
  return st;
}

wt_status wt_plan_get_info(const wt_plan *plan, wt_plan_info *info) {
  if (!plan || !info) return WT_E_INVAL;
  *info = plan->L.info;
  return WT_OK;
}

wt_status wt_plan_set_progress(wt_plan *plan, uint64_t *words, size_t n_words) {
  if (!plan) return WT_E_INVAL;
  bool expected = false;
  if (!plan->busy.compare_exchange_strong(expected, true)) {
    set_err(plan, "wt_prepare running on this plan");
    return WT_E_STATE;
  }
  wt_status st = WT_OK;
  try {
    DeviceGuard guard(plan->device);
    const size_t need = (size_t)plan->L.info.n_units;
    std::string err;
    if (!words) {
      plan->progress = nullptr;
    } else if ((uintptr_t)words % 8) {
      set_err(plan, "progress words not 8-byte aligned");
      st = WT_E_INVAL;
    } else if (n_words < need) {
      set_err(plan, "progress words: " + std::to_string(n_words) + " given, " + std::to_string(need) + " units");
      st = WT_E_INVAL;
    } else if ((st = check_memory(words, 8 * need, WT_MEM_PINNED_HOST, plan->device, "progress words", &err)) !=
               WT_OK) {
      set_err(plan, err);
    } else {
      // reset the replay counter; no replay of this plan is in flight
      const uint64_t zero = 0;
      hipError_t e = hipMemcpy(plan->epoch, &zero, sizeof zero, hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        set_err(plan, hip_msg("hipMemcpy(epoch)", e));
        st = WT_E_HIP;
      } else {
        plan->progress = words;
      }
    }
  } catch (...) {
    set_err(plan, "internal error");
    st = WT_E_INVAL;
  }
  plan->busy.store(false);
  return st;
}

wt_status wt_plan_task_unit(const wt_plan *plan, size_t task, int32_t *unit) {
  if (!plan || !unit || task >= plan->L.task_unit.size()) return WT_E_INVAL;
  *unit = plan->L.task_unit[task];
  return WT_OK;
}

wt_status wt_quantize_act_b128(const void *x, int64_t n_rows, int64_t cols, int64_t x_row_stride,
                               const int32_t *row_index, int64_t n_out, void *q, int64_t q_row_stride,
                               void *scales, int64_t scale_row_stride, void *stream) {
  auto bad = [](const char *m, wt_status st = WT_E_INVAL) {
    set_err(nullptr, std::string("wt_quantize_act_b128: ") + m);
    return st;
  };
  if (n_rows < 0 || n_out < 0) return bad("negative row count");
  if (cols < 1 || cols >= ((int64_t)1 << 31)) return bad("cols out of range");
  const int64_t nb = (cols + 127) / 128;
  if (x_row_stride < cols || q_row_stride < cols || scale_row_stride < 4 * nb) return bad("row stride too small");
  if (n_out == 0) return WT_OK;
  if (n_out > (((int64_t)1 << 31) - 1) / nb) return bad("n_out * ceil(cols / 128) >= 2^31");
  if (!q || !scales || (n_rows > 0 && !x)) return bad("NULL pointer");
  if (n_rows > 0 && (uint64_t)(n_rows - 1) > (UINT64_MAX / 2 - (uint64_t)cols) / (uint64_t)x_row_stride)
    return bad("x extent overflows");
  if ((uintptr_t)x % 2) return bad("x not 2-byte aligned", WT_E_ALIGN);
  if ((uintptr_t)scales % 4 || scale_row_stride % 4) return bad("scales not 4-byte aligned", WT_E_ALIGN);
  ActArgs a{};
  a.x = (uint64_t)(uintptr_t)x;
  a.index = (uint64_t)(uintptr_t)row_index;
  a.q = (uint64_t)(uintptr_t)q;
  a.s = (uint64_t)(uintptr_t)scales;
  a.n_rows = n_rows;
  a.cols = cols;
  a.x_stride = x_row_stride;
  a.q_stride = q_row_stride;
  a.s_stride = scale_row_stride;
  a.nb = (uint32_t)nb;
  a.n_blocks = (uint32_t)(n_out * nb);
  const bool fast = cols % 8 == 0 && x_row_stride % 8 == 0 && q_row_stride % 8 == 0 && (uintptr_t)x % 16 == 0 &&
                    (uintptr_t)q % 8 == 0;
  const hipError_t e = launch_act_quant(a, fast, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_err(nullptr, hip_msg("wt_quantize_act_b128 launch", e));
    return WT_E_HIP;
  }
  return WT_OK;
}

void wt_plan_destroy(wt_plan *plan) {
  if (!plan) return;
  {
    DeviceGuard guard(plan->device);
    destroy_resources(plan);
  }
  delete plan;
}

wt_status wt_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, int32_t path, uint8_t *out, void *stream) {
  if (n_amax < 0 || n_amax > (int64_t)1 << 20 || (path != 0 && path != 1)) return WT_E_INVAL;
  if (n_amax == 0) return WT_OK;
  if (!amax_bits || !out) return WT_E_INVAL;
  hipError_t e = launch_quantize_domain(amax_bits, n_amax, out, path, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_err(nullptr, hip_msg("quantize_domain launch", e));
    return WT_E_HIP;
  }
  return WT_OK;
}

wt_status wt_cast_f32_range(uint32_t first, uint64_t count, uint8_t *out, void *stream) {
  if (count > (1ull << 32)) return WT_E_INVAL;
  if (count == 0) return WT_OK;
  if (!out) return WT_E_INVAL;
  hipError_t e = launch_cast_range(first, count, out, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_err(nullptr, hip_msg("cast_range launch", e));
    return WT_E_HIP;
  }
  return WT_OK;
}

}  // extern "C"
