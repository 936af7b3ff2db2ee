// host_api.cpp -- the entry points of libwt.so that never touch a GPU: plan
// options, validation and shape of a task table (wt_plan_check), the list of
// operations one replay would enqueue (wt_plan_schedule), status texts, the
// calling thread's last error, and the host-side wait on a completion word.
// Separate from runtime.cpp so that the host logic also builds without HIP
// (the sanitizer builds of the tests link exactly this file, plan.cpp and
// schedule.cpp).
#include <chrono>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "plan.h"
#include "wt.h"

namespace wt {
namespace {
thread_local std::string g_last_error;
}  // namespace

void set_thread_error(const std::string &msg) { g_last_error = msg; }

wt_plan_options resolve_opts(const wt_plan_options *o) {
  wt_plan_options d;
  wt_plan_options_init(&d);
  if (!o) return d;
  wt_plan_options r = *o;
  if (r.watermark_bytes == 0) r.watermark_bytes = d.watermark_bytes;
  return r;
}
}  // namespace wt

using namespace wt;

extern "C" {

void wt_plan_options_init(wt_plan_options *opts) {
  if (!opts) return;
  std::memset(opts, 0, sizeof *opts);
  opts->watermark_bytes = 512ull << 20;
  opts->chunk_bytes = 0;
  opts->dst_write_mode = WT_DST_ZERO_COPY;
  opts->device = -1;
}

wt_status wt_plan_check(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                        const wt_plan_options *opts, wt_plan_info *info) {
  try {
    const wt_plan_options o = resolve_opts(opts);
    Layout L;
    std::string err;
    wt_status st = build_layout(tasks, n_tasks, dst_bytes, dst_kind, o, &L, &err);
    if (st != WT_OK) {
      set_thread_error(err);
      return st;
    }
    if (info) *info = L.info;
    return WT_OK;
  } catch (const std::bad_alloc &) {
    set_thread_error("host allocation failed");
    return WT_E_NOMEM;
  } catch (...) {
    set_thread_error("internal error");
    return WT_E_INVAL;
  }
}

wt_status wt_plan_schedule(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                           const wt_plan_options *opts, wt_sched_op *ops, size_t max_ops, size_t *n_ops) {
  try {
    if (!n_ops) return WT_E_INVAL;
    const wt_plan_options o = resolve_opts(opts);
    Layout L;
    std::string err;
    wt_status st = build_layout(tasks, n_tasks, dst_bytes, dst_kind, o, &L, &err);
    if (st != WT_OK) {
      set_thread_error(err);
      return st;
    }
    std::vector<wt_sched_op> v;
    schedule_ops(L, &v);
    *n_ops = v.size();
    if (ops)
      for (size_t i = 0; i < v.size() && i < max_ops; ++i) ops[i] = v[i];
    return WT_OK;
  } catch (const std::bad_alloc &) {
    set_thread_error("host allocation failed");
    return WT_E_NOMEM;
  } catch (...) {
    set_thread_error("internal error");
    return WT_E_INVAL;
  }
}

wt_status wt_progress_wait(const uint64_t *word, uint64_t target, uint64_t timeout_ns) {
  if (!word) return WT_E_INVAL;
  const auto t0 = std::chrono::steady_clock::now();
  for (uint32_t spin = 0;; ++spin) {
    if (__atomic_load_n(word, __ATOMIC_ACQUIRE) >= target) return WT_OK;
    if ((spin & 255u) == 0) {
      const auto dt = std::chrono::steady_clock::now() - t0;
      if ((uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(dt).count() >= timeout_ns) {
        return __atomic_load_n(word, __ATOMIC_ACQUIRE) >= target ? WT_OK : WT_E_TIMEOUT;
      }
    }
#if defined(__x86_64__)
    __builtin_ia32_pause();
#endif
  }
}

const char *wt_status_str(int status) {
  switch (status) {
    case WT_OK: return "WT_OK";
    case WT_E_INVAL: return "WT_E_INVAL: malformed task table or argument";
    case WT_E_RANGE: return "WT_E_RANGE: range outside the destination region or allocation";
    case WT_E_OVERLAP: return "WT_E_OVERLAP: destination ranges overlap";
    case WT_E_ALIGN: return "WT_E_ALIGN: misaligned pointer or offset";
    case WT_E_NOMEM: return "WT_E_NOMEM: allocation failed";
    case WT_E_HIP: return "WT_E_HIP: HIP runtime error";
    case WT_E_WATERMARK: return "WT_E_WATERMARK: watermark below one output's staging need";
    case WT_E_STATE: return "WT_E_STATE: plan busy";
    case WT_E_TIMEOUT: return "WT_E_TIMEOUT: progress word did not reach its target in time";
    default: return "unknown status";
  }
}

const char *wt_plan_last_error(const wt_plan *plan) {
  if (!plan) return g_last_error.c_str();
  return plan_error_text(plan);
}

}  // extern "C"
