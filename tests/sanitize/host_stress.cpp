// Host-side stress of libwt's plan logic for sanitizer builds (AddressSanitizer
// + UndefinedBehaviorSanitizer, ThreadSanitizer). Test infrastructure only.
//
// Each worker draws seeded random task tables -- ragged and tile-multiple
// shapes, 1..9 shards with empty ones, device and pinned-host shards, fusion
// groups, FP8 and BF16 outputs, packed or deliberately overlapping,
// misaligned or out-of-range offsets, small and large watermarks and chunk
// sizes, both write modes -- and runs wt_plan_check and wt_plan_schedule on
// them (no address is ever dereferenced: these calls only plan), then builds
// random static schedules (wt_schedule_build / info / output / tasks /
// destroy, including unknown and duplicate names). Results are checked for
// internal consistency: a table that validates has a schedule whose prepare
// launches cover its input bytes exactly, staging within the watermark.
//
// usage: host_stress ITERATIONS THREADS
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "wt.h"

namespace {

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    s ^= s << 13, s ^= s >> 7, s ^= s << 17;
    return s;
  }
  int64_t in(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
  bool p(int percent) { return (int)(next() % 100) < percent; }
};

int g_fail = 0;
// coverage counters (summed over threads at the end)
struct Counts {
  uint64_t accepted = 0, refused = 0, pipelined = 0, schedules = 0;
};
thread_local Counts t_counts;
Counts g_counts[64];

void fail(const char *what, uint64_t seed) {
  if (g_fail < 20) std::fprintf(stderr, "check failed (seed %llu): %s: %s\n", (unsigned long long)seed, what,
                                wt_plan_last_error(nullptr));
  ++g_fail;
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

void plan_case(uint64_t seed) {
  Rng r(seed);
  const int n_out = (int)r.in(1, 12);
  const bool host = r.p(40);
  std::vector<std::vector<wt_shard>> shards;
  std::vector<wt_task> tasks;
  uint64_t addr = 0x7f0000000000ull, dst = 0;
  const bool overlap = r.p(5), misalign = r.p(5), outside = r.p(5);
  int64_t in_bytes = 0;
  std::vector<size_t> first_task;  // per output
  std::vector<char> is_fp8;
  uint64_t end = 0;  // end of the last destination range
  for (int o = 0; o < n_out; ++o) {
    const bool fp8 = r.p(80);
    first_task.push_back(tasks.size());
    is_fp8.push_back(fp8);
    const int64_t cols = r.p(40) ? 128 * r.in(1, 24) : r.in(1, 3000);
    const int parts = r.p(30) ? (int)r.in(2, 3) : 1;
    const uint64_t data = dst;
    int64_t rows_total = 0;
    for (int p = 0; p < parts; ++p) {
      const int64_t rows = r.p(40) ? 128 * r.in(1, 16) : r.in(1, 3000);
      const int ns = (int)r.in(1, 9);
      std::vector<wt_shard> sh;
      const int64_t per = (rows + ns - 1) / ns;
      int64_t left = rows;
      for (int k = 0; k < ns; ++k) {
        const int64_t rk = left < per ? left : per;
        left -= rk;
        if (rk == 0) {
          sh.push_back(wt_shard{nullptr, 0});
          continue;
        }
        addr = align_up(addr, r.p(80) ? 256 : 2);
        sh.push_back(wt_shard{(const void *)(uintptr_t)addr, rk});
        addr += 2 * (uint64_t)rk * (uint64_t)cols;
      }
      shards.push_back(sh);
      rows_total += rows;
      wt_task t;
      std::memset(&t, 0, sizeof t);
      t.n_shards = ns;
      t.shard_mem = host ? WT_MEM_PINNED_HOST : WT_MEM_DEVICE;
      t.cols = cols;
      t.dtype = fp8 ? WT_FP8_E4M3FN_B128 : WT_BF16_COPY;
      t.fusion_group = parts > 1 ? o : -1;
      t.dst_offset = data;
      tasks.push_back(t);
    }
    in_bytes += 2 * rows_total * cols;
    const uint64_t db = fp8 ? (uint64_t)(rows_total * cols) : 2 * (uint64_t)(rows_total * cols);
    end = data + db;
    dst = align_up(data + db, r.p(80) ? 256 : 16);
    uint64_t sofs = 0;
    if (fp8) {
      sofs = dst;
      end = dst + 4 * (uint64_t)((rows_total + 127) / 128) * (uint64_t)((cols + 127) / 128);
      dst = align_up(end, 256);
    }
    for (int p = 0; p < parts; ++p) tasks[tasks.size() - parts + p].scale_offset = sofs;
  }
  size_t si = 0;
  for (wt_task &t : tasks) t.shards = shards[si++].data();
  // planted errors, each on a task whose offsets count (a group's first task)
  bool planted = false;
  if (overlap && n_out > 1) {
    tasks[first_task.back()].dst_offset = tasks[0].dst_offset;
    planted = true;
  }
  if (misalign) {
    for (int o = 0; o < n_out; ++o)
      if (is_fp8[o]) {
        tasks[first_task[o]].scale_offset += 2;
        planted = true;
        break;
      }
  }
  const uint64_t dst_bytes = outside ? end - 1 : dst + 64;
  planted |= outside;

  wt_plan_options o;
  wt_plan_options_init(&o);
  o.watermark_bytes = r.p(50) ? (uint64_t)r.in(1, 64) << 20 : 0;
  o.chunk_bytes = r.p(50) ? (uint64_t)r.in(1, 32) << 20 : 0;
  o.dst_write_mode = r.p(30) ? WT_DST_STAGED : WT_DST_ZERO_COPY;
  o.tile_group = (uint32_t)r.in(0, 2);
  o.load_hint = (uint32_t)r.in(0, 2);
  const int32_t kind = r.p(20) ? WT_MEM_PINNED_HOST : WT_MEM_DEVICE;

  wt_plan_info info;
  const wt_status st = wt_plan_check(tasks.data(), tasks.size(), dst_bytes, kind, &o, &info);
  ++(st == WT_OK ? t_counts.accepted : t_counts.refused);
  if (st == WT_OK && info.n_chunks > 0) ++t_counts.pipelined;
  if (st != WT_OK) {
    if (std::strlen(wt_plan_last_error(nullptr)) == 0) fail("error without a message", seed);
    if (!planted && st != WT_E_WATERMARK) fail("valid table refused", seed);
    return;
  }
  if (planted) fail("invalid table accepted", seed);
  if (info.input_bytes != in_bytes) fail("input bytes", seed);
  if ((uint64_t)info.staging_bytes > (o.watermark_bytes ? o.watermark_bytes : 512ull << 20)) fail("staging", seed);
  size_t n_ops = 0;
  if (wt_plan_schedule(tasks.data(), tasks.size(), dst_bytes, kind, &o, nullptr, 0, &n_ops) != WT_OK) {
    fail("schedule count", seed);
    return;
  }
  std::vector<wt_sched_op> ops(n_ops + 1);
  if (wt_plan_schedule(tasks.data(), tasks.size(), dst_bytes, kind, &o, ops.data(), n_ops, &n_ops) != WT_OK) {
    fail("schedule", seed);
    return;
  }
  int64_t prepared = 0;
  for (size_t i = 0; i < n_ops; ++i) {
    if (ops[i].stage == 1) prepared += ops[i].bytes;
    if (ops[i].staging_offset + ops[i].staging_bytes > info.staging_bytes && ops[i].staging_bytes > 0)
      fail("op outside staging", seed);
  }
  if (prepared != in_bytes) fail("prepare launches do not cover the input", seed);
}

void schedule_case(uint64_t seed) {
  Rng r(seed);
  const int np = (int)r.in(1, 40);
  std::vector<std::string> names;
  for (int i = 0; i < np; ++i) names.push_back("p" + std::to_string(i));
  if (r.p(5) && np > 1) names[1] = names[0];  // duplicate
  std::vector<wt_param_meta> pm(np);
  std::vector<int64_t> cols(np);
  std::vector<std::vector<const void *>> ptrs(np);
  uint64_t addr = 0x7e0000000000ull;
  for (int i = 0; i < np; ++i) {
    cols[i] = r.p(50) ? 128 * r.in(1, 8) : r.in(1, 500);
    const int64_t rows = r.in(r.p(3) ? 0 : 1, 2000);
    const int32_t ns = (int32_t)r.in(1, 9);
    for (int32_t k = 0; k < ns; ++k) {  // made-up shard addresses (never dereferenced)
      ptrs[i].push_back((const void *)(uintptr_t)addr);
      addr += align_up(2 * (uint64_t)(rows / ns + 1) * (uint64_t)cols[i], 256);
    }
    pm[i] = wt_param_meta{names[i].c_str(), rows, cols[i], ns, WT_MEM_DEVICE, r.p(90) ? ptrs[i].data() : nullptr};
  }
  const int nd = (int)r.in(1, np);
  std::vector<std::vector<const char *>> comps(nd);
  std::vector<std::string> dnames(nd);
  std::vector<wt_dst_meta> dm(nd);
  for (int d = 0; d < nd; ++d) {
    dnames[d] = "d" + std::to_string(d);
    comps[d].push_back(names[d].c_str());
    for (int j = d + 1; j < np && r.p(20); ++j)
      if (cols[j] == cols[d] || r.p(5)) comps[d].push_back(names[j].c_str());
    if (r.p(3)) comps[d].push_back("unknown");
    dm[d] = wt_dst_meta{dnames[d].c_str(), comps[d].data(), (int32_t)comps[d].size(),
                        r.p(80) ? WT_FP8_E4M3FN_B128 : WT_BF16_COPY};
  }
  wt_schedule_options so;
  std::memset(&so, 0, sizeof so);
  so.align = r.p(50) ? 256 : (uint64_t)1 << r.in(4, 12);
  so.n_sources = (int32_t)r.in(0, 16);
  wt_schedule *sch = nullptr;
  if (wt_schedule_build(pm.data(), pm.size(), dm.data(), dm.size(), &so, &sch) != WT_OK) {
    if (sch != nullptr) fail("schedule handle on failure", seed);
    if (std::strlen(wt_plan_last_error(nullptr)) == 0) fail("schedule error without a message", seed);
    return;
  }
  size_t nt = 0, ns = 0, nu = 0;
  uint64_t db = 0;
  ++t_counts.schedules;
  if (wt_schedule_info(sch, &nt, &ns, &db, &nu) != WT_OK) fail("schedule info", seed);
  for (size_t i = 0; i < dm.size(); ++i) {
    uint64_t d0 = 0, s0 = 0, ib = 0;
    int32_t src = 0;
    if (wt_schedule_output(sch, i, &d0, &s0, &src, &ib) != WT_OK) fail("schedule output", seed);
    if (d0 >= db || (s0 != 0 && s0 >= db)) fail("offset outside the region", seed);
  }
  const int32_t n_src = so.n_sources ? so.n_sources : 1;
  for (int32_t s = -1; s < n_src; ++s) {
    size_t t1 = 0, s1 = 0;
    wt_schedule_tasks(sch, s, nullptr, 0, nullptr, 0, &t1, &s1);  // sizes only (WT_E_RANGE)
    std::vector<wt_task> tt(t1 + 1);
    std::vector<wt_shard> ss(s1 + 1);
    if (wt_schedule_tasks(sch, s, tt.data(), tt.size(), ss.data(), ss.size(), &t1, &s1) != WT_OK)
      fail("schedule tasks", seed);
    bool with_ptrs = true;
    for (const wt_param_meta &m : pm) with_ptrs &= m.shard_ptrs != nullptr;
    wt_plan_info info;
    if (with_ptrs && t1 > 0 && wt_plan_check(tt.data(), t1, db, WT_MEM_DEVICE, nullptr, &info) != WT_OK)
      fail("scheduled table does not validate", seed);
  }
  wt_schedule_destroy(sch);
}

void worker(int t, uint64_t first, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) {
    plan_case(first + i);
    schedule_case(first + i);
  }
  g_counts[t] = t_counts;
}

}  // namespace

int main(int argc, char **argv) {
  const uint64_t iters = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 200;
  int threads = argc > 2 ? std::atoi(argv[2]) : 1;
  if (threads < 1 || threads > 64) threads = 1;
  std::vector<std::thread> ts;
  for (int t = 0; t < threads; ++t) ts.emplace_back(worker, t, 1000000ull * (uint64_t)(t + 1), iters);
  for (std::thread &t : ts) t.join();
  if (g_fail) return 1;
  Counts c;
  for (int t = 0; t < threads; ++t) {
    c.accepted += g_counts[t].accepted, c.refused += g_counts[t].refused;
    c.pipelined += g_counts[t].pipelined, c.schedules += g_counts[t].schedules;
  }
  std::printf("host stress ok: %llu tables x %d threads; %llu accepted (%llu pipelined), %llu refused, "
              "%llu schedules built\n", (unsigned long long)iters, threads, (unsigned long long)c.accepted,
              (unsigned long long)c.pipelined, (unsigned long long)c.refused, (unsigned long long)c.schedules);
  return 0;
}
