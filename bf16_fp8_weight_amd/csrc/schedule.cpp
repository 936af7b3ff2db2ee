// schedule.cpp -- the static schedule builder ("Weight transfer for RL
// post-training in under 2 seconds", section "High-level workflow": the
// controller collects parameter metadata from training and inference and
// computes a static transfer schedule; section "Static schedule": computed
// once at initialisation, replayed every step). Host only: name matching,
// fusion groups, destination packing, source assignment, task tables.
#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <unordered_map>
#include <vector>

#include "wt.h"
#include "wt_internal.h"

namespace wt {
void set_thread_error(const std::string &msg);  // host_api.cpp
}

struct wt_schedule {
  struct Param {
    std::string name;
    int64_t rows = 0, cols = 0;
    int32_t shard_mem = WT_MEM_DEVICE;
    std::vector<const void *> ptrs;  // empty: planned without memory
    std::vector<int64_t> shard_rows;
  };
  struct Out {
    std::string name;
    std::vector<int32_t> comps;  // indices into params
    int32_t dtype = WT_FP8_E4M3FN_B128;
    int64_t rows = 0, cols = 0;
    uint64_t dst_offset = 0, scale_offset = 0;
    uint64_t input_bytes = 0;
    int32_t source = 0;
  };
  std::vector<Param> params;
  std::vector<Out> outs;
  uint64_t dst_bytes = 0;
  size_t n_unused = 0;
  int32_t n_sources = 1;
};

namespace {

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

wt_status fail(const std::string &msg) {
  wt::set_thread_error(msg);
  return WT_E_INVAL;
}

// torch.chunk-style dim-0 split into exactly n shards.
std::vector<int64_t> split_rows(int64_t rows, int32_t n) {
  std::vector<int64_t> out(n, 0);
  const int64_t per = rows ? (rows + n - 1) / n : 0;
  int64_t left = rows;
  for (int32_t k = 0; k < n; ++k) {
    out[k] = std::min(per, left);
    left -= out[k];
  }
  return out;
}

wt_status build(const wt_param_meta *params, size_t n_params, const wt_dst_meta *dsts, size_t n_dsts,
                const wt_schedule_options &o, wt_schedule *S) {
  if (!params && n_params) return fail("params is NULL");
  if (!dsts || n_dsts == 0) return fail("no inference tensors");
  const uint64_t align = o.align ? o.align : 256;
  if (align < 16 || (align & (align - 1))) return fail("align must be a power of two >= 16");
  S->n_sources = o.n_sources ? o.n_sources : 1;
  if (S->n_sources < 1 || S->n_sources > 65536) return fail("n_sources out of range");

  std::unordered_map<std::string, int32_t> by_name;
  for (size_t i = 0; i < n_params; ++i) {
    const wt_param_meta &m = params[i];
    const std::string where = "parameter " + std::to_string(i) + ": ";
    if (!m.name) return fail(where + "NULL name");
    if (m.rows < 1 || m.cols < 1 || m.cols > (int64_t)INT32_MAX || m.rows > ((int64_t)1 << 40))
      return fail(where + "shape out of range");
    if (m.n_shards < 1 || m.n_shards > (1 << 20)) return fail(where + "n_shards out of range");
    if (m.shard_mem != WT_MEM_DEVICE && m.shard_mem != WT_MEM_PINNED_HOST) return fail(where + "bad shard_mem");
    wt_schedule::Param P;
    P.name = m.name;
    if (!by_name.emplace(P.name, (int32_t)i).second) return fail("duplicate parameter name '" + P.name + "'");
    P.rows = m.rows;
    P.cols = m.cols;
    P.shard_mem = m.shard_mem;
    P.shard_rows = split_rows(m.rows, m.n_shards);
    if (m.shard_ptrs) P.ptrs.assign(m.shard_ptrs, m.shard_ptrs + m.n_shards);
    S->params.push_back(std::move(P));
  }

  std::vector<char> used(n_params, 0);
  uint64_t cursor = 0;
  for (size_t d = 0; d < n_dsts; ++d) {
    const wt_dst_meta &m = dsts[d];
    const std::string where = "inference tensor " + std::to_string(d) + ": ";
    if (!m.name) return fail(where + "NULL name");
    if (m.n_components < 1 || !m.components) return fail(where + "no components");
    if (m.dtype != WT_FP8_E4M3FN_B128 && m.dtype != WT_BF16_COPY) return fail(where + "bad dtype");
    wt_schedule::Out O;
    O.name = m.name;
    O.dtype = m.dtype;
    for (int32_t c = 0; c < m.n_components; ++c) {
      if (!m.components[c]) return fail(where + "NULL component name");
      auto it = by_name.find(m.components[c]);
      if (it == by_name.end()) return fail(where + "unknown training parameter '" + std::string(m.components[c]) + "'");
      const wt_schedule::Param &P = S->params[it->second];
      if (c > 0 && P.cols != O.cols) return fail(where + "fusion components differ in cols");
      if (c > 0 && P.shard_mem != S->params[O.comps[0]].shard_mem)
        return fail(where + "fusion components differ in shard memory");
      O.cols = P.cols;
      O.rows += P.rows;
      O.comps.push_back(it->second);
      used[it->second] = 1;
    }
    const uint64_t elems = (uint64_t)O.rows * (uint64_t)O.cols;
    O.input_bytes = 2 * elems;
    // packing: data, then (FP8) the scale grid, each aligned
    cursor = align_up(cursor, align);
    O.dst_offset = cursor;
    cursor += O.dtype == WT_FP8_E4M3FN_B128 ? elems : 2 * elems;
    if (O.dtype == WT_FP8_E4M3FN_B128) {
      cursor = align_up(cursor, align);
      O.scale_offset = cursor;
      const uint64_t tiles = (uint64_t)((O.rows + wt::kTile - 1) / wt::kTile) * (uint64_t)((O.cols + wt::kTile - 1) / wt::kTile);
      cursor += 4 * tiles;
    }
    S->outs.push_back(std::move(O));
  }
  S->dst_bytes = align_up(cursor, align);
  S->n_unused = (size_t)std::count(used.begin(), used.end(), 0);

  // sources: longest processing time first over input bytes, ties to the
  // lower tensor index and then to the lower source index
  std::vector<size_t> order(S->outs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return S->outs[a].input_bytes > S->outs[b].input_bytes; });
  std::vector<uint64_t> load(S->n_sources, 0);
  for (size_t i : order) {
    int32_t best = 0;
    for (int32_t s = 1; s < S->n_sources; ++s)
      if (load[s] < load[best]) best = s;
    S->outs[i].source = best;
    load[best] += S->outs[i].input_bytes;
  }
  return WT_OK;
}

}  // namespace

extern "C" {

wt_status wt_schedule_build(const wt_param_meta *params, size_t n_params, const wt_dst_meta *dsts, size_t n_dsts,
                            const wt_schedule_options *opts, wt_schedule **out) {
  if (!out) return WT_E_INVAL;
  *out = nullptr;
  wt_schedule_options o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  wt_schedule *S = nullptr;
  try {
    S = new wt_schedule();
    const wt_status st = build(params, n_params, dsts, n_dsts, o, S);
    if (st != WT_OK) {
      delete S;
      return st;
    }
    *out = S;
    return WT_OK;
  } catch (const std::bad_alloc &) {
    delete S;
    wt::set_thread_error("host allocation failed");
    return WT_E_NOMEM;
  } catch (...) {
    delete S;
    wt::set_thread_error("internal error");
    return WT_E_INVAL;
  }
}

wt_status wt_schedule_info(const wt_schedule *S, size_t *n_tasks, size_t *n_shards, uint64_t *dst_bytes,
                           size_t *n_unused_params) {
  if (!S) return WT_E_INVAL;
  size_t t = 0, sh = 0;
  for (const auto &O : S->outs)
    for (int32_t c : O.comps) {
      ++t;
      sh += S->params[c].shard_rows.size();
    }
  if (n_tasks) *n_tasks = t;
  if (n_shards) *n_shards = sh;
  if (dst_bytes) *dst_bytes = S->dst_bytes;
  if (n_unused_params) *n_unused_params = S->n_unused;
  return WT_OK;
}

wt_status wt_schedule_output(const wt_schedule *S, size_t i, uint64_t *dst_offset, uint64_t *scale_offset,
                             int32_t *source, uint64_t *input_bytes) {
  if (!S || i >= S->outs.size()) return WT_E_INVAL;
  const auto &O = S->outs[i];
  if (dst_offset) *dst_offset = O.dst_offset;
  if (scale_offset) *scale_offset = O.scale_offset;
  if (source) *source = O.source;
  if (input_bytes) *input_bytes = O.input_bytes;
  return WT_OK;
}

wt_status wt_schedule_tasks(const wt_schedule *S, int32_t source, wt_task *tasks, size_t max_tasks, wt_shard *shards,
                            size_t max_shards, size_t *n_tasks, size_t *n_shards_out) {
  if (!S || source < -1 || source >= S->n_sources) return WT_E_INVAL;
  size_t t = 0, sh = 0;
  for (const auto &O : S->outs) {
    if (source >= 0 && O.source != source) continue;
    for (int32_t c : O.comps) {
      ++t;
      sh += S->params[c].shard_rows.size();
    }
  }
  if (n_tasks) *n_tasks = t;
  if (n_shards_out) *n_shards_out = sh;
  if (t > max_tasks || sh > max_shards || (t && (!tasks || !shards))) return WT_E_RANGE;
  size_t ti = 0, si = 0;
  for (size_t d = 0; d < S->outs.size(); ++d) {
    const auto &O = S->outs[d];
    if (source >= 0 && O.source != source) continue;
    for (int32_t c : O.comps) {
      const auto &P = S->params[c];
      wt_task &T = tasks[ti++];
      std::memset(&T, 0, sizeof T);
      T.shards = shards + si;
      T.n_shards = (int32_t)P.shard_rows.size();
      T.shard_mem = P.shard_mem;
      T.cols = P.cols;
      T.dtype = O.dtype;
      T.fusion_group = O.comps.size() > 1 ? (int32_t)d : -1;
      T.dst_offset = O.dst_offset;
      T.scale_offset = O.scale_offset;
      for (size_t k = 0; k < P.shard_rows.size(); ++k) {
        shards[si].ptr = P.ptrs.empty() ? nullptr : P.ptrs[k];
        shards[si].rows = P.shard_rows[k];
        ++si;
      }
    }
  }
  return WT_OK;
}

void wt_schedule_destroy(wt_schedule *S) { delete S; }

}  // extern "C"
