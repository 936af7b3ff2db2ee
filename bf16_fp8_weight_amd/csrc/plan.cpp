// plan.cpp -- host-only part of the static schedule ("Weight transfer for RL
// post-training in under 2 seconds", section "Static schedule": computed once
// at initialisation, replayed every iteration): task-table validation,
// assembly/fusion as row segments, pipeline chunks and their staging slots
// ("GPU memory usage control": in-flight temporary memory stays under a
// configurable watermark), and the per-launch work lists.
#include "plan.h"

#include <algorithm>
#include <cstring>
#include <map>

namespace wt {
namespace {

constexpr uint64_t kStageAlign = 16;   // staging keeps each range's address congruent mod 16
constexpr uint64_t kSlotAlign = 256;   // chunk slots start on 256-byte boundaries

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Offset >= cursor that is congruent to `addr` modulo kStageAlign.
int64_t congruent_at(int64_t cursor, uint64_t addr) {
  int64_t base = (int64_t)align_up((uint64_t)cursor, kStageAlign);
  return base + (int64_t)(addr % kStageAlign);
}

struct Interval {
  uint64_t lo, hi;  // [lo, hi)
  int32_t task;
  bool scale;
};

wt_status fail(std::string *err, wt_status st, const std::string &msg) {
  if (err) *err = msg;
  return st;
}

}  // namespace

void add_copy_items(std::vector<CopyItem> &v, uint64_t src, uint64_t dst, uint64_t bytes) {
  auto width_of = [](uint64_t s, uint64_t d, uint64_t n) -> uint32_t {
    for (uint32_t w : {16u, 4u, 2u})
      if (s % w == 0 && d % w == 0 && n % w == 0) return w;
    return 1u;
  };
  while (bytes > 0) {
    // Same misalignment on both sides: peel a short head so the body is 16-byte aligned.
    if ((src & 15) == (dst & 15) && (src & 15) != 0) {
      uint64_t head = std::min<uint64_t>(bytes, 16 - (src & 15));
      v.push_back(CopyItem{src, dst, (uint32_t)head, width_of(src, dst, head), 0});
      src += head, dst += head, bytes -= head;
      continue;
    }
    uint64_t n = std::min<uint64_t>(bytes, kCopyItemMax);
    if ((src & 15) == 0 && (dst & 15) == 0 && n >= 16) n &= ~uint64_t(15);
    v.push_back(CopyItem{src, dst, (uint32_t)n, width_of(src, dst, n), 0});
    src += n, dst += n, bytes -= n;
  }
}

wt_status build_layout(const wt_task *tasks, size_t n_tasks, size_t dst_bytes, int32_t dst_kind,
                       const wt_plan_options &opts, Layout *L, std::string *err) {
  *L = Layout{};
  if (n_tasks == 0) return fail(err, WT_E_INVAL, "empty task table");
  if (!tasks) return fail(err, WT_E_INVAL, "tasks is NULL");
  if (dst_kind != WT_MEM_DEVICE && dst_kind != WT_MEM_PINNED_HOST)
    return fail(err, WT_E_INVAL, "dst_kind must be WT_MEM_DEVICE or WT_MEM_PINNED_HOST");
  if (opts.dst_write_mode != WT_DST_ZERO_COPY && opts.dst_write_mode != WT_DST_STAGED)
    return fail(err, WT_E_INVAL, "dst_write_mode must be WT_DST_ZERO_COPY or WT_DST_STAGED");
  const uint64_t watermark = opts.watermark_bytes;
  if (watermark == 0) return fail(err, WT_E_INVAL, "watermark_bytes is 0");
  L->dst_mode = opts.dst_write_mode;
  if (opts.load_hint > WT_LOAD_STREAM) return fail(err, WT_E_INVAL, "load_hint out of range");
  L->load_hint = opts.load_hint;
  if (opts.max_replays_in_flight > 8) return fail(err, WT_E_INVAL, "max_replays_in_flight above 8");
  if (opts.tile_group > WT_GROUP_PAIR) return fail(err, WT_E_INVAL, "tile_group out of range");
  L->tile_group = opts.tile_group;
  L->max_replays_in_flight = opts.max_replays_in_flight ? opts.max_replays_in_flight : 1;

  // ---- per-task checks, grouping into outputs (first appearance order)
  std::map<int32_t, int32_t> group_out;
  std::vector<std::vector<int32_t>> out_tasks;
  for (size_t i = 0; i < n_tasks; ++i) {
    const wt_task &t = tasks[i];
    const std::string where = "task " + std::to_string(i) + ": ";
    if (t.n_shards < 1 || !t.shards) return fail(err, WT_E_INVAL, where + "needs at least one shard");
    if (t.cols < 1 || t.cols > (int64_t)INT32_MAX) return fail(err, WT_E_INVAL, where + "cols out of range");
    if (t.dtype != WT_FP8_E4M3FN_B128 && t.dtype != WT_BF16_COPY) return fail(err, WT_E_INVAL, where + "bad dtype");
    if (t.shard_mem != WT_MEM_DEVICE && t.shard_mem != WT_MEM_PINNED_HOST)
      return fail(err, WT_E_INVAL, where + "bad shard_mem");
    if (t.fusion_group < -1) return fail(err, WT_E_INVAL, where + "fusion_group must be >= -1");
    for (int32_t k = 0; k < t.n_shards; ++k) {
      const wt_shard &s = t.shards[k];
      if (s.rows < 0) return fail(err, WT_E_INVAL, where + "negative shard rows");
      if (s.rows > 0 && !s.ptr) return fail(err, WT_E_INVAL, where + "NULL shard pointer");
      if (s.rows > 0 && ((uintptr_t)s.ptr & 1)) return fail(err, WT_E_ALIGN, where + "shard pointer not 2-byte aligned");
      if (s.rows > (int64_t)1 << 40) return fail(err, WT_E_INVAL, where + "shard too large");
    }
    if (t.fusion_group < 0) {
      out_tasks.push_back({(int32_t)i});
    } else {
      auto it = group_out.find(t.fusion_group);
      if (it == group_out.end()) {
        group_out[t.fusion_group] = (int32_t)out_tasks.size();
        out_tasks.push_back({(int32_t)i});
      } else {
        const wt_task &f = tasks[out_tasks[it->second][0]];
        if (f.cols != t.cols || f.dtype != t.dtype || f.shard_mem != t.shard_mem)
          return fail(err, WT_E_INVAL, where + "fusion group members differ in cols, dtype or shard_mem");
        out_tasks[it->second].push_back((int32_t)i);
      }
    }
  }

  // ---- outputs: rows, segments, byte counts, destination ranges
  std::vector<Interval> ranges;
  for (size_t o = 0; o < out_tasks.size(); ++o) {
    const wt_task &f = tasks[out_tasks[o][0]];
    HostOutput H;
    H.dtype = f.dtype;
    H.mem = f.shard_mem;
    H.first_task = out_tasks[o][0];
    H.cols = f.cols;
    H.dst_off = f.dst_offset;
    H.scale_off = f.scale_offset;
    int64_t row = 0;
    for (int32_t ti : out_tasks[o])
      for (int32_t k = 0; k < tasks[ti].n_shards; ++k) {
        const wt_shard &s = tasks[ti].shards[k];
        if (s.rows > 0) H.segs.push_back(HostSeg{s.ptr, row, s.rows});
        row += s.rows;
      }
    H.rows = row;
    const std::string where = "output of task " + std::to_string(H.first_task) + ": ";
    if (H.rows < 1) return fail(err, WT_E_INVAL, where + "has no rows");
    if ((uint64_t)H.rows * (uint64_t)H.cols > ((uint64_t)1 << 46)) return fail(err, WT_E_INVAL, where + "too large");
    const uint64_t elems = (uint64_t)H.rows * (uint64_t)H.cols;
    H.in_bytes = (int64_t)(2 * elems);
    if (H.dtype == WT_FP8_E4M3FN_B128) {
      H.tiles_r = ceil_div(H.rows, kTile);
      H.tiles_c = ceil_div(H.cols, kTile);
      if (H.tiles_r > (int64_t)UINT32_MAX) return fail(err, WT_E_INVAL, where + "too many tile rows");
      H.data_bytes = (int64_t)elems;
      H.scale_bytes = 4 * H.tiles_r * H.tiles_c;
      if (H.scale_off % 4) return fail(err, WT_E_ALIGN, where + "scale_offset not a multiple of 4");
    } else {
      H.data_bytes = (int64_t)(2 * elems);
      if (H.dst_off % 2) return fail(err, WT_E_ALIGN, where + "BF16 dst_offset not even");
    }
    if (H.dst_off > dst_bytes || (uint64_t)H.data_bytes > dst_bytes - H.dst_off)
      return fail(err, WT_E_RANGE, where + "data range outside the destination region");
    ranges.push_back(Interval{H.dst_off, H.dst_off + (uint64_t)H.data_bytes, H.first_task, false});
    if (H.dtype == WT_FP8_E4M3FN_B128) {
      if (H.scale_off > dst_bytes || (uint64_t)H.scale_bytes > dst_bytes - H.scale_off)
        return fail(err, WT_E_RANGE, where + "scale range outside the destination region");
      ranges.push_back(Interval{H.scale_off, H.scale_off + (uint64_t)H.scale_bytes, H.first_task, true});
    }
    L->outs.push_back(std::move(H));
  }
  std::sort(ranges.begin(), ranges.end(), [](const Interval &a, const Interval &b) { return a.lo < b.lo; });
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].lo < ranges[i - 1].hi)
      return fail(err, WT_E_OVERLAP,
                  "destination ranges of tasks " + std::to_string(ranges[i - 1].task) + " and " +
                      std::to_string(ranges[i].task) + " overlap");

  // ---- batches: direct launch vs pipeline chunks
  const bool staged = opts.dst_write_mode == WT_DST_STAGED;
  std::vector<int32_t> piped;
  for (size_t o = 0; o < L->outs.size(); ++o) {
    if (!staged && L->outs[o].mem == WT_MEM_DEVICE)
      L->direct.push_back((int32_t)o);
    else
      piped.push_back((int32_t)o);
  }

  // Upper bound of one output's staging need (alignment slack included).
  auto need_of = [&](const HostOutput &H) -> int64_t {
    int64_t n = 0;
    if (H.mem == WT_MEM_PINNED_HOST) n += H.in_bytes + (int64_t)kStageAlign * (int64_t)(H.segs.size() + 1);
    if (staged) n += H.data_bytes + H.scale_bytes + 4 * (int64_t)kStageAlign;
    return (int64_t)align_up((uint64_t)n, kSlotAlign);
  };
  // Default chunk size: about kTargetChunks chunks per replay, at least 32 MiB,
  // and small enough that the ring holds one slot per stage that keeps a
  // chunk's staging busy (host-to-device copy, prepare, destination copy):
  // at most watermark / 2, or watermark / 3 when host-resident shards are
  // staged in and outputs staged out. Measured on MI355X with the pinned-host
  // MLA stack (1.72 GB, H2D-bound, bare copy 30.0 ms), one replay in flight:
  // 17 chunks 30.8 ms per replay, 40 chunks 31.2 ms; staged into pinned host
  // memory under a 256 MiB watermark, 24 chunks capped at watermark / 2 took
  // 46.1 ms (two slots for three stages), 33 chunks of 64 MiB 33.7 ms.
  int64_t piped_need = 0;
  bool any_h2d = false;
  for (int32_t o : piped) {
    piped_need += need_of(L->outs[o]);
    any_h2d |= L->outs[o].mem == WT_MEM_PINNED_HOST;
  }
  const int64_t busy_stages = (any_h2d && staged) ? 3 : 2;
  constexpr int64_t kTargetChunks = 16;
  const int64_t chunk_target =
      opts.chunk_bytes ? (int64_t)opts.chunk_bytes
                       : std::max<int64_t>(std::min<int64_t>(std::max<int64_t>(piped_need / kTargetChunks, 32ll << 20),
                                                             (int64_t)watermark / busy_stages),
                                           1);

  for (int32_t o : piped) {
    const int64_t need = need_of(L->outs[o]);
    if ((uint64_t)need > watermark)
      return fail(err, WT_E_WATERMARK,
                  "watermark " + std::to_string(watermark) + " below the staging need " + std::to_string(need) +
                      " of the output of task " + std::to_string(L->outs[o].first_task));
    const bool h2d = L->outs[o].mem == WT_MEM_PINNED_HOST;
    bool open_new = L->chunks.empty() || L->chunks.back().h2d != h2d;
    if (!open_new) {
      int64_t cur = 0;
      for (int32_t p : L->chunks.back().outputs) cur += need_of(L->outs[p]);
      open_new = cur + need > chunk_target;
    }
    if (open_new) {
      L->chunks.emplace_back();
      L->chunks.back().h2d = h2d;
    }
    L->chunks.back().outputs.push_back(o);
  }

  // ---- staging placement inside each chunk slot, copies, ring placement
  int64_t cursor_ring = 0;
  int64_t staging_hi = 0;
  for (size_t c = 0; c < L->chunks.size(); ++c) {
    Chunk &C = L->chunks[c];
    int64_t cur = 0;
    // inputs: host segments in order; host-adjacent segments stay adjacent
    const void *prev_end = nullptr;
    int64_t prev_stage_end = -1;
    for (int32_t o : C.outputs) {
      const HostOutput &H = L->outs[o];
      C.in_bytes += H.in_bytes;
      std::vector<int64_t> st;
      if (C.h2d) {
        for (const HostSeg &s : H.segs) {
          const int64_t bytes = 2 * s.nrows * H.cols;
          int64_t off;
          if (s.src == prev_end && prev_stage_end >= 0) {
            off = prev_stage_end;
            C.h2d_copies.back().bytes += bytes;
          } else {
            off = congruent_at(cur, (uint64_t)(uintptr_t)s.src);
            C.h2d_copies.push_back(H2DCopy{s.src, off, bytes});
          }
          st.push_back(off);
          cur = off + bytes;
          prev_end = (const char *)s.src + bytes;
          prev_stage_end = cur;
        }
      }
      C.seg_stage.push_back(std::move(st));
    }
    // outputs (staged mode): ranges in destination order; dst-adjacent ranges stay adjacent
    C.data_stage.assign(C.outputs.size(), -1);
    C.scale_stage.assign(C.outputs.size(), -1);
    if (staged) {
      struct R { uint64_t dst; int64_t bytes; size_t k; bool scale; };
      std::vector<R> rs;
      for (size_t k = 0; k < C.outputs.size(); ++k) {
        const HostOutput &H = L->outs[C.outputs[k]];
        rs.push_back(R{H.dst_off, H.data_bytes, k, false});
        if (H.dtype == WT_FP8_E4M3FN_B128) rs.push_back(R{H.scale_off, H.scale_bytes, k, true});
      }
      std::sort(rs.begin(), rs.end(), [](const R &a, const R &b) { return a.dst < b.dst; });
      uint64_t prev_dst_end = UINT64_MAX;
      int64_t prev_end = -1;
      for (const R &r : rs) {
        int64_t off;
        if (r.dst == prev_dst_end && prev_end >= 0) {
          off = prev_end;
          C.dst_copies.back().bytes += r.bytes;
        } else {
          off = congruent_at(cur, r.dst);
          C.dst_copies.push_back(DstCopy{off, r.dst, r.bytes});
        }
        (r.scale ? C.scale_stage : C.data_stage)[r.k] = off;
        cur = off + r.bytes;
        prev_dst_end = r.dst + (uint64_t)r.bytes;
        prev_end = cur;
      }
    }
    C.slot_bytes = (int64_t)align_up((uint64_t)std::max<int64_t>(cur, 1), kSlotAlign);
    if ((uint64_t)C.slot_bytes > watermark)
      return fail(err, WT_E_WATERMARK, "chunk staging exceeds the watermark");
    // ring: next free offset, wrapping to 0 when the slot would pass the watermark
    int64_t off = cursor_ring;
    if ((uint64_t)(off + C.slot_bytes) > watermark) off = 0;
    C.slot_off = off;
    cursor_ring = off + C.slot_bytes;
    staging_hi = std::max(staging_hi, cursor_ring);
    // the latest earlier chunk whose slot overlaps ours must be released first
    for (int64_t j = (int64_t)c - 1; j >= 0; --j) {
      const Chunk &P = L->chunks[j];
      if (P.slot_off < C.slot_off + C.slot_bytes && C.slot_off < P.slot_off + P.slot_bytes) {
        C.wait_for = (int32_t)j;
        break;
      }
    }
  }
  L->staging_bytes = staging_hi;

  // ---- info
  wt_plan_info &I = L->info;
  I.n_tasks = (int64_t)n_tasks;
  I.n_outputs = (int64_t)L->outs.size();
  for (const HostOutput &H : L->outs) {
    (H.dtype == WT_FP8_E4M3FN_B128 ? I.n_fp8_outputs : I.n_copy_outputs) += 1;
    I.n_tiles += H.tiles_r * H.tiles_c;
    I.input_bytes += H.in_bytes;
    I.output_bytes += H.data_bytes + H.scale_bytes;
  }
  I.n_chunks = (int64_t)L->chunks.size();
  for (const Chunk &C : L->chunks) {
    I.n_h2d_copies += (int64_t)C.h2d_copies.size();
    I.n_dst_copies += (int64_t)C.dst_copies.size();
  }
  I.staging_bytes = L->staging_bytes;

  // completion units: the direct launch first (when present), then each chunk
  {
    const int32_t base = L->direct.empty() ? 0 : 1;
    std::vector<int32_t> out_unit(L->outs.size(), 0);
    for (size_t c = 0; c < L->chunks.size(); ++c)
      for (int32_t o : L->chunks[c].outputs) out_unit[o] = base + (int32_t)c;
    L->task_unit.assign(n_tasks, 0);
    for (size_t o = 0; o < out_tasks.size(); ++o)
      for (int32_t t : out_tasks[o]) L->task_unit[t] = out_unit[o];
    I.n_units = base + (int64_t)L->chunks.size();
  }

  // Launch count: resolve addresses against aligned virtual bases (the
  // destination and staging bases are 256-byte aligned in a real plan).
  struct VirtAddr : BatchAddr {
    const Layout *L;
    const Chunk *C;
    uint64_t seg_src(int32_t k, int32_t o, int32_t s) const override {
      if (C && C->h2d) return (uint64_t)C->slot_off + (uint64_t)C->seg_stage[k][s];
      return (uint64_t)(uintptr_t)L->outs[o].segs[s].src;
    }
    uint64_t data_dst(int32_t k, int32_t o) const override {
      if (C && C->data_stage[k] >= 0) return (uint64_t)C->slot_off + (uint64_t)C->data_stage[k];
      return L->outs[o].dst_off;
    }
    uint64_t scale_dst(int32_t k, int32_t o) const override {
      if (C && C->scale_stage[k] >= 0) return (uint64_t)C->slot_off + (uint64_t)C->scale_stage[k];
      return L->outs[o].scale_off;
    }
  };
  VirtAddr va;
  va.L = L;
  if (!L->direct.empty()) {
    va.C = nullptr;
    HostTables t;
    build_tables(*L, L->direct, va, &t);
    I.n_launches += launches_for(t);
    I.n_regular_items += (int64_t)t.fast.size();
    I.n_edge_tiles += (int64_t)t.edge.size();
    I.n_general_tiles += (int64_t)t.general.size();
  }
  for (const Chunk &C : L->chunks) {
    va.C = &C;
    HostTables t;
    build_tables(*L, C.outputs, va, &t);
    I.n_launches += launches_for(t);
    I.n_regular_items += (int64_t)t.fast.size();
    I.n_edge_tiles += (int64_t)t.edge.size();
    I.n_general_tiles += (int64_t)t.general.size();
  }
  return WT_OK;
}



// Whether full tiles are read with non-temporal loads. Measured on MI355X
// with tile pairs and non-temporal stores, ms per launch, plain vs streaming
// loads: Kimi-K2-shaped MoE share 2.050 vs 2.015, 7B-shaped dense model 3.165
// vs 3.106, MLA attention stack 0.444 vs 0.421. (With one tile per
// workgroup the MoE share preferred plain loads, 2.075 vs 2.146.) The default
// streams.
static bool stream_loads(uint32_t hint) { return hint != WT_LOAD_PLAIN; }

// Full tiles in a launch at or below which WT_GROUP_AUTO takes single tiles:
// one round of workgroups on MI355X (256 compute units x 3 workgroups). Such
// a launch is latency-bound, and single tiles halve each workgroup's chain.
// Measured on MI355X, one dense layer of hidden size 1024 (720 tiles): 14.2 us
// per launch in pairs, 12.8 us as single tiles.
constexpr int64_t kOneRoundTiles = 256 * 3;

void build_tables(const Layout &L, const std::vector<int32_t> &outputs, const BatchAddr &addr, HostTables *t) {
  *t = HostTables{};
  // tiles of aligned-path outputs in this launch (an upper bound of its full tiles)
  int64_t batch_tiles = 0;
  for (int32_t o : outputs)
    if (L.outs[o].dtype != WT_BF16_COPY) batch_tiles += L.outs[o].tiles_r * L.outs[o].tiles_c;
  const int group = L.tile_group == WT_GROUP_SINGLE ? 1
                    : L.tile_group == WT_GROUP_PAIR ? std::min(kGroupTiles, 2)
                    : batch_tiles <= kOneRoundTiles ? 1
                                                    : kGroupTiles;
  for (size_t k = 0; k < outputs.size(); ++k) {
    const int32_t o = outputs[k];
    const HostOutput &H = L.outs[o];
    if (H.dtype == WT_BF16_COPY) {
      const uint64_t base = addr.data_dst((int32_t)k, o);
      for (size_t s = 0; s < H.segs.size(); ++s) {
        const uint64_t bytes = 2ull * (uint64_t)H.segs[s].nrows * (uint64_t)H.cols;
        add_copy_items(t->copies, addr.seg_src((int32_t)k, o, (int32_t)s),
                       base + 2ull * (uint64_t)H.segs[s].row0 * (uint64_t)H.cols, bytes);
      }
      continue;
    }
    const uint32_t out_idx = (uint32_t)t->outs.size();
    const uint32_t seg_base = (uint32_t)t->segs.size();
    DevOut d{};
    d.q = addr.data_dst((int32_t)k, o);
    d.s = addr.scale_dst((int32_t)k, o);
    d.rows = H.rows;
    d.cols = (int32_t)H.cols;
    d.tiles_c = (int32_t)H.tiles_c;
    bool fast = (H.cols % 8 == 0) && (H.cols < (1 << 24)) && (d.q % 8 == 0);
    for (size_t s = 0; s < H.segs.size(); ++s) {
      DevSeg g{};
      g.src = addr.seg_src((int32_t)k, o, (int32_t)s);
      g.row0 = H.segs[s].row0;
      g.row_end = H.segs[s].row0 + H.segs[s].nrows;
      if (g.src % 16) fast = false;
      t->segs.push_back(g);
    }
    d.flags = fast ? kOutFast : 0;
    t->outs.push_back(d);
    // a tile row is 256 bytes of BF16 and 128 of FP8: unless both row strides
    // and both bases are multiples of 128 bytes, the first and last line of
    // each tile row segment are shared with the neighbouring tiles
    if (fast && (H.cols % 128 != 0 || d.q % 128 != 0)) t->xcd_order = true;
    if (fast)
      for (size_t s2 = 0; s2 < H.segs.size(); ++s2)
        if (t->segs[seg_base + s2].src % 128 != 0) t->xcd_order = true;
    size_t s = 0;
    for (int64_t I = 0; I < H.tiles_r; ++I) {
      while (s + 1 < H.segs.size() && H.segs[s].row0 + H.segs[s].nrows <= I * kTile) ++s;
      const bool full_rows = (I + 1) * kTile <= H.rows;
      const bool one_seg = H.segs[s].row0 + H.segs[s].nrows >= std::min<int64_t>((I + 1) * kTile, H.rows);
      for (int64_t J = 0; J < H.tiles_c; ++J) {
        const bool full = full_rows && (J + 1) * kTile <= H.cols;
        const TileItem item{out_idx, (uint32_t)I, (uint32_t)J, seg_base + (uint32_t)s};
        if (!fast) {
          GenDesc gd{};
          gd.q = d.q + (uint64_t)(I * kTile) * (uint64_t)H.cols + (uint64_t)(J * kTile);
          gd.s = d.s + 4 * ((uint64_t)I * (uint64_t)H.tiles_c + (uint64_t)J);
          gd.C = (uint32_t)H.cols;
          gd.nr = (uint16_t)std::min<int64_t>(kTile, H.rows - I * kTile);
          gd.w = (uint16_t)std::min<int64_t>(kTile, H.cols - J * kTile);
          gd.tile_row = (uint32_t)I;
          gd.tile_col = (uint32_t)J;
          gd.seg = seg_base + (uint32_t)s;
          if (one_seg) {
            const DevSeg &g = t->segs[seg_base + s];
            gd.src = g.src + 2 * ((uint64_t)(I * kTile - g.row0) * (uint64_t)H.cols + (uint64_t)(J * kTile));
          }
          t->general.push_back(gd);
        } else if (!(full && one_seg)) {
          t->edge.push_back(item);
        } else {
          const DevSeg &g = t->segs[seg_base + s];
          RegDesc r{};
          r.src = g.src + 2 * ((uint64_t)(I * kTile - g.row0) * (uint64_t)H.cols + (uint64_t)(J * kTile));
          r.q = d.q + (uint64_t)(I * kTile) * (uint64_t)H.cols + (uint64_t)(J * kTile);
          r.s = d.s + 4 * ((uint64_t)I * (uint64_t)H.tiles_c + (uint64_t)J);
          r.C = (uint32_t)H.cols;
          r.flags = stream_loads(L.load_hint) ? kRegStream : 0;
          // the next tiles of the row band are full too (same rows, same segment): one descriptor for a group
          if (group >= 4 && (J + 4) * kTile <= H.cols) {
            r.flags |= kRegQuad;
            J += 3;
          } else if (group >= 2 && (J + 2) * kTile <= H.cols) {
            r.flags |= kRegPair;
            J += 1;
          }
          t->fast.push_back(r);
        }
      }
    }
  }
}

int launches_for(const HostTables &t) {
  return ((t.fast.size() + t.edge.size() + t.copies.size()) > 0 ? 1 : 0) + (t.general.empty() ? 0 : 1);
}

void schedule_ops(const Layout &L, std::vector<wt_sched_op> *ops) {
  ops->clear();
  if (!L.direct.empty()) {
    int64_t in = 0;
    for (int32_t o : L.direct) in += L.outs[o].in_bytes;
    ops->push_back(wt_sched_op{1, -1, -1, 0, in, 0, 0});
  }
  for (size_t c = 0; c < L.chunks.size(); ++c) {
    const Chunk &C = L.chunks[c];
    if (C.h2d) {
      int64_t b = 0;
      for (const H2DCopy &h : C.h2d_copies) b += h.bytes;
      ops->push_back(wt_sched_op{0, (int32_t)c, C.wait_for, 0, b, C.slot_off, C.slot_bytes});
    }
    ops->push_back(wt_sched_op{1, (int32_t)c, C.h2d ? -1 : C.wait_for, 0, C.in_bytes, C.slot_off, C.slot_bytes});
    if (L.dst_mode == WT_DST_STAGED) {
      int64_t b = 0;
      for (const DstCopy &d : C.dst_copies) b += d.bytes;
      ops->push_back(wt_sched_op{2, (int32_t)c, -1, 0, b, C.slot_off, C.slot_bytes});
    }
  }
}

}  // namespace wt
