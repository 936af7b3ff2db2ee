// wt_internal.h -- descriptor tables shared by the host plan builder and the
// HIP kernels of libwt.so. Plain structs, identical layout on host and device.
#pragma once

#include <cstdint>

namespace wt {

constexpr int kTile = 128;            // FP8 scale tile edge (128 x 128 elements)
constexpr uint32_t kCopyItemMax = 16384;  // bytes per copy work item (one wave each)

// Output flags.
enum : int32_t {
  kOutFast = 1,  // cols % 8 == 0, cols < 2^24, data base 8-byte aligned, every segment 16-byte aligned
};

// One FP8 output tensor of a launch.
struct DevOut {
  uint64_t q;       // address of FP8 byte (0, 0) of the output
  uint64_t s;       // address of the fp32 scale grid
  int64_t rows;     // R (fused rows)
  int32_t cols;     // C
  int32_t tiles_c;  // ceil(C / 128)
  int32_t flags;
  int32_t pad0;
  int64_t pad1;
};
static_assert(sizeof(DevOut) == 48, "DevOut layout");

// A run of output rows [row0, row_end) read from one shard, rows contiguous
// with stride cols (BF16). src is the address of output row row0.
struct DevSeg {
  uint64_t src;
  int64_t row0;
  int64_t row_end;
  int64_t pad;
};
static_assert(sizeof(DevSeg) == 32, "DevSeg layout");

// One 128 x 128 tile of an FP8 output. seg = index of the first segment of
// the output that overlaps the tile's rows.
struct TileItem {
  uint32_t out;
  uint32_t tile_row;
  uint32_t tile_col;
  uint32_t seg;
};
static_assert(sizeof(TileItem) == 16, "TileItem layout");

// One tile of the general path, every address resolved at plan time.
struct GenDesc {
  uint64_t src;       // BF16 address of element (0, 0) when all rows come from one shard, else 0
  uint64_t q;         // FP8 address of element (0, 0)
  uint64_t s;         // address of the tile's scale
  uint32_t C;         // row length in elements (BF16 and FP8 rows alike)
  uint16_t nr;        // rows in the tile (<= 128)
  uint16_t w;         // columns in the tile (<= 128)
  uint32_t tile_row;  // for the segment walk when src == 0
  uint32_t tile_col;
  uint32_t seg;       // first segment that can hold the tile's rows
  uint32_t pad;
};
static_assert(sizeof(GenDesc) == 48, "GenDesc layout");

// One regular tile (full 128 x 128, rows from one shard, aligned output),
// with every address resolved at plan time: one scalar load per tile.
struct RegDesc {
  uint64_t src;  // BF16 address of the tile's element (0, 0)
  uint64_t q;    // FP8 address of the tile's element (0, 0)
  uint64_t s;    // address of the tile's scale
  uint32_t C;    // row length in elements (< 2^24)
  uint32_t flags;  // kRegStream: read with non-temporal loads
};
static_assert(sizeof(RegDesc) == 32, "RegDesc layout");
constexpr uint32_t kRegStream = 1;
constexpr uint32_t kRegPair = 2;  // the descriptor covers tiles (I, J) and (I, J + 1)
constexpr uint32_t kRegQuad = 4;  // the descriptor covers tiles (I, J) .. (I, J + 3)

// Up to this many adjacent full tiles of a row band (1, 2 or 4) are prepared
// by one workgroup; the plan emits groups no larger than this and the kernel
// compiles only those paths (a larger group needs more registers). Measured
// on MI355X with streaming loads, ms per launch for 1 / 2 / 4 tiles: Kimi-K2
// MoE share 2.146 / 2.006 / 2.253, 7B dense 3.245 / 3.097 / 3.387 (four
// tiles need 94 VGPRs, which caps a compute unit at two workgroups).
#ifndef WT_GROUP_TILES
#define WT_GROUP_TILES 2
#endif
constexpr int kGroupTiles = WT_GROUP_TILES;
static_assert(kGroupTiles == 1 || kGroupTiles == 2 || kGroupTiles == 4, "tiles per group");

// One byte-range copy (BF16 pass-through). width = 16, 4 or 2: src, dst and
// bytes are all multiples of width.
struct CopyItem {
  uint64_t src;
  uint64_t dst;
  uint32_t bytes;
  uint32_t width;
  uint64_t pad;
};
static_assert(sizeof(CopyItem) == 32, "CopyItem layout");

// Device tables of one launch batch.
struct LaunchTables {
  const DevOut *outs;
  const DevSeg *segs;
  const RegDesc *fast_tiles;      // regular tiles of kOutFast outputs: full, rows from one shard
  const TileItem *edge_tiles;     // other tiles of kOutFast outputs: partial, or rows from several shards
  const GenDesc *general_tiles;   // tiles of the other outputs
  const CopyItem *copies;
  uint32_t n_fast;
  uint32_t n_edge;
  uint32_t n_general;
  uint32_t n_copies;
  // 1: aligned-path work items go to XCDs in contiguous ranges (set when an
  // output's rows do not start on 128-byte lines, so that neighbouring tiles
  // share lines)
  uint32_t xcd_order;
  uint32_t pad;
};

// Arguments of the block-scaled activation quantization (one launch).
struct ActArgs {
  uint64_t x;         // BF16 rows, x_stride elements apart
  uint64_t index;     // int32 output-row -> input-row map, or 0
  uint64_t q;         // FP8 rows, q_stride bytes apart
  uint64_t s;         // fp32 scale rows, s_stride bytes apart
  int64_t n_rows;
  int64_t cols;
  int64_t x_stride;
  int64_t q_stride;
  int64_t s_stride;
  uint32_t nb;        // blocks per row, ceil(cols / 128)
  uint32_t n_blocks;  // n_out * nb < 2^31
};

}  // namespace wt
