// moe_ffn_ws.h -- layout of the expert-FFN workspace (int32), shared by the tile schedule and
// the grouped GEMMs (bf16 and MX).
#pragma once

namespace moe_ffn_ws {

constexpr int kXcds = 8;  // gfx950: workgroup w runs on XCD w % 8
// [0] tile count; [8 + x] FC1 item counter of XCD x, [16 + x] FC2's; [24] FC1 / [25] FC2
// finished-workgroup counters; from [32]: max_blocks block indices sorted by expert, then the
// tiles, 7 ints each (expert, first row and row count of half 0, first row and row count of
// half 1 (count 0 = no half 1), the expert's first tile and its tile count).
// [1] error word of the last tile schedule (the FFN_ERR_* bits of the blocks it skipped).
constexpr int WS_NTILES = 0, WS_ERR = 1, WS_CTR_FC1 = 8, WS_CTR_FC2 = 16, WS_DONE_FC1 = 24,
              WS_DONE_FC2 = 25;
constexpr int WS_HEAD = 32;
constexpr int TILE_INTS = 7;
constexpr int HALF = 128;  // rows per tile half
// The largest block the FFN takes (the plan's largest block_m): with it, an expert's pieces
// number at most twice its blocks, so the tiles fit the workspace's 2 * max_blocks records.
constexpr int kMaxBlockRows = 256;
// Error bits of a block table entry (rank, expert, first row, rows) the FFN skips: expert
// outside [0, E_loc), rows outside [0, kMaxBlockRows], rows outside [0, max_rows); and
// n_blocks outside [0, max_blocks] (clamped).  A block with 0 rows is skipped silently.
constexpr int FFN_ERR_EXPERT = 1, FFN_ERR_ROWS = 2, FFN_ERR_RANGE = 4, FFN_ERR_COUNT = 8;

// Items of one expert are taken in groups of up to kGroupTiles tiles, column tile by column
// tile within a group: the items in flight on an XCD then share a few A tiles and a few B
// column tiles, which stay in its L2 instead of being fetched again from HBM.
#ifndef GROUP_TILES
#define GROUP_TILES 4
#endif
constexpr int kGroupTiles = GROUP_TILES;

}  // namespace moe_ffn_ws
