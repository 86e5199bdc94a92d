// Tile tables of the flow kernel (host only, no HIP; see flow_kernels.hip).
#pragma once

#include <cstdint>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {

// Every item of every step is cut at the multiples of `col_elems` (columns);
// a tile is one step's chunks in one column.  Tiles are listed step after
// step, columns ascending within a step (the ticket order); a tile's seq
// counts the earlier tiles of its column, and its chunks are contiguous in
// the chunk table, in item order.
struct FlowTable {
  uint64_t col_elems = 0;
  uint32_t ncols = 0;
  std::vector<FlowTile> tiles;
  std::vector<uint32_t> tile_step;   // the step of each tile
  std::vector<FlowChunk> chunks;
  std::vector<uint32_t> chunk_item;  // each chunk's item, numbered over all steps in order
  uint64_t max_step_write = 0;       // most bytes one step writes (chooses the store hint)
};

// Build the table of steps [first, last) of `sched` over `count` elements of
// `esize` bytes (seq then counts from 0 within the range; items keep their
// numbers over all steps); false when an item has more than kFlowOperands
// operands or a count does not fit the records.
bool build_flow(const Schedule& sched, int first, int last, uint64_t count, uint32_t esize, uint64_t col_elems,
                FlowTable* out);

}  // namespace hbmc
