// Column decomposition of a schedule (host only, no HIP): every item is cut
// into chunks at multiples of a chunk length, and each chunk lists the earlier
// chunks it must follow; all of them lie in its own column of elements, so a
// column's chunks can run in schedule order independently of other columns.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace hbmc {

struct ColumnChunk {
  uint64_t begin = 0;     // first element
  uint32_t count = 0;     // elements
  uint32_t item = 0;      // index into the plan's item table (all steps, in order)
  uint32_t step = 0;
  uint32_t dep_lo = 0, dep_hi = 0;  // range of deps[] (chunk indices, all of earlier steps)
};

// Chunks are cut at multiples of chunk_elems of the element index.  Every
// step combines operands at equal element offsets, so a chunk depends only on
// chunks over the same elements: the chunks of one "column" (elements
// [g*chunk_elems, (g+1)*chunk_elems)) form a dependency graph of their own,
// and running a column's chunks in ascending index (step by step) honours it.
struct ColumnTable {
  std::vector<ColumnChunk> chunks;       // step after step, item after item, ascending begin
  std::vector<uint32_t> deps;
  std::vector<uint32_t> step_first;    // chunks of step s: [step_first[s], step_first[s+1])
  std::vector<uint32_t> col_list;      // column g's chunk indices, ascending: col_list[col_off[g] .. col_off[g+1])
  std::vector<uint32_t> col_off;
  uint64_t max_per_col = 0;            // chunks of the longest column (run one after another by one wave)
  uint64_t chunk_elems = 0;
  bool with_deps = false;
};

// Cut every item of `sched` at the multiples of `chunk_elems`, and derive each chunk's
// dependencies: for every rank range it reads, the last earlier chunk that
// wrote an overlapping range; for every range it writes, also each earlier
// chunk that read an overlapping range since that write.  Dependencies are
// direct only; waiting on them orders a chunk after everything they waited
// for.  A step's own accesses enter the history only after all its chunks are
// cut, so every dependency lies in an earlier step (a step's items never
// conflict).  Also builds the per-column chunk lists.  Returns false for a bad
// argument, a table beyond 2^32 entries, or a dependency across columns
// (impossible for element-aligned items).
// Without `with_deps` the dependency lists stay empty (the kernel does not
// need them: a column runs in index order).
bool build_columns(const Schedule& sched, int P, uint64_t chunk_elems, bool with_deps, ColumnTable* out);

}  // namespace hbmc
