// Tile tables of the flow kernel (host only).
#include "flow.hpp"

#include <algorithm>
#include <cstring>

namespace hbmc {

bool build_flow(const Schedule& sched, int first, int last, uint64_t count, uint32_t esize, uint64_t col_elems,
                FlowTable* out) {
  *out = FlowTable();
  if (col_elems == 0 || col_elems > UINT32_MAX) return false;
  if (first < 0 || last > static_cast<int>(sched.steps.size()) || first > last) return false;
  const uint64_t ncols = (count + col_elems - 1) / col_elems;
  if (ncols > UINT32_MAX) return false;
  out->col_elems = col_elems;
  out->ncols = static_cast<uint32_t>(ncols);
  std::vector<uint32_t> seq(ncols, 0);
  struct Cut {
    uint64_t col, begin, count;
    uint32_t item;
  };
  std::vector<Cut> cuts;
  uint32_t item_base = 0;
  for (int s = 0; s < first; ++s) item_base += static_cast<uint32_t>(sched.steps[s].items.size());
  for (int s = first; s < last; ++s) {
    const Step& st = sched.steps[s];
    cuts.clear();
    uint64_t write = 0;
    for (size_t i = 0; i < st.items.size(); ++i) {
      const Item& it = st.items[i];
      if (it.nsrc + it.ndst > kFlowOperands) return false;
      write += it.count * uint64_t(it.ndst) * esize;
      for (uint64_t b = it.begin; b < it.begin + it.count;) {
        const uint64_t g = b / col_elems;
        const uint64_t e = std::min(it.begin + it.count, (g + 1) * col_elems);
        cuts.push_back(Cut{g, b, e - b, item_base + static_cast<uint32_t>(i)});
        b = e;
      }
    }
    out->max_step_write = std::max(out->max_step_write, write);
    // columns ascending, items in order within a column
    std::stable_sort(cuts.begin(), cuts.end(), [](const Cut& a, const Cut& b) { return a.col < b.col; });
    for (size_t k = 0; k < cuts.size();) {
      const uint64_t g = cuts[k].col;
      FlowTile t;
      t.col = static_cast<uint32_t>(g);
      t.seq = seq[g]++;
      if (out->chunks.size() >= UINT32_MAX) return false;
      t.c_lo = static_cast<uint32_t>(out->chunks.size());
      for (; k < cuts.size() && cuts[k].col == g; ++k) {
        const Cut& c = cuts[k];
        const Item& it = st.items[c.item - item_base];
        FlowChunk ch;
        std::memset(&ch, 0, sizeof(ch));
        ch.begin = c.begin;
        ch.count = static_cast<uint32_t>(c.count);
        ch.shape = static_cast<uint32_t>(st.mode) | uint32_t(it.nsrc) << 8 | uint32_t(it.ndst) << 16;
        for (int q = 0; q < it.nsrc + it.ndst; ++q) ch.rank[q] = it.rank[q];
        out->chunks.push_back(ch);
        out->chunk_item.push_back(c.item);
      }
      t.c_hi = static_cast<uint32_t>(out->chunks.size());
      if (out->tiles.size() >= UINT32_MAX) return false;
      out->tiles.push_back(t);
      out->tile_step.push_back(static_cast<uint32_t>(s));
    }
    item_base += static_cast<uint32_t>(st.items.size());
  }
  return true;
}

}  // namespace hbmc
