// Column decomposition of a schedule: chunks, their dependencies, per-column lists.
#include "columns.hpp"

#include <algorithm>
#include <iterator>
#include <map>

namespace hbmc {

namespace {

// Access history of one rank buffer: disjoint segments [start, end) with the
// last chunk that wrote them and the chunks that read them since.
struct Seg {
  uint64_t end;
  int64_t writer;
  std::vector<uint32_t> readers;
};

using History = std::map<uint64_t, Seg>;

// Make `x` a segment boundary.
void split(History& h, uint64_t x) {
  auto it = h.upper_bound(x);
  if (it == h.begin()) return;
  --it;
  if (it->first == x || it->second.end <= x) return;
  Seg tail = it->second;
  it->second.end = x;
  h.emplace(x, std::move(tail));
}

}  // namespace

bool build_columns(const Schedule& sched, int P, uint64_t chunk_elems, bool with_deps, ColumnTable* out) {
  if (chunk_elems == 0 || P < 1 || P > kMaxRanks) return false;
  out->chunks.clear();
  out->deps.clear();
  out->step_first.clear();
  out->chunk_elems = chunk_elems;
  out->with_deps = with_deps;
  std::vector<History> hist(with_deps ? P : 0);
  for (size_t r = 0; r < hist.size(); ++r) hist[r].emplace(0, Seg{UINT64_MAX, -1, {}});

  uint64_t item_index = 0;
  std::vector<uint32_t> d;
  for (size_t s = 0; s < sched.steps.size(); ++s) {
    const Step& step = sched.steps[s];
    out->step_first.push_back(static_cast<uint32_t>(out->chunks.size()));
    const size_t step_lo = out->chunks.size();
    // dependencies of all of this step's chunks first, then the step's
    // accesses enter the history (the step's chunks are mutually independent)
    for (const Item& it : step.items) {
      for (uint64_t b = it.begin; b < it.begin + it.count;) {
        const uint64_t e = std::min(it.begin + it.count, (b / chunk_elems + 1) * chunk_elems);
        ColumnChunk ch;
        ch.begin = b;
        ch.count = static_cast<uint32_t>(e - b);
        ch.item = static_cast<uint32_t>(item_index);
        ch.step = static_cast<uint32_t>(s);
        d.clear();
        for (int k = 0; with_deps && k < it.nsrc + it.ndst; ++k) {
          const bool write = k >= it.nsrc;
          History& h = hist[it.rank[k]];
          auto seg = h.upper_bound(b);
          --seg;
          for (; seg != h.end() && seg->first < e; ++seg) {
            if (seg->second.end <= b) continue;
            if (seg->second.writer >= 0) d.push_back(static_cast<uint32_t>(seg->second.writer));
            if (write) d.insert(d.end(), seg->second.readers.begin(), seg->second.readers.end());
          }
        }
        std::sort(d.begin(), d.end());
        d.erase(std::unique(d.begin(), d.end()), d.end());
        if (out->deps.size() + d.size() > UINT32_MAX || out->chunks.size() >= UINT32_MAX) return false;
        ch.dep_lo = static_cast<uint32_t>(out->deps.size());
        out->deps.insert(out->deps.end(), d.begin(), d.end());
        ch.dep_hi = static_cast<uint32_t>(out->deps.size());
        for (uint32_t dj : d)
          if (out->chunks[dj].begin / chunk_elems != b / chunk_elems) return false;
        out->chunks.push_back(ch);
        b = e;
      }
      ++item_index;
    }
    // record the step's accesses
    for (size_t c = step_lo; with_deps && c < out->chunks.size(); ++c) {
      const ColumnChunk& ch = out->chunks[c];
      const Item& it = step.items[ch.item - (item_index - step.items.size())];
      const uint64_t b = ch.begin, e = ch.begin + ch.count;
      // sources before destinations: a range a chunk reads and writes ends
      // with the write alone, which already orders every later access
      for (int k = 0; k < it.nsrc + it.ndst; ++k) {
        const bool write = k >= it.nsrc;
        History& h = hist[it.rank[k]];
        split(h, b);
        split(h, e);
        for (auto seg = h.find(b); seg != h.end() && seg->first < e; ++seg) {
          if (write) {
            seg->second.writer = static_cast<int64_t>(c);
            seg->second.readers.clear();
          } else {
            seg->second.readers.push_back(static_cast<uint32_t>(c));
          }
        }
      }
    }
  }
  out->step_first.push_back(static_cast<uint32_t>(out->chunks.size()));

  // per-column chunk lists, ascending index
  uint64_t ncols = 0;
  for (const ColumnChunk& ch : out->chunks) ncols = std::max(ncols, ch.begin / chunk_elems + 1);
  if (ncols >= UINT32_MAX) return false;
  out->col_off.assign(ncols + 1, 0);
  for (const ColumnChunk& ch : out->chunks) ++out->col_off[ch.begin / chunk_elems + 1];
  for (uint64_t g = 0; g < ncols; ++g) out->col_off[g + 1] += out->col_off[g];
  out->col_list.assign(out->chunks.size(), 0);
  out->max_per_col = 0;
  for (uint64_t g = 0; g < ncols; ++g)
    out->max_per_col = std::max<uint64_t>(out->max_per_col, out->col_off[g + 1] - out->col_off[g]);
  std::vector<uint32_t> fill(out->col_off.begin(), out->col_off.end() - 1);
  for (size_t c = 0; c < out->chunks.size(); ++c)
    out->col_list[fill[out->chunks[c].begin / chunk_elems]++] = static_cast<uint32_t>(c);
  return true;
}

}  // namespace hbmc
