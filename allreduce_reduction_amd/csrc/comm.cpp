// Communicator internals: schedule cache, device item tables, step launches.
#include "comm.hpp"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>

namespace hbmc {

uint32_t elem_bytes(int dtype) {
  switch (dtype) {
    case HBMC_FP32: return 4;
    case HBMC_FP16: return 2;
    case HBMC_BF16: return 2;
    case HBMC_INT32: return 4;
    case HBMC_INT8: return 1;
    default: return 0;
  }
}

namespace {

hbmc_status_t from_build(BuildStatus b) {
  switch (b) {
    case kBuilt: return HBMC_OK;
    case kUnsupported: return HBMC_ERR_UNSUPPORTED;
    default: return HBMC_ERR_INVALID_ARG;
  }
}

}  // namespace

bool valid_coll(int c) { return c >= HBMC_COLL_ALLREDUCE && c <= HBMC_COLL_BROADCAST; }
bool valid_op(int op) { return op >= HBMC_SUM && op <= HBMC_MIN; }

namespace {

hbmc_status_t plan_for(hbmc_comm* c, int ti, int coll, int root, size_t count, int dtype, Plan** out) {
  const uint32_t e = elem_bytes(dtype);
  auto key = std::make_tuple(ti, coll, root, static_cast<uint64_t>(count), dtype);
  auto it = c->plans.find(key);
  if (it != c->plans.end()) {
    *out = it->second.get();
    return HBMC_OK;
  }
  std::unique_ptr<Plan> p(new (std::nothrow) Plan);
  if (!p) return HBMC_ERR_NOMEM;
  hbmc_status_t st =
      from_build(build_schedule(c->topos[ti], static_cast<Coll>(coll), count, e, root, &p->sched));
  if (st != HBMC_OK) return st;
  size_t off = 0;
  for (const Step& s : p->sched.steps) {
    p->first_item.push_back(off);
    off += s.items.size();
  }
  p->coll = coll;
  *out = p.get();
  c->plans.emplace(key, std::move(p));
  return HBMC_OK;
}

hbmc_status_t normalise(hbmc_comm* c, int coll, int* root, size_t count, int dtype) {
  const uint32_t e = elem_bytes(dtype);
  if (!c || e == 0 || !valid_coll(coll) || c->topos.empty()) return HBMC_ERR_INVALID_ARG;
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  const bool rooted = coll == HBMC_COLL_REDUCE || coll == HBMC_COLL_BROADCAST;
  if (rooted && (*root < 0 || *root >= c->topos[0].P)) return HBMC_ERR_INVALID_ARG;
  if (!rooted) *root = 0;
  return HBMC_OK;
}

}  // namespace

hbmc_status_t choose_topology(hbmc_comm* c, int coll, int root, size_t count, int dtype, int* index) {
  hbmc_status_t st = normalise(c, coll, &root, count, dtype);
  if (st != HBMC_OK) return st;
  if (!c->auto_select) {
    *index = 0;
    return HBMC_OK;
  }
  if (c->auto_rules) {
    // topos: 0 ring, 1 RHD, 2 Flat
    const int P = c->topos[0].P;
    const bool pow2 = (P & (P - 1)) == 0;
    if (coll == HBMC_COLL_ALLREDUCE && uint64_t(count) * elem_bytes(dtype) < kFlatRuleBytes) *index = 2;
    else if (coll == HBMC_COLL_REDUCE || coll == HBMC_COLL_BROADCAST) *index = 1;
    else *index = pow2 ? 1 : 0;
    return HBMC_OK;
  }
  auto key = std::make_tuple(coll, root, static_cast<uint64_t>(count), dtype);
  auto it = c->chosen.find(key);
  if (it != c->chosen.end()) {
    *index = it->second;
    return HBMC_OK;
  }
  int best = -1;
  double best_t = 0;
  size_t best_steps = 0;
  hbmc_status_t first_err = HBMC_ERR_UNSUPPORTED;
  for (int ti = 0; ti < static_cast<int>(c->topos.size()); ++ti) {
    Plan* p = nullptr;
    st = plan_for(c, ti, coll, root, count, dtype, &p);
    if (st == HBMC_ERR_UNSUPPORTED) continue;
    if (st != HBMC_OK) {
      first_err = st;
      continue;
    }
    size_t launches = 0;
    for (const Step& s : p->sched.steps) launches += s.items.empty() ? 0 : 1;
    const double t = double(launches) * c->alpha_us + double(p->sched.hbm_bytes) / (c->beta_gbps * 1e3);
    if (best < 0 || t < best_t || (t == best_t && launches < best_steps)) {
      best = ti;
      best_t = t;
      best_steps = launches;
    }
  }
  if (best < 0) return first_err;
  c->chosen.emplace(key, best);
  *index = best;
  return HBMC_OK;
}

hbmc_status_t get_plan(hbmc_comm* c, int coll, int root, size_t count, int dtype, Plan** out) {
  hbmc_status_t st = normalise(c, coll, &root, count, dtype);
  if (st != HBMC_OK) return st;
  int ti = 0;
  st = choose_topology(c, coll, root, count, dtype, &ti);
  if (st != HBMC_OK) return st;
  return plan_for(c, ti, coll, root, count, dtype, out);
}

hbmc_status_t upload(Plan* p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HBMC_ERR_HIP;
  if (p->dev) return p->device == dev ? HBMC_OK : HBMC_ERR_INVALID_ARG;
  size_t n = 0;
  for (const Step& s : p->sched.steps) n += s.items.size();
  if (n == 0) {
    p->device = dev;
    return HBMC_OK;
  }
  std::vector<DevItem> host(n);
  size_t k = 0;
  for (const Step& s : p->sched.steps)
    for (const Item& it : s.items) {
      DevItem& d = host[k++];
      std::memset(&d, 0, sizeof(d));
      d.begin = it.begin;
      d.count = it.count;
      d.nsrc = static_cast<uint32_t>(it.nsrc);
      d.ndst = static_cast<uint32_t>(it.ndst);
      std::memcpy(d.rank, it.rank, sizeof(d.rank));
    }
  std::vector<FusedStep> fs(p->sched.steps.size());
  for (size_t s = 0; s < fs.size(); ++s) {
    fs[s].first_item = static_cast<uint32_t>(p->first_item[s]);
    fs[s].nitems = static_cast<uint32_t>(p->sched.steps[s].items.size());
    fs[s].mode = static_cast<uint32_t>(p->sched.steps[s].mode);
    fs[s].pad = 0;
  }
  const size_t item_bytes = n * sizeof(DevItem), step_bytes = fs.size() * sizeof(FusedStep);
  void* mem = nullptr;
  if (hipMalloc(&mem, item_bytes + step_bytes) != hipSuccess) return HBMC_ERR_NOMEM;
  if (hipMemcpy(mem, host.data(), item_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(static_cast<char*>(mem) + item_bytes, fs.data(), step_bytes, hipMemcpyHostToDevice) !=
          hipSuccess) {
    (void)hipFree(mem);
    return HBMC_ERR_HIP;
  }
  p->dev = static_cast<DevItem*>(mem);
  p->dev_steps = reinterpret_cast<FusedStep*>(static_cast<char*>(mem) + item_bytes);
  p->device = dev;
  return HBMC_OK;
}

uint64_t column_elems(uint64_t column_bytes, uint64_t count, uint32_t e, uint32_t compute_units) {
  if (column_bytes > 0) return std::max<uint64_t>(16, column_bytes / 16 * 16) / e;
  const uint64_t cols = uint64_t(compute_units) * 4;
  uint64_t b = (count * e + cols - 1) / cols;
  b = std::max<uint64_t>(1024, (b + 1023) / 1024 * 1024);
  return b / e;
}

hbmc_status_t column_table(Plan* p, int P, uint64_t chunk_elems, const ColumnTable** out) {
  if (p->cols.chunk_elems != chunk_elems || p->cols.col_off.empty()) {
    if (p->cols_mem) {
      // the device copy belongs to the old length; launches already enqueued
      // and graphs built earlier may still read it
      p->retired.push_back(p->cols_mem);
      p->cols_mem = nullptr;
    }
    if (!build_columns(p->sched, P, chunk_elems, false, &p->cols)) return HBMC_ERR_INVALID_ARG;
  }
  *out = &p->cols;
  return HBMC_OK;
}

hbmc_status_t upload_columns(Plan* p) {
  if (p->cols_mem) return HBMC_OK;
  const ColumnTable& f = p->cols;
  const size_t n = f.chunks.size();
  std::vector<DevChunk> host(n);
  for (size_t i = 0; i < n; ++i) {
    const ColumnChunk& c = f.chunks[i];
    host[i].begin = c.begin;
    host[i].count = c.count;
    host[i].item = c.item;
    host[i].mode = static_cast<uint32_t>(p->sched.steps[c.step].mode);
    host[i].step = c.step;
    host[i].pad0 = host[i].pad1 = 0;
  }
  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t b_chunks = up(n * sizeof(DevChunk) + 16);
  const size_t b_list = up(f.col_list.size() * sizeof(uint32_t) + 4);
  const size_t b_off = up(f.col_off.size() * sizeof(uint32_t) + 4);
  void* mem = nullptr;
  if (hipMalloc(&mem, b_chunks + b_list + b_off) != hipSuccess) return HBMC_ERR_NOMEM;
  char* base = static_cast<char*>(mem);
  if ((n && hipMemcpy(base, host.data(), n * sizeof(DevChunk), hipMemcpyHostToDevice) != hipSuccess) ||
      (!f.col_list.empty() && hipMemcpy(base + b_chunks, f.col_list.data(), f.col_list.size() * sizeof(uint32_t),
                                        hipMemcpyHostToDevice) != hipSuccess) ||
      (!f.col_off.empty() && hipMemcpy(base + b_chunks + b_list, f.col_off.data(),
                                       f.col_off.size() * sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess)) {
    (void)hipFree(mem);
    return HBMC_ERR_HIP;
  }
  p->cols_mem = mem;
  p->dev_chunks = reinterpret_cast<DevChunk*>(base);
  p->dev_col_list = reinterpret_cast<uint32_t*>(base + b_chunks);
  p->dev_col_off = reinterpret_cast<uint32_t*>(base + b_chunks + b_list);
  return HBMC_OK;
}

hbmc_status_t flow_host(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, FlowSet** out) {
  const uint64_t col = std::max<uint64_t>(16, c->flow_tile_bytes / 16 * 16) / e;
  FlowSet& f = p->flow[std::make_pair(first, last)];
  *out = &f;
  if (f.built && f.table.col_elems == col) return HBMC_OK;
  if (f.mem) {
    // launches already enqueued and graphs built earlier may still read it
    p->retired.push_back(f.mem);
    p->flow_old.push_back(f.mem);
    f.mem = nullptr;
  }
  f.ok = build_flow(p->sched, first, last, count, e, col, &f.table);
  f.table.col_elems = col;
  f.built = true;
  return HBMC_OK;
}

// Byte offsets in a plan's flow allocation: the control block, the count
// of waits that gave up, then the column counters, tiles and chunks.
constexpr size_t kFlowTimeoutsAt = 128;
constexpr size_t kFlowHeadBytes = 256;

hbmc_status_t upload_flow(Plan*, FlowSet* fs) {
  if (fs->mem) return HBMC_OK;
  const FlowTable& f = fs->table;
  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t b_ctrl = kFlowHeadBytes;
  const size_t b_prog = up(size_t(f.ncols) * sizeof(uint32_t) + 4);
  const size_t b_tiles = up(f.tiles.size() * sizeof(FlowTile) + 16);
  const size_t b_chunks = up(f.chunks.size() * sizeof(FlowChunk) + 16);
  void* mem = nullptr;
  if (hipMalloc(&mem, b_ctrl + b_prog + b_tiles + b_chunks) != hipSuccess) return HBMC_ERR_NOMEM;
  char* base = static_cast<char*>(mem);
  const std::vector<char> zero(b_ctrl + b_prog, 0);
  if (hipMemcpy(base, zero.data(), zero.size(), hipMemcpyHostToDevice) != hipSuccess ||
      (!f.tiles.empty() && hipMemcpy(base + b_ctrl + b_prog, f.tiles.data(), f.tiles.size() * sizeof(FlowTile),
                                     hipMemcpyHostToDevice) != hipSuccess) ||
      (!f.chunks.empty() && hipMemcpy(base + b_ctrl + b_prog + b_tiles, f.chunks.data(),
                                      f.chunks.size() * sizeof(FlowChunk), hipMemcpyHostToDevice) != hipSuccess)) {
    (void)hipFree(mem);
    return HBMC_ERR_HIP;
  }
  fs->mem = mem;
  fs->ctrl = reinterpret_cast<FlowCtrl*>(base);
  fs->timeouts = reinterpret_cast<uint32_t*>(base + kFlowTimeoutsAt);
  fs->prog = reinterpret_cast<uint32_t*>(base + b_ctrl);
  fs->tiles = reinterpret_cast<FlowTile*>(base + b_ctrl + b_prog);
  fs->chunks = reinterpret_cast<FlowChunk*>(base + b_ctrl + b_prog + b_tiles);
  return HBMC_OK;
}

hbmc_status_t flow_timeouts(hbmc_comm* c, uint32_t* count) {
  *count = 0;
  const uint32_t zero = 0;
  for (auto& kv : c->plans) {
    Plan* p = kv.second.get();
    std::vector<void*> blocks = p->flow_old;
    for (auto& f : p->flow)
      if (f.second.mem) blocks.push_back(f.second.mem);
    for (void* m : blocks) {
      // the counter lives on the plan's device; unified addressing lets the
      // copies find it from the pointer
      uint32_t* t = reinterpret_cast<uint32_t*>(static_cast<char*>(m) + kFlowTimeoutsAt);
      uint32_t n = 0;
      if (hipMemcpy(&n, t, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess ||
          hipMemcpy(t, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
        return HBMC_ERR_HIP;
      *count += n;
    }
  }
  return HBMC_OK;
}

namespace {

void lds_limits(uint64_t* per_block, uint64_t* per_cu);

// Trailing copy steps a column must have for its copies to be composed into
// stores (measured on MI355X: with 3, RHD over 8 ranks at 4 MiB per rank
// took 12.9 instead of 14.0 us per AllReduce and 9.1 instead of 15.0 us per
// all-gather; at 1-64 KiB per rank no difference showed).
constexpr uint32_t kMinStoreSteps = 3;

// Bytes [lo, hi) of a column of one rank's final values come from the LDS
// copy of rank `src`.
struct Piece {
  uint32_t lo, hi, src;
};

// `pieces` (ascending, covering [0, n)) with [lo, hi) replaced by `with`.
void replace_range(std::vector<Piece>& pieces, uint32_t lo, uint32_t hi, const std::vector<Piece>& with,
                   std::vector<Piece>& tmp) {
  tmp.clear();
  for (const Piece& q : pieces)
    if (q.lo < lo) tmp.push_back({q.lo, std::min(q.hi, lo), q.src});
  for (const Piece& q : with) tmp.push_back(q);
  for (const Piece& q : pieces)
    if (q.hi > hi) tmp.push_back({std::max(q.lo, hi), q.hi, q.src});
  pieces.clear();
  for (const Piece& q : tmp) {
    if (!pieces.empty() && pieces.back().src == q.src && pieces.back().hi == q.lo) pieces.back().hi = q.hi;
    else pieces.push_back(q);
  }
}

}  // namespace

hbmc_status_t lds_host_tables(Plan* p, int P, uint64_t count, uint32_t e) {
  if (p->lh.built_col == p->lds_col && p->lds_col > 0) return HBMC_OK;
  if (p->lds_cols.chunk_elems != p->lds_col || p->lds_cols.col_off.empty())
    if (!build_columns(p->sched, P, p->lds_col, false, &p->lds_cols)) return HBMC_ERR_INVALID_ARG;
  const ColumnTable& f = p->lds_cols;
  const size_t n = f.col_list.size();
  const size_t ncols = f.col_off.size() - 1;
  std::vector<DevColChunk>& host = p->lh.image;
  host.assign(n + 1, DevColChunk{});
  std::memset(host.data(), 0, host.size() * sizeof(DevColChunk));
  for (size_t g = 0; g < ncols; ++g) {
    const uint64_t col_begin = uint64_t(g) * f.chunk_elems;
    for (uint32_t k = f.col_off[g]; k < f.col_off[g + 1]; ++k) {
      const ColumnChunk& c = f.chunks[f.col_list[k]];
      const Step& st = p->sched.steps[c.step];
      const Item& it = st.items[c.item - p->first_item[c.step]];
      DevColChunk& d = host[k];
      d.lo = static_cast<uint32_t>((c.begin - col_begin) * e);
      d.hi = d.lo + c.count * e;
      d.step = c.step;
      d.shape = static_cast<uint32_t>(st.mode) | (static_cast<uint32_t>(it.nsrc) << 8) |
                (static_cast<uint32_t>(it.ndst) << 16);
      d.dst_mask = 0;
      d.batch = 1;
      for (int q = 0; q < it.nsrc + it.ndst; ++q) d.rank[q] = it.rank[q];
      for (int q = it.nsrc; q < it.nsrc + it.ndst; ++q) d.dst_mask |= uint64_t(1) << it.rank[q];
    }
    // runs of same-step, same-range records of the reduce (2 sources, 1
    // destination) or copy (1, 1) shape, cut into batches of 8, 4 or 2
    auto batchable = [&](const DevColChunk& a, const DevColChunk& b) {
      const uint32_t sh = a.shape;
      const bool shape_ok = sh == (uint32_t(kRecvFold) | (2u << 8) | (1u << 16)) ||
                            sh == (uint32_t(kCopy) | (1u << 8) | (1u << 16));
      return shape_ok && b.shape == sh && a.step == b.step && a.lo == b.lo && a.hi == b.hi;
    };
    for (uint32_t k = f.col_off[g]; k < f.col_off[g + 1];) {
      uint32_t run = 1;
      while (k + run < f.col_off[g + 1] && batchable(host[k], host[k + run])) ++run;
      while (run > 0) {
        const uint32_t b = run >= 8 ? 8 : (run >= 4 ? 4 : (run >= 2 ? 2 : 1));
        host[k].batch = b;
        for (uint32_t q = 1; q < b; ++q) host[k + q].batch = 0;
        k += b;
        run -= b;
      }
    }
  }
  // Launches of all steps: each column's trailing copy chunks composed into
  // store records.  Every rank starts as its own source; a copy chunk gives
  // each destination, over the chunk's range, the sources its source has
  // there.  Every rank some chunk of the column writes is stored.
  std::vector<DevColStore>& stores = p->lh.stores;
  std::vector<uint32_t>& col_run = p->lh.col_run;
  std::vector<uint32_t>& st_off = p->lh.st_off;
  stores.clear();
  col_run.assign(ncols, 0);
  st_off.assign(ncols + 1, 0);
  const uint64_t all_ranks = P >= 64 ? ~uint64_t(0) : ((uint64_t(1) << P) - 1);
  std::vector<uint64_t>& col_load = p->lh.col_load;
  col_load.assign(ncols, all_ranks);
  std::vector<std::vector<Piece>> map(P);
  std::vector<Piece> part, tmp;
  uint64_t meta_steps = 0, meta_whole = 0;
  bool any_tail = false;
  for (size_t g = 0; g < ncols; ++g) {
    const uint64_t col_begin = uint64_t(g) * f.chunk_elems;
    const uint32_t nbytes = static_cast<uint32_t>(std::min<uint64_t>(f.chunk_elems, count - col_begin) * e);
    const uint32_t k0 = f.col_off[g], k1 = f.col_off[g + 1];
    uint32_t cut = k1;
    while (cut > k0 && (host[cut - 1].shape & 0xffu) == uint32_t(kCopy)) --cut;
    col_run[g] = cut - k0;
    uint64_t dirty = 0;
    for (uint32_t k = k0; k < k1; ++k) dirty |= host[k].dst_mask;
    for (int r = 0; r < P; ++r) map[r].assign(1, Piece{0, nbytes, static_cast<uint32_t>(r)});
    for (uint32_t k = cut; k < k1; ++k) {
      const DevColChunk& c = host[k];
      const int nd = static_cast<int>(c.shape >> 16);
      part.clear();
      for (const Piece& q : map[c.rank[0]])
        if (q.hi > c.lo && q.lo < c.hi) part.push_back({std::max(q.lo, c.lo), std::min(q.hi, c.hi), q.src});
      for (int q = 1; q <= nd; ++q) replace_range(map[c.rank[q]], c.lo, c.hi, part, tmp);
    }
    // composed only where every written rank takes its bytes from at most two
    // copies (a column within one or two segments): the kernel walks store
    // records one after another, while the copy chunks it would skip go in
    // batches; other columns run every chunk and store their written ranks
    // whole (no store records)
    size_t nrec = 0;
    for (int r = 0; r < P; ++r)
      if ((dirty >> r) & 1u) nrec += map[r].size();
    uint32_t tail_steps = 0;
    for (uint32_t k = cut; k < k1; ++k) tail_steps += (k == cut || host[k].step != host[k - 1].step) ? 1u : 0u;
    if (tail_steps >= kMinStoreSteps && nrec <= 2 * size_t(__builtin_popcountll(dirty))) {
      // loaded: the ranks the remaining chunks name and the stores' sources
      uint64_t load = 0;
      for (uint32_t k = k0; k < cut; ++k) {
        const int nr = static_cast<int>(((host[k].shape >> 8) & 0xffu) + (host[k].shape >> 16));
        for (int q = 0; q < nr; ++q) load |= uint64_t(1) << host[k].rank[q];
      }
      for (int r = 0; r < P; ++r) {
        if (!((dirty >> r) & 1u)) continue;
        for (const Piece& q : map[r]) {
          stores.push_back(DevColStore{q.lo, q.hi, static_cast<uint32_t>(r), q.src});
          load |= uint64_t(1) << q.src;
        }
      }
      col_load[g] = load;
    } else {
      cut = k1;
      col_run[g] = k1 - k0;
    }
    st_off[g + 1] = static_cast<uint32_t>(stores.size());
    any_tail = any_tail || cut < k1;
    meta_steps = std::max<uint64_t>(meta_steps, uint64_t(k1 - k0) * sizeof(DevColChunk));
    meta_whole = std::max<uint64_t>(meta_whole, uint64_t(cut - k0) * sizeof(DevColChunk) +
                                                    uint64_t(st_off[g + 1] - st_off[g]) * sizeof(DevColStore));
  }
  p->lh.meta_steps = meta_steps;
  p->lh.meta_whole = meta_whole;
  p->lh.any_tail = any_tail;
  uint64_t per_block = 0, per_cu = 0;
  lds_limits(&per_block, &per_cu);
  p->lh.stores_fit = any_tail && uint64_t(P) * lds_slot_bytes(p->lds_col, e) + meta_whole <= per_block;
  p->lh.built_col = p->lds_col;
  return HBMC_OK;
}

hbmc_status_t upload_lds_tables(Plan* p, int P, uint64_t count, uint32_t e) {
  if (p->lds_mem) return HBMC_OK;
  hbmc_status_t hs = lds_host_tables(p, P, count, e);
  if (hs != HBMC_OK) return hs;
  const ColumnTable& f = p->lds_cols;
  const std::vector<DevColChunk>& host = p->lh.image;
  const std::vector<DevColStore>& stores = p->lh.stores;
  const std::vector<uint32_t>& col_run = p->lh.col_run;
  const std::vector<uint32_t>& st_off = p->lh.st_off;
  const std::vector<uint64_t>& col_load = p->lh.col_load;
  const uint64_t meta_steps = p->lh.meta_steps, meta_whole = p->lh.meta_whole;

  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t b_image = up(host.size() * sizeof(DevColChunk));
  const size_t b_off = up(f.col_off.size() * sizeof(uint32_t));
  const size_t b_st = up((stores.size() + 1) * sizeof(DevColStore));
  const size_t b_run = up(col_run.size() * sizeof(uint32_t) + 4);
  const size_t b_st_off = up(st_off.size() * sizeof(uint32_t));
  const size_t b_load = col_load.size() * sizeof(uint64_t) + 8;
  void* mem = nullptr;
  if (hipMalloc(&mem, b_image + b_off + b_st + b_run + b_st_off + b_load) != hipSuccess) return HBMC_ERR_NOMEM;
  char* base = static_cast<char*>(mem);
  if (hipMemcpy(base, host.data(), host.size() * sizeof(DevColChunk), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(base + b_image, f.col_off.data(), f.col_off.size() * sizeof(uint32_t), hipMemcpyHostToDevice) !=
          hipSuccess ||
      (!stores.empty() && hipMemcpy(base + b_image + b_off, stores.data(), stores.size() * sizeof(DevColStore),
                                    hipMemcpyHostToDevice) != hipSuccess) ||
      hipMemcpy(base + b_image + b_off + b_st, col_run.data(), col_run.size() * sizeof(uint32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(base + b_image + b_off + b_st + b_run, st_off.data(), st_off.size() * sizeof(uint32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(base + b_image + b_off + b_st + b_run + b_st_off, col_load.data(),
                col_load.size() * sizeof(uint64_t), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(mem);
    return HBMC_ERR_HIP;
  }
  p->lds_mem = mem;
  p->dev_image = reinterpret_cast<DevColChunk*>(base);
  p->dev_lds_col_off = reinterpret_cast<uint32_t*>(base + b_image);
  p->dev_stores = reinterpret_cast<DevColStore*>(base + b_image + b_off);
  p->dev_col_run = reinterpret_cast<uint32_t*>(base + b_image + b_off + b_st);
  p->dev_st_off = reinterpret_cast<uint32_t*>(base + b_image + b_off + b_st + b_run);
  p->dev_col_load = reinterpret_cast<uint64_t*>(base + b_image + b_off + b_st + b_run + b_st_off);
  p->lds_meta_steps = meta_steps;
  p->lds_meta_whole = meta_whole;
  p->lds_stores = p->lh.stores_fit;
  return HBMC_OK;
}

hbmc_status_t check_bufs(int P, void* const bufs[], size_t count, uint32_t e) {
  if (!bufs) return HBMC_ERR_INVALID_ARG;
  const uint64_t bytes = uint64_t(count) * e;
  for (int r = 0; r < P; ++r) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(bufs[r]);
    if (!a || a % e) return HBMC_ERR_INVALID_ARG;
    if (a + bytes < a) return HBMC_ERR_INVALID_ARG;
    for (int q = 0; q < r; ++q) {
      const uintptr_t b = reinterpret_cast<uintptr_t>(bufs[q]);
      if (a < b + bytes && b < a + bytes) return HBMC_ERR_INVALID_ARG;  // aliased / overlapping
    }
  }
  return HBMC_OK;
}

namespace {

// Device attributes are cached per device in atomics: communicators on other
// host threads may query them at the same time.
uint32_t compute_units() {
  static std::atomic<uint32_t> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  uint32_t v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    v = static_cast<uint32_t>(cus);
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// The wall clock's rate (kHz) on the current device: the unit of the flow
// kernel's wait bound.
uint64_t wall_clock_khz() {
  static std::atomic<uint32_t> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000;
  uint32_t v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
    v = static_cast<uint32_t>(khz);
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Dynamic LDS one workgroup may use, and LDS per compute unit, of the current
// device.
void lds_limits(uint64_t* per_block, uint64_t* per_cu) {
  static std::atomic<uint64_t> blk[64] = {}, cu[64] = {};
  int dev = 0;
  *per_block = 64 << 10;
  *per_cu = 64 << 10;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return;
  // cu is published before blk, so a reader that sees blk sees cu
  const uint64_t b0 = blk[dev].load(std::memory_order_acquire);
  if (b0 != 0) {
    *per_block = b0;
    *per_cu = cu[dev].load(std::memory_order_relaxed);
    return;
  }
  int b = 0, m = 0;
  if (hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || b <= 0)
    b = 64 << 10;
  if (hipDeviceGetAttribute(&m, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || m < b)
    m = b;
  cu[dev].store(static_cast<uint64_t>(m), std::memory_order_relaxed);
  blk[dev].store(static_cast<uint64_t>(b), std::memory_order_release);
  *per_block = static_cast<uint64_t>(b);
  *per_cu = static_cast<uint64_t>(m);
}

// Workgroups of the LDS-resident column kernel: one per column, at most as
// many as the compute units hold at once.
uint32_t lds_grid(uint32_t ncols, uint64_t shared_bytes) {
  uint64_t per_block = 0, per_cu = 0;
  lds_limits(&per_block, &per_cu);
  const uint64_t per = std::max<uint64_t>(1, std::min<uint64_t>(8, per_cu / std::max<uint64_t>(1, shared_bytes)));
  return static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(ncols, compute_units() * per)));
}

// Chunks of the longest column for a column length of `col` elements: each
// item adds one chunk to every column it meets.
uint64_t longest_column(const Schedule& s, uint64_t count, uint64_t col) {
  const uint64_t ncols = (count + col - 1) / col;
  std::vector<int64_t> diff(ncols + 1, 0);
  for (const Step& st : s.steps)
    for (const Item& it : st.items) {
      if (it.count == 0) continue;
      diff[it.begin / col] += 1;
      diff[(it.begin + it.count - 1) / col + 1] -= 1;
    }
  int64_t run = 0, best = 0;
  for (uint64_t g = 0; g < ncols; ++g) {
    run += diff[g];
    best = std::max(best, run);
  }
  return static_cast<uint64_t>(best);
}

// Serial chunk passes of the busiest column for a column length of `col`
// elements, in units of one chunk's pass: per step, the chunks that cover a
// whole column go in batches of 8, 4, 2 or 1 (the kernel's runs of
// same-range chunks, assuming one shape per step), a batch of n costing
// 1 + 0.75 (n - 1) passes (fitted on MI355X: a batch's loads overlap, its
// element ops mostly do not); every chunk that covers part of a column goes
// alone.  Only steps before `steps_end` count.  Beyond 2^24 column-steps it
// falls back to counting every chunk.
double longest_passes(const Schedule& s, uint64_t count, uint64_t col, size_t steps_end) {
  const uint64_t ncols = (count + col - 1) / col;
  if (ncols * s.steps.size() > (uint64_t(1) << 24)) return double(longest_column(s, count, col));
  std::vector<double> passes(ncols, 0.0);
  std::vector<int64_t> full(ncols + 1), part(ncols + 1);
  for (size_t si = 0; si < steps_end && si < s.steps.size(); ++si) {
    const Step& st = s.steps[si];
    std::fill(full.begin(), full.end(), 0);
    std::fill(part.begin(), part.end(), 0);
    for (const Item& it : st.items) {
      if (it.count == 0) continue;
      const uint64_t b = it.begin, e = it.begin + it.count;
      const uint64_t g0 = b / col, g1 = (e - 1) / col;  // columns met
      // columns covered whole: [f0, f1) (the last column ends at count)
      const uint64_t f0 = (b + col - 1) / col, f1 = e == count ? ncols : e / col;
      if (f0 < f1) {
        full[f0] += 1;
        full[f1] -= 1;
      }
      const bool cut_first = g0 < f0, cut_last = g1 >= f1;
      if (cut_first) part[g0] += 1;
      if (cut_last && !(cut_first && g1 == g0)) part[g1] += 1;
    }
    int64_t run = 0;
    for (uint64_t g = 0; g < ncols; ++g) {
      run += full[g];
      uint64_t n = static_cast<uint64_t>(run);
      double t = double(part[g]);
      for (uint64_t b : {8u, 4u, 2u, 1u})
        for (; n >= b; n -= b) t += 1.0 + 0.75 * double(b - 1);
      passes[g] += t;
    }
  }
  double best = 0.0;
  for (double v : passes) best = std::max(best, v);
  return best;
}

// Modelled time of the LDS-resident form with columns of `col` elements,
// `chunks` chunks in the longest column's list (its LDS records) and
// `longest` serial chunk passes in the busiest column (`share`: the
// fraction of the schedule's busy steps the launch runs): the columns a
// workgroup runs one after another, times those passes, times the 16-byte
// positions each lane takes per chunk; plus moving `buffers` rank buffers'
// worth of bytes (2 P: every rank loaded and stored).
double lds_time(const ExecModel& m, int P, uint64_t count, uint32_t e, uint64_t col, uint64_t chunks,
                double longest, double share, double buffers) {
  const uint64_t ncols = (count + col - 1) / col;
  const uint32_t grid = lds_grid(static_cast<uint32_t>(std::min<uint64_t>(ncols, UINT32_MAX)),
                                 lds_bytes(P, col, e, chunks));
  const double rounds = std::ceil(double(ncols) / grid);
  const uint64_t positions = std::max<uint64_t>(1, col * e / 16);
  const uint64_t lanes = lds_threads(col, e);
  const double per_lane = std::ceil(double(positions) / lanes);
  return m.lds_us + rounds * longest * share * per_lane * m.lds_chunk_us +
         buffers * double(count) * e / (m.lds_gbps * 1e3);
}

}  // namespace

hbmc_status_t lds_layout(hbmc_comm* c, Plan* p, int P, uint64_t count, uint32_t e) {
  if (p->lds_key == c->column_bytes) return HBMC_OK;
  if (p->lds_mem) {
    // the device tables belong to the old length; launches already enqueued
    // and graphs built earlier may still read them
    p->retired.push_back(p->lds_mem);
    p->lds_mem = nullptr;
  }
  uint64_t per_block = 0, per_cu = 0;
  lds_limits(&per_block, &per_cu);
  p->lds_col = 0;
  p->lds_chunks = 0;
  p->lds_longest = 0.0;
  auto fits = [&](uint64_t col, uint64_t longest) { return lds_bytes(P, col, e, longest) <= per_block; };
  // the schedule's trailing copy steps, which a launch of all steps replaces
  // by composed stores
  size_t body = p->sched.steps.size();
  while (body > 0 && (p->sched.steps[body - 1].mode == kCopy || p->sched.steps[body - 1].items.empty())) --body;
  const size_t all = p->sched.steps.size();
  // the stores replace those copies only in columns that meet at most two of
  // their items per rank: taken as columns no longer than the shortest
  uint64_t tail_item = UINT64_MAX;
  for (size_t si = body; si < all; ++si)
    for (const Item& it : p->sched.steps[si].items) tail_item = std::min(tail_item, it.count);
  const bool composable = all - body >= kMinStoreSteps;
  auto whole_end = [&](uint64_t col) { return composable && col <= tail_item ? body : all; };
  // the composed stores cost about one chunk pass
  auto whole_passes = [&](uint64_t col) {
    const size_t end = whole_end(col);
    return longest_passes(p->sched, count, col, end) + (end < all ? 1.0 : 0.0);
  };
  if (c->column_bytes > 0) {
    const uint64_t col = column_elems(c->column_bytes, count, e, compute_units());
    const uint64_t chunks = longest_column(p->sched, count, col);
    if (fits(col, chunks)) {
      p->lds_col = col;
      p->lds_chunks = chunks;
      p->lds_longest = longest_passes(p->sched, count, col, all);
      p->lds_longest_whole = whole_passes(col);
    }
  } else {
    // 16-byte multiples from the longest that can fit down to 16 bytes
    double best = 0.0;
    uint64_t top = 16;
    while (top * 2 <= uint64_t(count) * e && top * 2 * P <= per_block) top *= 2;
    for (uint64_t bytes = top; bytes >= 16; bytes /= 2) {
      const uint64_t col = bytes / e;
      const uint64_t chunks = longest_column(p->sched, count, col);
      if (!fits(col, chunks)) continue;
      const double passes = whole_passes(col);
      const double t = lds_time(c->model, P, count, e, col, chunks, passes, 1.0, 2.0 * P);
      if (p->lds_col == 0 || t < best * 0.98) {
        best = t;
        p->lds_col = col;
        p->lds_chunks = chunks;
        p->lds_longest = longest_passes(p->sched, count, col, all);
        p->lds_longest_whole = passes;
      }
    }
  }
  // a schedule of copies only (a stand-alone all-gather), composed: each
  // column loads its owners' copies alone, about one rank buffer in all
  p->lds_whole_buffers = body == 0 && whole_end(p->lds_col) == body ? P + 1.0 : 2.0 * P;
  p->lds_key = c->column_bytes;
  return HBMC_OK;
}

hbmc_status_t choose_exec(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, bool aligned,
                          int* mode) {
  const int P = c->topos[0].P;
  const ExecModel& m = c->model;
  uint64_t bytes = 0;
  int busy = 0, busy_all = 0;
  bool items_ok = true;
  double t_steps = 0.0;
  for (size_t s = 0; s < p->sched.steps.size(); ++s) busy_all += p->sched.steps[s].items.empty() ? 0 : 1;
  for (int s = first; s < last; ++s) {
    const Step& st = p->sched.steps[s];
    if (st.items.empty()) continue;
    ++busy;
    bytes += st.hbm_bytes;
    items_ok = items_ok && st.items.size() <= kFusedMaxItems;
    t_steps += std::max(m.launch_us, m.step_us + double(st.hbm_bytes) / (m.hbm_gbps * 1e3));
  }
  const bool fused_ok = aligned && busy > 0 && items_ok && bytes <= c->fused_limit;
  const bool cols_ok = aligned && busy > 1 && count * e <= c->columns_limit / uint64_t(P);
  // the LDS-resident form: when some column length fits one workgroup's LDS
  bool lds_ok = false;
  if (cols_ok && (c->exec_mode == kExecLds || c->exec_mode == kExecAuto)) {
    hbmc_status_t st = lds_layout(c, p, P, count, e);
    if (st != HBMC_OK) return st;
    lds_ok = p->lds_col > 0;
  }
  // the register form: a whole call whose every element ends with one of
  // the register form's expressions (see regs.hpp), within the column limit
  const bool whole = first == 0 && last == static_cast<int>(p->sched.steps.size());
  bool regs_ok = false;
  if (cols_ok && whole && (c->exec_mode == kExecRegs || c->exec_mode == kExecAuto)) {
    if (!p->regs_built) {
      derive_regs(p->sched, P, count, &p->regs);
      p->regs_built = true;
    }
    regs_ok = p->regs.ok;
  }
  *mode = kExecSteps;
  if (c->exec_mode == kExecFlow) {
    // a step range of two or more busy steps, every item within the records
    if (aligned && busy > 1) {
      FlowSet* f = nullptr;
      hbmc_status_t st = flow_host(c, p, first, last, count, e, &f);
      if (st != HBMC_OK) return st;
      // the ticket counter runs to the tiles plus one batch per workgroup
      // past them (and one more taken ahead): it must not wrap
      const uint64_t tickets = uint64_t(f->table.tiles.size()) + uint64_t(compute_units()) *
                                                                    std::max<uint32_t>(1, c->flow_wgs_per_cu) *
                                                                    std::max<uint32_t>(1, c->flow_batch) * 2;
      if (f->ok && tickets < UINT32_MAX) *mode = kExecFlow;
    }
    return HBMC_OK;
  }
  if (c->exec_mode == kExecRegs) {
    if (regs_ok) *mode = kExecRegs;
    return HBMC_OK;
  }
  if (c->exec_mode == kExecFused) {
    if (fused_ok) *mode = kExecFused;
    return HBMC_OK;
  }
  if (c->exec_mode == kExecColumns) {
    if (cols_ok) *mode = kExecColumns;
    return HBMC_OK;
  }
  if (c->exec_mode == kExecLds) {
    if (lds_ok) *mode = kExecLds;
    return HBMC_OK;
  }
  if (c->exec_mode != kExecAuto) return HBMC_OK;
  double best = t_steps;
  if (fused_ok) {
    const double t = m.fused_us + busy * m.fused_step_us + double(bytes) / (m.fused_gbps * 1e3);
    if (t < best) {
      best = t;
      *mode = kExecFused;
    }
  }
  if (cols_ok) {
    const ColumnTable* f = nullptr;
    hbmc_status_t st = column_table(p, P, column_elems(c->column_bytes, count, e, compute_units()), &f);
    if (st != HBMC_OK) return st;
    const double hops = double(f->max_per_col) * busy / std::max(1, busy_all);
    const double t = m.col_us + hops * m.col_hop_us + double(bytes) / (m.col_gbps * 1e3);
    if (t < best) {
      best = t;
      *mode = kExecColumns;
    }
  }
  if (lds_ok) {
    // a launch of all steps stores the trailing copies' results directly
    const bool all_steps = first == 0 && last == static_cast<int>(p->sched.steps.size());
    const double t = lds_time(m, P, count, e, p->lds_col, p->lds_chunks,
                              all_steps ? p->lds_longest_whole : p->lds_longest,
                              all_steps ? 1.0 : double(busy) / std::max(1, busy_all),
                              all_steps ? p->lds_whole_buffers : 2.0 * P);
    if (t < best) {
      best = t;
      *mode = kExecLds;
    }
  }
  // the register form, where eligible, measured fastest or within 11% of the
  // fastest form in every case timed on MI355X (AllReduce over rings, RHD,
  // Flat and trees of 3-17 ranks; the ring's reduce-scatter, ring and RHD
  // all-gathers, RHD broadcast; 1 KiB-4 MiB per rank, graphs of ten calls),
  // and 1.5-5x faster than the LDS form up to 1 MiB per rank
  if (regs_ok) *mode = kExecRegs;
  (void)best;
  return HBMC_OK;
}

namespace {

// Length of the union of half-open ranges (sorted in place).
uint64_t union_length(std::vector<std::pair<uint64_t, uint64_t>>& v) {
  std::sort(v.begin(), v.end());
  uint64_t total = 0, lo = 0, hi = 0;
  bool open = false;
  for (const auto& r : v) {
    if (open && r.first <= hi) {
      hi = std::max(hi, r.second);
      continue;
    }
    if (open) total += hi - lo;
    lo = r.first;
    hi = r.second;
    open = true;
  }
  if (open) total += hi - lo;
  return total;
}

}  // namespace

hbmc_status_t exec_bytes(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, int mode,
                         uint64_t* bytes) {
  const int P = c->topos[0].P;
  *bytes = 0;
  if (count == 0 || P == 1) return HBMC_OK;
  if (mode == kExecSteps || mode == kExecFlow) {
    // the flow kernel moves every step's bytes, as one launch per step does
    for (int s = first; s < last; ++s) *bytes += p->sched.steps[s].hbm_bytes;
    return HBMC_OK;
  }
  if (mode == kExecFused || mode == kExecColumns) {
    // each rank's elements read by some step once, and those written once
    std::vector<std::vector<std::pair<uint64_t, uint64_t>>> rd(P), wr(P);
    for (int s = first; s < last; ++s)
      for (const Item& it : p->sched.steps[s].items) {
        for (int q = 0; q < it.nsrc; ++q) rd[it.rank[q]].emplace_back(it.begin, it.begin + it.count);
        for (int q = it.nsrc; q < it.nsrc + it.ndst; ++q) wr[it.rank[q]].emplace_back(it.begin, it.begin + it.count);
      }
    for (int r = 0; r < P; ++r) *bytes += (union_length(rd[r]) + union_length(wr[r])) * e;
    return HBMC_OK;
  }
  if (mode == kExecRegs) {
    // every operand's vector loaded once, every destination's stored once
    if (first != 0 || last != static_cast<int>(p->sched.steps.size())) return HBMC_ERR_INVALID_ARG;
    if (!p->regs_built) {
      derive_regs(p->sched, P, count, &p->regs);
      p->regs_built = true;
    }
    if (!p->regs.ok) return HBMC_ERR_INVALID_ARG;
    if (p->regs.form != kRegNodes) {
      *bytes = uint64_t(p->regs.loads + p->regs.stores) * count * e;
      return HBMC_OK;
    }
    // the node form: every rank loaded; per region, the ranks that receive a node
    *bytes = uint64_t(p->regs.loads) * count * e;
    uint64_t start = 0;
    for (const RegRegion& q : p->regs.regions) {
      uint64_t st = 0;
      for (uint32_t v = 0; v < p->regs.n; ++v) st += q.lvl[v] != 0 && q.lvl[v] != 0xff;
      *bytes += st * (q.end - start) * e;
      start = q.end;
    }
    return HBMC_OK;
  }
  if (mode != kExecLds) return HBMC_ERR_INVALID_ARG;
  hbmc_status_t st = lds_layout(c, p, P, count, e);
  if (st != HBMC_OK) return st;
  if (p->lds_col == 0) return HBMC_ERR_INVALID_ARG;
  st = lds_host_tables(p, P, count, e);
  if (st != HBMC_OK) return st;
  const LdsHost& h = p->lh;
  const ColumnTable& f = p->lds_cols;
  const size_t ncols = f.col_off.size() - 1;
  const bool stores = h.stores_fit && first == 0 && last == static_cast<int>(p->sched.steps.size());
  for (size_t g = 0; g < ncols; ++g) {
    const uint64_t nbytes = std::min<uint64_t>(p->lds_col, count - uint64_t(g) * p->lds_col) * e;
    const uint32_t k0 = f.col_off[g];
    const uint32_t k1 = stores ? k0 + h.col_run[g] : f.col_off[g + 1];
    const uint32_t nst = stores ? h.st_off[g + 1] - h.st_off[g] : 0;
    const uint64_t loaded = stores ? h.col_load[g] : (P >= 64 ? ~uint64_t(0) : (uint64_t(1) << P) - 1);
    *bytes += uint64_t(__builtin_popcountll(loaded)) * nbytes;
    if (nst > 0) {
      for (uint32_t i = h.st_off[g]; i < h.st_off[g + 1]; ++i) *bytes += h.stores[i].hi - h.stores[i].lo;
    } else {
      uint64_t dirty = 0;
      for (uint32_t k = k0; k < k1; ++k)
        if (h.image[k].step >= uint32_t(first) && h.image[k].step < uint32_t(last)) dirty |= h.image[k].dst_mask;
      *bytes += uint64_t(__builtin_popcountll(dirty)) * nbytes;
    }
  }
  return HBMC_OK;
}

hbmc_status_t prepare(hbmc_comm* c, int coll, int root, void* const bufs[], size_t count, int dtype,
                      int op, int first, int last, bool whole, std::vector<KernelDesc>* launches) {
  launches->clear();
  if (!c || !valid_op(op) || !valid_coll(coll) || elem_bytes(dtype) == 0) return HBMC_ERR_INVALID_ARG;
  const uint32_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(c, coll, root, count, dtype, &p);
  if (st != HBMC_OK) return st;
  const int nsteps = static_cast<int>(p->sched.steps.size());
  if (whole) {
    first = 0;
    last = nsteps;
  } else if (first < 0 || last > nsteps || first >= last) {
    return HBMC_ERR_INVALID_ARG;
  }
  const int P = c->topos[0].P;
  if (count == 0 || P == 1) return HBMC_OK;
  st = check_bufs(P, bufs, count, e);
  if (st != HBMC_OK) return st;
  st = upload(p);
  if (st != HBMC_OK) return st;

  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(bufs[0]) & 15u);
  bool aligned = true;
  for (int r = 0; r < P; ++r) {
    ptrs.p[r] = static_cast<unsigned char*>(bufs[r]);
    aligned = aligned && (reinterpret_cast<uintptr_t>(bufs[r]) & 15u) == phase;
  }
  int mode = kExecSteps;
  st = choose_exec(c, p, first, last, count, e, aligned, &mode);
  if (st != HBMC_OK) return st;
  if (mode == kExecRegs) {
    // the whole call as one register-form launch
    KernelDesc k;
    describe_regs(dtype, op, ptrs, P, p->regs, count, phase, &k);
    launches->push_back(k);
    return HBMC_OK;
  }
  if (mode == kExecFlow) {
    // the step range as one flow-kernel launch
    FlowSet* fs = &p->flow.at(std::make_pair(first, last));  // made by choose_exec
    st = upload_flow(p, fs);
    if (st != HBMC_OK) return st;
    const FlowTable& f = fs->table;
    const uint32_t grid = std::max<uint32_t>(1, compute_units() * std::max<uint32_t>(1, c->flow_wgs_per_cu));
    const uint64_t ticks = uint64_t(c->flow_wait_us) * wall_clock_khz() / 1000;
    const uint32_t flags = c->flow_flags | (f.max_step_write > kCacheBytes ? kFlowNtStores : 0u);
    KernelDesc k;
    describe_flow(dtype, op, ptrs, fs->tiles, fs->chunks, static_cast<uint32_t>(f.tiles.size()),
                  fs->ctrl, fs->prog, f.ncols, fs->timeouts, phase, flags, ticks,
                  std::max<uint32_t>(1, c->flow_batch), grid, &k);
    launches->push_back(k);
    return HBMC_OK;
  }
  if (mode == kExecFused) {
    // the whole step range as one single-workgroup launch
    KernelDesc k;
    describe_fused(dtype, op, ptrs, p->dev, p->dev_steps + first, static_cast<uint32_t>(last - first), phase, &k);
    launches->push_back(k);
    return HBMC_OK;
  }
  if (mode == kExecColumns) {
    // the whole step range as one column-kernel launch
    const uint32_t cus = compute_units();
    const ColumnTable* f = nullptr;
    st = column_table(p, P, column_elems(c->column_bytes, count, e, cus), &f);
    if (st == HBMC_OK) st = upload_columns(p);
    if (st != HBMC_OK) return st;
    const uint32_t ncols = static_cast<uint32_t>(f->col_off.size() - 1);
    const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(ncols, cus * 8));
    KernelDesc k;
    describe_columns(dtype, op, ptrs, p->dev, p->dev_chunks, p->dev_col_list, p->dev_col_off, ncols,
                     f->step_first[first], f->step_first[last], phase, grid, &k);
    launches->push_back(k);
    return HBMC_OK;
  }
  if (mode == kExecLds) {
    // the whole step range as one LDS-resident column-kernel launch; a
    // launch of all steps stores the trailing copies' results directly
    st = upload_lds_tables(p, P, count, e);
    if (st != HBMC_OK) return st;
    const ColumnTable& f = p->lds_cols;
    const uint32_t ncols = static_cast<uint32_t>(f.col_off.size() - 1);
    const bool stores = p->lds_stores && first == 0 && last == nsteps;
    const uint64_t meta = stores ? p->lds_meta_whole : p->lds_meta_steps;
    const uint64_t shared = uint64_t(P) * lds_slot_bytes(p->lds_col, e) + meta;
    KernelDesc k;
    describe_columns_lds(dtype, op, ptrs, p->dev_image, p->dev_lds_col_off, ncols, static_cast<uint32_t>(first),
                         static_cast<uint32_t>(last), phase, p->lds_col, count, static_cast<uint32_t>(P), meta,
                         lds_grid(ncols, shared), stores ? p->dev_stores : nullptr,
                         stores ? p->dev_col_run : nullptr, stores ? p->dev_st_off : nullptr,
                         stores ? p->dev_col_load : nullptr, &k);
    if (shared > (64u << 10) &&
        hipFuncSetAttribute(k.func, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shared)) !=
            hipSuccess)
      return HBMC_ERR_HIP;
    launches->push_back(k);
    return HBMC_OK;
  }
  launches->reserve(static_cast<size_t>(last - first));
  for (int s = first; s < last; ++s) {
    const Step& step = p->sched.steps[s];
    if (step.items.empty()) continue;
    StepLaunch L;
    L.dtype = dtype;
    L.op = op;
    L.mode = step.mode;
    L.nsrc = step.nsrc;
    L.ndst = step.ndst;
    L.items = p->dev + p->first_item[s];
    L.host_items = step.items.data();
    L.nitems = static_cast<int>(step.items.size());
    L.max_count = step.max_count;
    L.aligned = aligned;
    L.phase = phase;
    L.xcd_split = c->xcd_split;
    L.write_bytes = 0;
    for (const Item& it : step.items) L.write_bytes += it.count * uint64_t(it.ndst) * elem_bytes(dtype);
    launches->emplace_back();
    // describe_step calls no HIP function; it refuses only a step whose
    // items exceed what one launch's grid can hold
    if (describe_step(L, ptrs, &launches->back()) != hipSuccess) return HBMC_ERR_INVALID_ARG;
  }
  return HBMC_OK;
}

// hipLaunchKernel reports its own failure; hipGetLastError is not consulted,
// so an earlier, unrelated error of the calling thread is neither reported
// here nor cleared.
hbmc_status_t launch(KernelDesc& k, void* stream) {
  k.bind();
  const hipError_t e =
      hipLaunchKernel(k.func, k.grid, k.block, k.argv, k.shared_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HBMC_OK : HBMC_ERR_HIP;
}

hbmc_status_t run(hbmc_comm* c, int coll, int root, void* const bufs[], size_t count, int dtype,
                  int op, int first, int last, bool whole, void* stream) {
  std::vector<KernelDesc> launches;
  hbmc_status_t st = prepare(c, coll, root, bufs, count, dtype, op, first, last, whole, &launches);
  for (size_t i = 0; st == HBMC_OK && i < launches.size(); ++i) st = launch(launches[i], stream);
  return st;
}

namespace {

constexpr int kCopyChunk = kDevRanks / 2;  // ranks per LocalCopy launch: sources then destinations

// Plan of the LocalCopy: one copy step whose item j moves table slot j
// (a send buffer) to slot kCopyChunk + j (its recv buffer), whole vector.
hbmc_status_t local_copy_plan(hbmc_comm* c, size_t count, int dtype, Plan** out) {
  auto key = std::make_tuple(-1, -1, 0, static_cast<uint64_t>(count), dtype);
  auto it = c->plans.find(key);
  if (it == c->plans.end()) {
    std::unique_ptr<Plan> p(new (std::nothrow) Plan);
    if (!p) return HBMC_ERR_NOMEM;
    Step st;
    st.mode = kCopy;
    st.nsrc = st.ndst = 1;
    for (int j = 0; j < kCopyChunk; ++j) {
      Item item;
      item.begin = 0;
      item.count = count;
      item.nsrc = item.ndst = 1;
      item.rank[0] = static_cast<uint8_t>(j);
      item.rank[1] = static_cast<uint8_t>(kCopyChunk + j);
      st.items.push_back(item);
    }
    st.max_count = count;
    st.hbm_bytes = uint64_t(2) * count * elem_bytes(dtype) * kCopyChunk;
    p->sched.steps.push_back(st);
    p->first_item.push_back(0);
    it = c->plans.emplace(key, std::move(p)).first;
  }
  *out = it->second.get();
  return upload(*out);
}

}  // namespace

hbmc_status_t run_out_of_place(hbmc_comm* c, int coll, int root, const void* const send[],
                               void* const recv[], size_t count, int dtype, int op, void* stream) {
  // every host-side check before any device work
  if (!c || c->topos.empty() || !valid_op(op) || !valid_coll(coll) || elem_bytes(dtype) == 0)
    return HBMC_ERR_INVALID_ARG;
  const int P = c->topos[0].P;
  const uint32_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  Plan* plan = nullptr;
  hbmc_status_t st = get_plan(c, coll, root, count, dtype, &plan);
  if (st != HBMC_OK) return st;
  if (count == 0) return HBMC_OK;
  if (!send) return HBMC_ERR_INVALID_ARG;
  st = check_bufs(P, recv, count, e);
  if (st != HBMC_OK) return st;
  const uint64_t bytes = uint64_t(count) * e;
  std::vector<int> moved;
  for (int r = 0; r < P; ++r) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(send[r]);
    if (!a || a % e || a + bytes < a) return HBMC_ERR_INVALID_ARG;
    if (send[r] == recv[r]) continue;
    for (int q = 0; q < P; ++q) {
      const uintptr_t b = reinterpret_cast<uintptr_t>(recv[q]);
      if (a < b + bytes && b < a + bytes) return HBMC_ERR_INVALID_ARG;  // input overlaps an output
    }
    moved.push_back(r);
  }
  std::vector<KernelDesc> launches;
  st = prepare(c, coll, root, recv, count, dtype, op, 0, 0, true, &launches);
  if (st != HBMC_OK) return st;
  if (!moved.empty()) {
    Plan* lc = nullptr;
    st = local_copy_plan(c, count, dtype, &lc);
    if (st != HBMC_OK) return st;
    for (size_t base = 0; base < moved.size(); base += kCopyChunk) {
      const int n = static_cast<int>(std::min<size_t>(kCopyChunk, moved.size() - base));
      RankPtrs cp;
      std::memset(&cp, 0, sizeof(cp));
      const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(send[moved[base]]) & 15u);
      bool aligned = true;
      for (int j = 0; j < n; ++j) {
        const int r = moved[base + j];
        cp.p[j] = static_cast<unsigned char*>(const_cast<void*>(send[r]));
        cp.p[kCopyChunk + j] = static_cast<unsigned char*>(recv[r]);
        aligned = aligned && (reinterpret_cast<uintptr_t>(send[r]) & 15u) == phase &&
                  (reinterpret_cast<uintptr_t>(recv[r]) & 15u) == phase;
      }
      StepLaunch L;
      L.dtype = dtype;
      L.op = op;
      L.mode = kCopy;
      L.nsrc = L.ndst = 1;
      L.items = lc->dev;
      L.host_items = lc->sched.steps[0].items.data();
      L.nitems = n;
      L.max_count = count;
      L.aligned = aligned;
      L.phase = phase;
      L.xcd_split = false;
      L.write_bytes = uint64_t(n) * count * elem_bytes(dtype);
      if (launch_step(L, cp, static_cast<hipStream_t>(stream)) != hipSuccess) return HBMC_ERR_HIP;
    }
  }
  for (size_t i = 0; st == HBMC_OK && i < launches.size(); ++i) st = launch(launches[i], stream);
  return st;
}

}  // namespace hbmc
