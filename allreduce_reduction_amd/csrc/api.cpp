// C ABI of hbmcoll: argument checks, schedule cache, step launches.
#include "hbmcoll.h"

#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <string>

#include "comm.hpp"

using namespace hbmc;

namespace {

// Body of hbmc_comm_create (out is non-null and cleared).
hbmc_status_t comm_create(int nranks, hbmc_algo_t algo, int servers, int ranks_per_server, size_t loop_bytes,
                          hbmc_comm_t* out) {
  if (nranks < 1 || nranks > kMaxRanks) return HBMC_ERR_INVALID_ARG;
  int a = algo;
  if (a == HBMC_ALGO_ENV) {
    const char* env = std::getenv("HBMC_ALGO");
    if (!env) return HBMC_ERR_INVALID_ARG;
    std::string v(env);
    if (v == "ring") a = HBMC_ALGO_RING;
    else if (v == "rhd" || v == "H-D_R") a = HBMC_ALGO_RHD;
    else if (v == "pipeline") a = HBMC_ALGO_PIPELINE;
    else if (v == "flat") a = HBMC_ALGO_FLAT;
    else if (v == "tree") a = HBMC_ALGO_TREE;
    else if (v == "hier") a = HBMC_ALGO_HIER;
    else if (v == "auto") a = HBMC_ALGO_AUTO;
    else if (v == "auto_rules") a = HBMC_ALGO_AUTO_RULES;
    else return HBMC_ERR_INVALID_ARG;
  }
  Topology t;
  t.P = nranks;
  std::vector<Topology> topos;
  switch (a) {
    case HBMC_ALGO_RING: t.algo = kRing; break;
    case HBMC_ALGO_RHD: t.algo = kRhd; break;
    case HBMC_ALGO_FLAT: t.algo = kFlat; break;
    case HBMC_ALGO_TREE:
      t.algo = kTree;
      t.K = ranks_per_server == 0 ? 2 : ranks_per_server;
      if (t.K < 2 || t.K > kMaxRanks) return HBMC_ERR_INVALID_ARG;
      break;
    case HBMC_ALGO_PIPELINE:
    case HBMC_ALGO_HIER:
      t.algo = a == HBMC_ALGO_PIPELINE ? kPipeline : kHier;
      if (servers < 1 || ranks_per_server < 1 || int64_t(servers) * ranks_per_server != nranks)
        return HBMC_ERR_INVALID_ARG;
      t.S = servers;
      t.M = ranks_per_server;
      t.loop_bytes = loop_bytes;
      break;
    case HBMC_ALGO_AUTO: {
      // candidates: ring, RHD, Flat, binary tree; with a server shape also
      // the pipeline and the hierarchical AllReduce
      for (Algo al : {kRing, kRhd, kFlat, kTree}) {
        Topology c = t;
        c.algo = al;
        topos.push_back(c);
      }
      if (servers > 0 || ranks_per_server > 0) {
        if (servers < 1 || ranks_per_server < 1 || int64_t(servers) * ranks_per_server != nranks)
          return HBMC_ERR_INVALID_ARG;
        for (Algo al : {kPipeline, kHier}) {
          Topology c = t;
          c.algo = al;
          c.S = servers;
          c.M = ranks_per_server;
          c.loop_bytes = loop_bytes;
          topos.push_back(c);
        }
      }
      break;
    }
    case HBMC_ALGO_AUTO_RULES:
      // the rules pick among these three, by index (see choose_topology)
      for (Algo al : {kRing, kRhd, kFlat}) {
        Topology c = t;
        c.algo = al;
        topos.push_back(c);
      }
      break;
    default: return HBMC_ERR_INVALID_ARG;
  }
  if (topos.empty()) topos.push_back(t);
  std::unique_ptr<hbmc_comm> c(new (std::nothrow) hbmc_comm);
  if (!c) return HBMC_ERR_NOMEM;
  c->topos = topos;
  c->auto_select = a == HBMC_ALGO_AUTO || a == HBMC_ALGO_AUTO_RULES;
  c->auto_rules = a == HBMC_ALGO_AUTO_RULES;
  if (const char* fl = std::getenv("HBMC_FUSED_LIMIT")) c->fused_limit = std::strtoull(fl, nullptr, 10);
  if (const char* cl = std::getenv("HBMC_COLUMNS_LIMIT")) c->columns_limit = std::strtoull(cl, nullptr, 10);
  if (const char* ex = std::getenv("HBMC_EXEC")) {
    const std::string v(ex);
    if (v == "steps") c->exec_mode = kExecSteps;
    else if (v == "fused") c->exec_mode = kExecFused;
    else if (v == "columns") c->exec_mode = kExecColumns;
    else if (v == "lds") c->exec_mode = kExecLds;
    else if (v == "regs") c->exec_mode = kExecRegs;
    else if (v == "flow") c->exec_mode = kExecFlow;
    else if (v == "auto") c->exec_mode = kExecAuto;
  }
  const char* xs = std::getenv("HBMC_XCD_SPLIT");
  c->xcd_split = xs && xs[0] == '1';
  *out = c.release();
  return HBMC_OK;
}

}  // namespace

extern "C" {

hbmc_status_t hbmc_comm_create(int nranks, hbmc_algo_t algo, int servers, int ranks_per_server,
                               size_t loop_bytes, hbmc_comm_t* out) {
  if (!out) return HBMC_ERR_INVALID_ARG;
  *out = nullptr;
  return no_throw([&] { return comm_create(nranks, algo, servers, ranks_per_server, loop_bytes, out); });
}

hbmc_status_t hbmc_comm_set_fused_limit(hbmc_comm_t comm, uint64_t max_bytes) {
  if (!comm) return HBMC_ERR_INVALID_ARG;
  comm->fused_limit = max_bytes;
  return HBMC_OK;
}

hbmc_status_t hbmc_comm_set_columns(hbmc_comm_t comm, uint64_t max_total_bytes, uint64_t column_bytes) {
  if (!comm) return HBMC_ERR_INVALID_ARG;
  if (column_bytes != 0 && (column_bytes < 16 || column_bytes > (uint64_t(1) << 31))) return HBMC_ERR_INVALID_ARG;
  comm->columns_limit = max_total_bytes;
  comm->column_bytes = column_bytes;
  return HBMC_OK;
}

hbmc_status_t hbmc_comm_set_flow(hbmc_comm_t comm, uint64_t tile_bytes, uint32_t wgs_per_cu,
                                 uint32_t tiles_per_ticket, uint32_t wait_us, uint32_t flags) {
  if (!comm || tile_bytes < 16 || tile_bytes > (uint64_t(1) << 31) || wgs_per_cu == 0 || wgs_per_cu > 64 ||
      tiles_per_ticket == 0 || tiles_per_ticket > 4096 || wait_us == 0 ||
      (flags & ~uint32_t(HBMC_FLOW_UNREACHABLE)) != 0)
    return HBMC_ERR_INVALID_ARG;
  comm->flow_tile_bytes = tile_bytes;
  comm->flow_wgs_per_cu = wgs_per_cu;
  comm->flow_batch = tiles_per_ticket;
  comm->flow_wait_us = wait_us;
  comm->flow_flags = (flags & HBMC_FLOW_UNREACHABLE) ? kFlowUnreachable : 0u;
  return HBMC_OK;
}

hbmc_status_t hbmc_comm_flow_timeouts(hbmc_comm_t comm, uint32_t* count) {
  if (!comm || !count) return HBMC_ERR_INVALID_ARG;
  return no_throw([&] { return flow_timeouts(comm, count); });
}

hbmc_status_t hbmc_comm_set_exec_mode(hbmc_comm_t comm, hbmc_exec_t mode) {
  if (!comm || mode < HBMC_EXEC_AUTO || mode > HBMC_EXEC_FLOW) return HBMC_ERR_INVALID_ARG;
  comm->exec_mode = static_cast<int>(mode);
  return HBMC_OK;
}

hbmc_status_t hbmc_exec_choice(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                               int first_step, int last_step, hbmc_exec_t* mode) {
  return no_throw([&]() -> hbmc_status_t {
    if (!mode) return HBMC_ERR_INVALID_ARG;
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    const int nsteps = static_cast<int>(p->sched.steps.size());
    if (first_step == 0 && last_step == 0) last_step = nsteps;
    if (first_step < 0 || last_step > nsteps || first_step > last_step) return HBMC_ERR_INVALID_ARG;
    *mode = HBMC_EXEC_STEPS;
    if (count == 0 || comm->topos[0].P == 1 || first_step == last_step) return HBMC_OK;
    int m = kExecSteps;
    st = choose_exec(comm, p, first_step, last_step, count, elem_bytes(dtype), true, &m);
    if (st != HBMC_OK) return st;
    *mode = static_cast<hbmc_exec_t>(m);
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_exec_bytes(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                              int first_step, int last_step, hbmc_exec_t mode, uint64_t* bytes) {
  return no_throw([&]() -> hbmc_status_t {
    if (!bytes || mode < HBMC_EXEC_AUTO || mode > HBMC_EXEC_FLOW) return HBMC_ERR_INVALID_ARG;
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    const int nsteps = static_cast<int>(p->sched.steps.size());
    if (first_step == 0 && last_step == 0) last_step = nsteps;
    if (first_step < 0 || last_step > nsteps || first_step > last_step) return HBMC_ERR_INVALID_ARG;
    int m = static_cast<int>(mode);
    if (m == kExecAuto) {
      m = kExecSteps;
      if (count > 0 && comm->topos[0].P > 1 && first_step < last_step) {
        st = choose_exec(comm, p, first_step, last_step, count, elem_bytes(dtype), true, &m);
        if (st != HBMC_OK) return st;
      }
    }
    return exec_bytes(comm, p, first_step, last_step, count, elem_bytes(dtype), m, bytes);
  });
}

hbmc_status_t hbmc_comm_set_cost_model(hbmc_comm_t comm, double alpha_us, double beta_gbps) {
  if (!comm || !(alpha_us >= 0.0) || !(beta_gbps > 0.0)) return HBMC_ERR_INVALID_ARG;
  comm->alpha_us = alpha_us;
  comm->beta_gbps = beta_gbps;
  comm->chosen.clear();
  return HBMC_OK;
}

hbmc_status_t hbmc_auto_choice(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                               hbmc_dtype_t dtype, hbmc_algo_t* algo) {
  return no_throw([&]() -> hbmc_status_t {
    if (!algo) return HBMC_ERR_INVALID_ARG;
    int ti = 0;
    hbmc_status_t st = choose_topology(comm, coll, root, count, dtype, &ti);
    if (st != HBMC_OK) return st;
    switch (comm->topos[ti].algo) {
      case kRing: *algo = HBMC_ALGO_RING; break;
      case kRhd: *algo = HBMC_ALGO_RHD; break;
      case kPipeline: *algo = HBMC_ALGO_PIPELINE; break;
      case kFlat: *algo = HBMC_ALGO_FLAT; break;
      case kTree: *algo = HBMC_ALGO_TREE; break;
      default: *algo = HBMC_ALGO_HIER; break;
    }
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_comm_destroy(hbmc_comm_t comm) {
  if (!comm) return HBMC_ERR_INVALID_ARG;
  hbmc_status_t st = HBMC_OK;
  for (auto& kv : comm->plans) {
    if (kv.second->dev && hipFree(kv.second->dev) != hipSuccess) st = HBMC_ERR_HIP;
    if (kv.second->cols_mem && hipFree(kv.second->cols_mem) != hipSuccess) st = HBMC_ERR_HIP;
    if (kv.second->lds_mem && hipFree(kv.second->lds_mem) != hipSuccess) st = HBMC_ERR_HIP;
    for (auto& f : kv.second->flow)
      if (f.second.mem && hipFree(f.second.mem) != hipSuccess) st = HBMC_ERR_HIP;
    for (void* m : kv.second->retired)
      if (hipFree(m) != hipSuccess) st = HBMC_ERR_HIP;
  }
  delete comm;
  return st;
}

hbmc_status_t hbmc_allreduce(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                             hbmc_op_t op, void* stream) {
  return no_throw([&] { return run(comm, HBMC_COLL_ALLREDUCE, 0, bufs, count, dtype, op, 0, 0, true, stream); });
}

hbmc_status_t hbmc_allreduce_noalloc(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                                     hbmc_op_t op, void* stream) {
  return no_throw([&] { return allreduce_noalloc(comm, bufs, count, dtype, op, stream); });
}

hbmc_status_t hbmc_reduce_scatter(hbmc_comm_t comm, void* const bufs[], size_t count,
                                  hbmc_dtype_t dtype, hbmc_op_t op, void* stream) {
  return no_throw([&] { return run(comm, HBMC_COLL_REDUCE_SCATTER, 0, bufs, count, dtype, op, 0, 0, true, stream); });
}

hbmc_status_t hbmc_all_gather(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                              hbmc_op_t op, void* stream) {
  return no_throw([&] { return run(comm, HBMC_COLL_ALL_GATHER, 0, bufs, count, dtype, op, 0, 0, true, stream); });
}

hbmc_status_t hbmc_reduce(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                          hbmc_op_t op, int root, void* stream) {
  return no_throw([&] { return run(comm, HBMC_COLL_REDUCE, root, bufs, count, dtype, op, 0, 0, true, stream); });
}

hbmc_status_t hbmc_broadcast(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                             int root, void* stream) {
  return no_throw([&] { return run(comm, HBMC_COLL_BROADCAST, root, bufs, count, dtype, HBMC_SUM, 0, 0, true, stream); });
}

hbmc_status_t hbmc_collective_oop(hbmc_comm_t comm, hbmc_coll_t coll, int root, const void* const send[],
                                  void* const recv[], size_t count, hbmc_dtype_t dtype, hbmc_op_t op,
                                  void* stream) {
  return no_throw([&] { return run_out_of_place(comm, coll, root, send, recv, count, dtype, op, stream); });
}

hbmc_status_t hbmc_run_steps(hbmc_comm_t comm, hbmc_coll_t coll, int root, void* const bufs[],
                             size_t count, hbmc_dtype_t dtype, hbmc_op_t op, int first_step,
                             int last_step, void* stream) {
  return no_throw([&] { return run(comm, coll, root, bufs, count, dtype, op, first_step, last_step, false, stream); });
}

hbmc_status_t hbmc_plan_info(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                             hbmc_dtype_t dtype, int* nsteps, uint64_t* hbm_bytes,
                             uint64_t* max_recv_bytes) {
  return no_throw([&]() -> hbmc_status_t {
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    if (nsteps) *nsteps = static_cast<int>(p->sched.steps.size());
    if (hbm_bytes) *hbm_bytes = p->sched.hbm_bytes;
    if (max_recv_bytes) *max_recv_bytes = p->sched.max_recv_bytes;
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_plan_step_info(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                                  hbmc_dtype_t dtype, int step, int* nitems, uint64_t* hbm_bytes) {
  return no_throw([&]() -> hbmc_status_t {
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    if (step < 0 || step >= static_cast<int>(p->sched.steps.size())) return HBMC_ERR_INVALID_ARG;
    const Step& s = p->sched.steps[step];
    if (nitems) *nitems = static_cast<int>(s.items.size());
    if (hbm_bytes) *hbm_bytes = s.hbm_bytes;
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_plan_items(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                              hbmc_dtype_t dtype, hbmc_item_t* out, size_t cap, size_t* n_items) {
  return no_throw([&]() -> hbmc_status_t {
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    size_t k = 0;
    for (size_t s = 0; s < p->sched.steps.size(); ++s) {
      const Step& step = p->sched.steps[s];
      for (const Item& it : step.items) {
        if (out && k < cap) {
          hbmc_item_t& o = out[k];
          o.step = static_cast<int32_t>(s);
          o.mode = step.mode;
          o.nsrc = it.nsrc;
          o.ndst = it.ndst;
          o.begin = it.begin;
          o.count = it.count;
          std::memcpy(o.rank, it.rank, sizeof(o.rank));
        }
        ++k;
      }
    }
    if (n_items) *n_items = k;
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_plan_chunks(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                               hbmc_dtype_t dtype, uint64_t chunk_bytes, hbmc_chunk_t* chunks, size_t cap,
                               size_t* n_chunks, uint32_t* deps, size_t dcap, size_t* n_deps) {
  return no_throw([&]() -> hbmc_status_t {
    if (chunk_bytes < 16 || chunk_bytes > (uint64_t(1) << 31)) return HBMC_ERR_INVALID_ARG;
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    ColumnTable f;
    if (!build_columns(p->sched, comm->topos[0].P, column_elems(chunk_bytes, count, elem_bytes(dtype), 1), true, &f))
      return HBMC_ERR_INVALID_ARG;
    for (size_t i = 0; chunks && i < f.chunks.size() && i < cap; ++i) {
      const ColumnChunk& c = f.chunks[i];
      chunks[i] = hbmc_chunk_t{c.begin, c.count, c.item, c.step, c.dep_lo, c.dep_hi, 0};
    }
    for (size_t i = 0; deps && i < f.deps.size() && i < dcap; ++i) deps[i] = f.deps[i];
    if (n_chunks) *n_chunks = f.chunks.size();
    if (n_deps) *n_deps = f.deps.size();
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_plan_flow(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                             int first_step, int last_step, uint64_t tile_bytes, hbmc_flow_tile_t* tiles,
                             size_t cap, size_t* n_tiles, hbmc_flow_chunk_t* chunks, size_t ccap,
                             size_t* n_chunks) {
  return no_throw([&]() -> hbmc_status_t {
    if (tile_bytes < 16 || tile_bytes > (uint64_t(1) << 31)) return HBMC_ERR_INVALID_ARG;
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    const int nsteps = static_cast<int>(p->sched.steps.size());
    const int last = last_step < 0 ? nsteps : last_step;
    if (first_step < 0 || first_step > last || last > nsteps) return HBMC_ERR_INVALID_ARG;
    const uint32_t e = elem_bytes(dtype);
    FlowTable f;
    if (!build_flow(p->sched, first_step, last, count, e, tile_bytes / 16 * 16 / e, &f))
      return HBMC_ERR_UNSUPPORTED;
    for (size_t i = 0; tiles && i < f.tiles.size() && i < cap; ++i) {
      const FlowTile& t = f.tiles[i];
      tiles[i] = hbmc_flow_tile_t{t.col, t.seq, f.tile_step[i], t.c_lo, t.c_hi, 0};
    }
    for (size_t i = 0; chunks && i < f.chunks.size() && i < ccap; ++i)
      chunks[i] = hbmc_flow_chunk_t{f.chunks[i].begin, f.chunks[i].count, f.chunk_item[i]};
    if (n_tiles) *n_tiles = f.tiles.size();
    if (n_chunks) *n_chunks = f.chunks.size();
    return HBMC_OK;
  });
}

const char* hbmc_status_string(hbmc_status_t status) {
  switch (status) {
    case HBMC_OK: return "success";
    case HBMC_ERR_INVALID_ARG: return "invalid argument";
    case HBMC_ERR_UNSUPPORTED: return "unsupported collective for this algorithm (Reduce / Broadcast: RHD only; Flat, tree, hierarchical: AllReduce only)";
    case HBMC_ERR_HIP: return "HIP error";
    case HBMC_ERR_NOMEM: return "out of memory";
    case HBMC_ERR_SCRATCH: return "the schedule's work-item table exceeds the no-allocation AllReduce's 2 MiB device array";
    default: return "unknown status";
  }
}

}  // extern "C"
