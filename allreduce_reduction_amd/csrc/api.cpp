// C ABI of hbmcoll: argument checks, schedule cache, step launches.
#include "hbmcoll.h"

#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"

using namespace hbmc;

namespace {

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

struct Plan {
  Schedule sched;
  std::vector<size_t> first_item;  // offset of each step's items in the device table
  DevItem* dev = nullptr;
  int device = -1;
};

}  // namespace

struct hbmc_comm {
  Topology topo;
  bool xcd_split = false;
  std::map<std::tuple<int, uint64_t, int>, std::unique_ptr<Plan>> plans;
};

namespace {

hbmc_status_t from_build(BuildStatus b) {
  switch (b) {
    case kBuilt: return HBMC_OK;
    case kUnsupported: return HBMC_ERR_UNSUPPORTED;
    default: return HBMC_ERR_INVALID_ARG;
  }
}

bool valid_coll(int c) { return c >= HBMC_COLL_ALLREDUCE && c <= HBMC_COLL_ALL_GATHER; }
bool valid_op(int op) { return op >= HBMC_SUM && op <= HBMC_MIN; }

// Build (or fetch) the host schedule of (coll, count, dtype).
hbmc_status_t get_plan(hbmc_comm* c, int coll, size_t count, int dtype, Plan** out) {
  const uint32_t e = elem_bytes(dtype);
  if (!c || e == 0 || !valid_coll(coll)) return HBMC_ERR_INVALID_ARG;
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  auto key = std::make_tuple(coll, static_cast<uint64_t>(count), dtype);
  auto it = c->plans.find(key);
  if (it != c->plans.end()) {
    *out = it->second.get();
    return HBMC_OK;
  }
  std::unique_ptr<Plan> p(new (std::nothrow) Plan);
  if (!p) return HBMC_ERR_NOMEM;
  hbmc_status_t st = from_build(build_schedule(c->topo, static_cast<Coll>(coll), count, e, &p->sched));
  if (st != HBMC_OK) return st;
  size_t off = 0;
  for (const Step& s : p->sched.steps) {
    p->first_item.push_back(off);
    off += s.items.size();
  }
  *out = p.get();
  c->plans.emplace(key, std::move(p));
  return HBMC_OK;
}

// Copy the plan's item tables to the current device (once per plan).
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
  void* mem = nullptr;
  if (hipMalloc(&mem, n * sizeof(DevItem)) != hipSuccess) return HBMC_ERR_NOMEM;
  if (hipMemcpy(mem, host.data(), n * sizeof(DevItem), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(mem);
    return HBMC_ERR_HIP;
  }
  p->dev = static_cast<DevItem*>(mem);
  p->device = dev;
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

hbmc_status_t run(hbmc_comm* c, int coll, void* const bufs[], size_t count, int dtype, int op,
                  int first, int last, bool whole, void* stream) {
  if (!c || !valid_op(op) || !valid_coll(coll) || elem_bytes(dtype) == 0) return HBMC_ERR_INVALID_ARG;
  const uint32_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(c, coll, count, dtype, &p);
  if (st != HBMC_OK) return st;
  const int nsteps = static_cast<int>(p->sched.steps.size());
  if (whole) {
    first = 0;
    last = nsteps;
  } else if (first < 0 || last > nsteps || first >= last) {
    return HBMC_ERR_INVALID_ARG;
  }
  if (count == 0 || c->topo.P == 1) return HBMC_OK;
  st = check_bufs(c->topo.P, bufs, count, e);
  if (st != HBMC_OK) return st;
  st = upload(p);
  if (st != HBMC_OK) return st;

  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(bufs[0]) & 15u);
  bool aligned = true;
  for (int r = 0; r < c->topo.P; ++r) {
    ptrs.p[r] = static_cast<unsigned char*>(bufs[r]);
    aligned = aligned && (reinterpret_cast<uintptr_t>(bufs[r]) & 15u) == phase;
  }
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
    L.nitems = static_cast<int>(step.items.size());
    L.max_count = step.max_count;
    L.aligned = aligned;
    L.phase = phase;
    L.xcd_split = c->xcd_split;
    if (launch_step(L, ptrs, static_cast<hipStream_t>(stream)) != hipSuccess) return HBMC_ERR_HIP;
  }
  return HBMC_OK;
}

}  // namespace

extern "C" {

hbmc_status_t hbmc_comm_create(int nranks, hbmc_algo_t algo, int servers, int ranks_per_server,
                               size_t loop_bytes, hbmc_comm_t* out) {
  if (!out) return HBMC_ERR_INVALID_ARG;
  *out = nullptr;
  if (nranks < 1 || nranks > kMaxRanks) return HBMC_ERR_INVALID_ARG;
  int a = algo;
  if (a == HBMC_ALGO_ENV) {
    const char* env = std::getenv("HBMC_ALGO");
    if (!env) return HBMC_ERR_INVALID_ARG;
    std::string v(env);
    if (v == "ring") a = HBMC_ALGO_RING;
    else if (v == "rhd" || v == "H-D_R") a = HBMC_ALGO_RHD;
    else if (v == "pipeline") a = HBMC_ALGO_PIPELINE;
    else return HBMC_ERR_INVALID_ARG;
  }
  if (a < HBMC_ALGO_RING || a > HBMC_ALGO_PIPELINE) return HBMC_ERR_INVALID_ARG;
  Topology t;
  t.P = nranks;
  t.algo = static_cast<Algo>(a);
  if (a == HBMC_ALGO_PIPELINE) {
    if (servers < 1 || ranks_per_server < 1 || servers * ranks_per_server != nranks)
      return HBMC_ERR_INVALID_ARG;
    t.S = servers;
    t.M = ranks_per_server;
    t.loop_bytes = loop_bytes;
  }
  hbmc_comm* c = new (std::nothrow) hbmc_comm;
  if (!c) return HBMC_ERR_NOMEM;
  c->topo = t;
  const char* xs = std::getenv("HBMC_XCD_SPLIT");
  c->xcd_split = xs && xs[0] == '1';
  *out = c;
  return HBMC_OK;
}

hbmc_status_t hbmc_comm_destroy(hbmc_comm_t comm) {
  if (!comm) return HBMC_ERR_INVALID_ARG;
  hbmc_status_t st = HBMC_OK;
  for (auto& kv : comm->plans)
    if (kv.second->dev && hipFree(kv.second->dev) != hipSuccess) st = HBMC_ERR_HIP;
  delete comm;
  return st;
}

hbmc_status_t hbmc_allreduce(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                             hbmc_op_t op, void* stream) {
  return run(comm, HBMC_COLL_ALLREDUCE, bufs, count, dtype, op, 0, 0, true, stream);
}

hbmc_status_t hbmc_reduce_scatter(hbmc_comm_t comm, void* const bufs[], size_t count,
                                  hbmc_dtype_t dtype, hbmc_op_t op, void* stream) {
  return run(comm, HBMC_COLL_REDUCE_SCATTER, bufs, count, dtype, op, 0, 0, true, stream);
}

hbmc_status_t hbmc_all_gather(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                              hbmc_op_t op, void* stream) {
  return run(comm, HBMC_COLL_ALL_GATHER, bufs, count, dtype, op, 0, 0, true, stream);
}

hbmc_status_t hbmc_run_steps(hbmc_comm_t comm, hbmc_coll_t coll, void* const bufs[], size_t count,
                             hbmc_dtype_t dtype, hbmc_op_t op, int first_step, int last_step,
                             void* stream) {
  return run(comm, coll, bufs, count, dtype, op, first_step, last_step, false, stream);
}

hbmc_status_t hbmc_plan_info(hbmc_comm_t comm, hbmc_coll_t coll, size_t count, hbmc_dtype_t dtype,
                             int* nsteps, uint64_t* hbm_bytes, uint64_t* max_recv_bytes) {
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(comm, coll, count, dtype, &p);
  if (st != HBMC_OK) return st;
  if (nsteps) *nsteps = static_cast<int>(p->sched.steps.size());
  if (hbm_bytes) *hbm_bytes = p->sched.hbm_bytes;
  if (max_recv_bytes) *max_recv_bytes = p->sched.max_recv_bytes;
  return HBMC_OK;
}

hbmc_status_t hbmc_plan_step_info(hbmc_comm_t comm, hbmc_coll_t coll, size_t count,
                                  hbmc_dtype_t dtype, int step, int* nitems, uint64_t* hbm_bytes) {
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(comm, coll, count, dtype, &p);
  if (st != HBMC_OK) return st;
  if (step < 0 || step >= static_cast<int>(p->sched.steps.size())) return HBMC_ERR_INVALID_ARG;
  const Step& s = p->sched.steps[step];
  if (nitems) *nitems = static_cast<int>(s.items.size());
  if (hbm_bytes) *hbm_bytes = s.hbm_bytes;
  return HBMC_OK;
}

hbmc_status_t hbmc_plan_items(hbmc_comm_t comm, hbmc_coll_t coll, size_t count, hbmc_dtype_t dtype,
                              hbmc_item_t* out, size_t cap, size_t* n_items) {
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(comm, coll, count, dtype, &p);
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
}

const char* hbmc_status_string(hbmc_status_t status) {
  switch (status) {
    case HBMC_OK: return "success";
    case HBMC_ERR_INVALID_ARG: return "invalid argument";
    case HBMC_ERR_UNSUPPORTED: return "unsupported (RHD reduce_scatter/all_gather needs a power-of-two rank count)";
    case HBMC_ERR_HIP: return "HIP error";
    case HBMC_ERR_NOMEM: return "out of memory";
    default: return "unknown status";
  }
}

}  // extern "C"
