// Graph mode: collectives are added to a graph, their dependencies are
// analysed, and the whole graph is instantiated once and launched as a unit
// ([RING-RHD] "Ascend950的AIVAICPU通信引擎与图模式": add nodes, analyse data
// dependencies, schedule, generate the task list).  Each collective's step
// launches are captured into a child graph; a node depends on every earlier
// node whose rank buffers overlap its own, so collectives on disjoint
// buffers may run concurrently.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "comm.hpp"

using namespace hbmc;

struct hbmc_graph {
  struct Node {
    hbmc_comm* comm;
    int coll, root;
    std::vector<void*> bufs;
    size_t count;
    int dtype, op;
  };
  std::vector<Node> nodes;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool built = false;
};

namespace {

bool overlaps(const hbmc_graph::Node& a, const hbmc_graph::Node& b) {
  const uint64_t la = uint64_t(a.count) * elem_bytes(a.dtype), lb = uint64_t(b.count) * elem_bytes(b.dtype);
  if (la == 0 || lb == 0) return false;
  for (void* pa : a.bufs)
    for (void* pb : b.bufs) {
      const uintptr_t x = reinterpret_cast<uintptr_t>(pa), y = reinterpret_cast<uintptr_t>(pb);
      if (x < y + lb && y < x + la) return true;
    }
  return false;
}

void release(hbmc_graph* g) {
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  g->exec = nullptr;
  g->graph = nullptr;
}

// Body of hbmc_graph_build (the caller releases the graph on failure).
hbmc_status_t graph_build(hbmc_graph* g) {
  if (hipGraphCreate(&g->graph, 0) != hipSuccess) return HBMC_ERR_HIP;
  hbmc_status_t st = HBMC_OK;
  std::vector<hipGraphNode_t> last(g->nodes.size(), nullptr);  // each collective's final node
  // flow launches of one plan share its counters: each waits for the one before
  std::map<const void*, hipGraphNode_t> flow_last;
  for (size_t i = 0; i < g->nodes.size() && st == HBMC_OK; ++i) {
    const hbmc_graph::Node& n = g->nodes[i];
    std::vector<hipGraphNode_t> deps;
    for (size_t j = 0; j < i; ++j)
      if (overlaps(n, g->nodes[j])) deps.push_back(last[j]);
    std::vector<KernelDesc> launches;
    st = prepare(n.comm, n.coll, n.root, n.bufs.data(), n.count, n.dtype, n.op, 0, 0, true, &launches);
    if (st != HBMC_OK) break;
    if (launches.empty()) {
      if (hipGraphAddEmptyNode(&last[i], g->graph, deps.data(), deps.size()) != hipSuccess) st = HBMC_ERR_HIP;
      continue;
    }
    for (KernelDesc& k : launches) {
      k.bind();
      if (k.kind == KernelDesc::kFlow) {
        auto f = flow_last.find(k.fctrl);
        if (f != flow_last.end() && std::find(deps.begin(), deps.end(), f->second) == deps.end())
          deps.push_back(f->second);
      }
      hipKernelNodeParams prm{};
      prm.func = const_cast<void*>(k.func);
      prm.gridDim = k.grid;
      prm.blockDim = k.block;
      prm.sharedMemBytes = k.shared_bytes;
      prm.kernelParams = k.argv;
      prm.extra = nullptr;
      hipGraphNode_t node = nullptr;
      if (hipGraphAddKernelNode(&node, g->graph, deps.data(), deps.size(), &prm) != hipSuccess) {
        st = HBMC_ERR_HIP;
        break;
      }
      if (k.kind == KernelDesc::kFlow) flow_last[k.fctrl] = node;
      deps.assign(1, node);  // the next launch waits for this one
      last[i] = node;
    }
  }
  if (st == HBMC_OK && hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess)
    st = HBMC_ERR_HIP;
  if (st == HBMC_OK) g->built = true;
  return st;
}

}  // namespace

extern "C" {

hbmc_status_t hbmc_graph_create(hbmc_graph_t* out) {
  if (!out) return HBMC_ERR_INVALID_ARG;
  *out = new (std::nothrow) hbmc_graph;
  return *out ? HBMC_OK : HBMC_ERR_NOMEM;
}

hbmc_status_t hbmc_graph_add(hbmc_graph_t g, hbmc_comm_t comm, hbmc_coll_t coll, int root,
                             void* const bufs[], size_t count, hbmc_dtype_t dtype, hbmc_op_t op) {
  if (!g || g->built || !comm || !valid_op(op) || !valid_coll(coll) || elem_bytes(dtype) == 0)
    return HBMC_ERR_INVALID_ARG;
  return no_throw([&]() -> hbmc_status_t {
    Plan* p = nullptr;
    hbmc_status_t st = get_plan(comm, coll, root, count, dtype, &p);
    if (st != HBMC_OK) return st;
    hbmc_graph::Node n{comm, coll, root, {}, count, dtype, op};
    if (count > 0 && comm->topos[0].P > 1) {
      st = check_bufs(comm->topos[0].P, bufs, count, elem_bytes(dtype));
      if (st != HBMC_OK) return st;
      n.bufs.assign(bufs, bufs + comm->topos[0].P);
    }
    g->nodes.push_back(std::move(n));
    return HBMC_OK;
  });
}

hbmc_status_t hbmc_graph_build(hbmc_graph_t g) {
  if (!g || g->built) return HBMC_ERR_INVALID_ARG;
  const hbmc_status_t st = no_throw([&] { return graph_build(g); });
  if (st != HBMC_OK) release(g);  // also after an allocation failure part-way
  return st;
}

hbmc_status_t hbmc_graph_launch(hbmc_graph_t g, void* stream) {
  if (!g || !g->built) return HBMC_ERR_INVALID_ARG;
  return hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? HBMC_OK : HBMC_ERR_HIP;
}

hbmc_status_t hbmc_graph_destroy(hbmc_graph_t g) {
  if (!g) return HBMC_ERR_INVALID_ARG;
  release(g);
  delete g;
  return HBMC_OK;
}

}  // extern "C"
