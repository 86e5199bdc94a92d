// AllReduce without device allocation: hbmc_allreduce's schedule and step
// kernels, with the step kernels' work-item tables kept in a fixed device
// array of this library instead of memory from hipMalloc.
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy until the process ends.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; host code only ever passes that address, never
// the variable's name, to kernels and copies.  Each call copies its plan's
// item table into the array (one host-to-device copy, ordered on the call's
// stream) and then launches one step kernel per non-empty step, all of which
// read their items from the array.  Every call on one GPU shares that GPU's
// array, so calls that overlap in time on one GPU (different streams, or
// host threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "comm.hpp"
#include "launch.hpp"

namespace hbmc {
namespace {

constexpr size_t kScratchBytes = size_t(2) << 20;  // 13107 work items of 160 bytes

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of the current device's `scratch`, looked up on the
// first call on that device.
hbmc_status_t scratch_ptr(unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HBMC_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HBMC_ERR_INVALID_ARG;
  unsigned char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return HBMC_ERR_HIP;
      p = static_cast<unsigned char*>(a);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return HBMC_OK;
}

// The plan's items as the step kernels read them, step after step (built on
// the host once per plan and kept with it: the copy into the array reads it
// after the call returns).
void host_item_table(Plan* p) {
  if (p->host_table_built) return;
  size_t n = 0;
  for (const Step& s : p->sched.steps) n += s.items.size();
  p->host_table.assign(n, DevItem{});
  size_t k = 0;
  for (const Step& s : p->sched.steps)
    for (const Item& it : s.items) {
      DevItem& d = p->host_table[k++];
      std::memset(&d, 0, sizeof(d));
      d.begin = it.begin;
      d.count = it.count;
      d.nsrc = static_cast<uint32_t>(it.nsrc);
      d.ndst = static_cast<uint32_t>(it.ndst);
      std::memcpy(d.rank, it.rank, sizeof(d.rank));
    }
  p->host_table_built = true;
}

}  // namespace

hbmc_status_t allreduce_noalloc(hbmc_comm* c, void* const bufs[], size_t count, int dtype, int op, void* stream) {
  if (!c || c->topos.empty() || !valid_op(op) || elem_bytes(dtype) == 0) return HBMC_ERR_INVALID_ARG;
  const uint32_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e) return HBMC_ERR_INVALID_ARG;
  Plan* p = nullptr;
  hbmc_status_t st = get_plan(c, HBMC_COLL_ALLREDUCE, 0, count, dtype, &p);
  if (st != HBMC_OK) return st;
  const int P = c->topos[0].P;
  if (count == 0 || P == 1) return HBMC_OK;
  st = check_bufs(P, bufs, count, e);
  if (st != HBMC_OK) return st;
  size_t nitems = 0;
  for (const Step& s : p->sched.steps) nitems += s.items.size();
  if (nitems * sizeof(DevItem) > kScratchBytes) return HBMC_ERR_SCRATCH;

  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(bufs[0]) & 15u);
  bool aligned = true;
  for (int r = 0; r < P; ++r) {
    ptrs.p[r] = static_cast<unsigned char*>(bufs[r]);
    aligned = aligned && (reinterpret_cast<uintptr_t>(bufs[r]) & 15u) == phase;
  }
  // every launch is described before anything is enqueued
  std::vector<StepLaunch> steps;
  for (size_t s = 0; s < p->sched.steps.size(); ++s) {
    const Step& step = p->sched.steps[s];
    if (step.items.empty()) continue;
    StepLaunch L;
    L.dtype = dtype;
    L.op = op;
    L.mode = step.mode;
    L.nsrc = step.nsrc;
    L.ndst = step.ndst;
    L.items = nullptr;  // set below, inside the array
    L.host_items = nullptr;  // items from the device table, never the kernel arguments
    L.nitems = static_cast<int>(step.items.size());
    L.max_count = step.max_count;
    L.aligned = aligned;
    L.phase = phase;
    L.xcd_split = c->xcd_split;
    L.write_bytes = 0;
    for (const Item& it : step.items) L.write_bytes += it.count * uint64_t(it.ndst) * e;
    KernelDesc probe;
    if (describe_step(L, ptrs, &probe) != hipSuccess) return HBMC_ERR_INVALID_ARG;
    steps.push_back(L);
  }
  unsigned char* base = nullptr;
  st = scratch_ptr(&base);
  if (st != HBMC_OK) return st;
  host_item_table(p);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(base, p->host_table.data(), nitems * sizeof(DevItem), hipMemcpyHostToDevice, s) !=
      hipSuccess)
    return HBMC_ERR_HIP;
  size_t si = 0;
  for (size_t k = 0; k < p->sched.steps.size(); ++k) {
    if (p->sched.steps[k].items.empty()) continue;
    StepLaunch& L = steps[si++];
    L.items = reinterpret_cast<const DevItem*>(base) + p->first_item[k];
    if (launch_step(L, ptrs, s) != hipSuccess) return HBMC_ERR_HIP;
  }
  return HBMC_OK;
}

}  // namespace hbmc
