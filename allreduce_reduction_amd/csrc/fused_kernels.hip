// Single-workgroup plan kernel: for collectives that move little data, one
// launch runs a whole range of schedule steps, with a workgroup barrier in
// place of the stream-ordered launch boundary between consecutive steps.
// Fewer launches attack the per-step fixed cost, the pages' alpha term
// ([RHD] "耗时计算": one step costs alpha + n beta + n gamma; [RING-RHD]
// "Ascend950的AIVAICPU通信引擎与图模式": short messages pay mostly control
// overhead).  Items, element ops and their order are those of the step
// kernels; every vector of a step is combined by one thread, and all waves
// of the workgroup share one CU, so the barrier orders each step's writes
// before the next step's reads.
#include <hip/hip_runtime.h>

#include "elemops.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace {

using namespace dev;

constexpr int kFusedThreads = 1024;

template <int DT, int OP, int MODE>
__device__ __forceinline__ u32x4 combine_vec(const RankPtrs& ptrs, const DevItem* it, int ns, uint64_t off) {
  auto ld = [&](int s) { return *reinterpret_cast<const u32x4*>(rank_buf(ptrs, it, s) + off); };
  if constexpr (MODE == kCopy) {
    return ld(0);
  } else if constexpr (MODE == kFold) {
    u32x4 acc = ld(0);
    for (int s = 1; s < ns; ++s) acc = op_vec<DT, OP>(acc, ld(s));
    return acc;
  } else {
    u32x4 acc = ld(1);
    for (int s = 2; s < ns; ++s) acc = op_vec<DT, OP>(acc, ld(s));
    return op_vec<DT, OP>(ld(0), acc);
  }
}

// One step, all items, by the whole workgroup: the items' 16-byte bodies are
// concatenated and dealt to the threads; 16 lanes per item take the head
// elements and 16 the tail elements.
template <int DT, int OP, int MODE>
__device__ void fused_step(const RankPtrs& ptrs, const DevItem* its, uint32_t nitems, uint32_t phase,
                           uint64_t* s_start, uint32_t* s_head) {
  constexpr uint32_t E = Width<DT>::bytes;
  for (uint32_t i = threadIdx.x; i < nitems; i += blockDim.x) {
    const DevItem* it = its + i;
    uint64_t head = ((16u - ((phase + it->begin * E) & 15u)) & 15u) / E;
    if (head > it->count) head = it->count;
    s_head[i] = static_cast<uint32_t>(head);
    s_start[i + 1] = (it->count - head) * E / 16;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_start[0] = 0;
    for (uint32_t i = 0; i < nitems; ++i) s_start[i + 1] += s_start[i];
  }
  __syncthreads();
  const uint64_t total = s_start[nitems];
  for (uint64_t v = threadIdx.x; v < total; v += blockDim.x) {
    uint32_t lo = 0, hi = nitems;  // s_start[lo] <= v < s_start[hi]
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (s_start[mid] <= v) lo = mid; else hi = mid;
    }
    const DevItem* it = its + lo;
    const int ns = static_cast<int>(it->nsrc), nd = static_cast<int>(it->ndst);
    const uint64_t off = (it->begin + s_head[lo]) * E + (v - s_start[lo]) * 16;
    const u32x4 r = combine_vec<DT, OP, MODE>(ptrs, it, ns, off);
    for (int d = 0; d < nd; ++d) *reinterpret_cast<u32x4*>(rank_buf(ptrs, it, ns + d) + off) = r;
  }
  for (uint32_t k = threadIdx.x; k < nitems * 32; k += blockDim.x) {
    const uint32_t i = k / 32, lane = k % 32;
    const DevItem* it = its + i;
    const int ns = static_cast<int>(it->nsrc), nd = static_cast<int>(it->ndst);
    const uint64_t head = s_head[i];
    const uint64_t body_end = head + (s_start[i + 1] - s_start[i]) * (16 / E);
    if (lane < 16) {
      if (lane < head) do_elem<DT, OP, MODE>(ptrs, it, ns, nd, it->begin + lane);
    } else if (lane - 16 < it->count - body_end) {
      do_elem<DT, OP, MODE>(ptrs, it, ns, nd, it->begin + body_end + (lane - 16));
    }
  }
}

template <int DT, int OP>
__global__ void __launch_bounds__(kFusedThreads)
plan_fused(RankPtrs ptrs, const DevItem* __restrict__ items, const FusedStep* __restrict__ steps,
           uint32_t nsteps, uint32_t phase) {
  __shared__ uint64_t s_start[kFusedMaxItems + 1];
  __shared__ uint32_t s_head[kFusedMaxItems];
  for (uint32_t s = 0; s < nsteps; ++s) {
    const FusedStep st = steps[s];
    if (st.nitems > kFusedMaxItems) break;  // never launched so; keeps the tables in bounds
    const DevItem* its = items + st.first_item;
    switch (st.mode) {
      case kCopy: fused_step<DT, kSum, kCopy>(ptrs, its, st.nitems, phase, s_start, s_head); break;
      case kFold: fused_step<DT, OP, kFold>(ptrs, its, st.nitems, phase, s_start, s_head); break;
      default: fused_step<DT, OP, kRecvFold>(ptrs, its, st.nitems, phase, s_start, s_head); break;
    }
    __syncthreads();  // this step's writes before the next step's reads
  }
}

template <int DT>
const void* fused_fn(int op) {
  switch (op) {
    case kSum: return reinterpret_cast<const void*>(plan_fused<DT, kSum>);
    case kProd: return reinterpret_cast<const void*>(plan_fused<DT, kProd>);
    case kMax: return reinterpret_cast<const void*>(plan_fused<DT, kMax>);
    default: return reinterpret_cast<const void*>(plan_fused<DT, kMin>);
  }
}

}  // namespace

void describe_fused(int dtype, int op, const RankPtrs& ptrs, const DevItem* items, const FusedStep* steps,
                    uint32_t nsteps, uint32_t phase, KernelDesc* k) {
  switch (dtype) {
    case kF32: k->func = fused_fn<kF32>(op); break;
    case kF16: k->func = fused_fn<kF16>(op); break;
    case kBF16: k->func = fused_fn<kBF16>(op); break;
    case kI32: k->func = fused_fn<kI32>(op); break;
    default: k->func = fused_fn<kI8>(op); break;
  }
  k->kind = KernelDesc::kFused;
  k->grid = dim3(1);
  k->block = dim3(kFusedThreads);
  k->ptrs = ptrs;
  k->items = items;
  k->steps = steps;
  k->nsteps = nsteps;
  k->phase = phase;
  k->bind();
}

}  // namespace hbmc
