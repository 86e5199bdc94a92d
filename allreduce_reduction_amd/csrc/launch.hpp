// Host <-> kernel interface of one schedule step.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace hbmc {

constexpr int kDevRanks = 64;

// Device addresses of every rank's buffer for one call (kernel argument).
struct RankPtrs {
  unsigned char* p[kDevRanks];
};

// A work item as the kernels read it from device memory: every destination's
// elements [begin, begin+count) receive the step's combination of the
// sources' same elements.  rank[0..nsrc) are sources, then ndst destinations.
struct alignas(16) DevItem {
  uint64_t begin, count;
  uint32_t nsrc, ndst, pad0, pad1;
  uint8_t rank[2 * kDevRanks];
};

struct StepLaunch {
  int dtype, op, mode;    // element type, reduce op, Mode of plan.hpp
  int nsrc, ndst;         // one item shape per step
  const DevItem* items;   // device table of the step's items
  int nitems;
  uint64_t max_count;     // largest item, elements
  bool aligned;           // every rank buffer has the same 16-byte phase
  uint32_t phase;         // that phase, bytes
  bool xcd_split;         // give each XCD one contiguous range of tiles
};

// A step of the single-workgroup plan kernel (device table).
constexpr uint32_t kFusedMaxItems = 256;
struct FusedStep {
  uint32_t first_item, nitems, mode, pad;
};

// One kernel launch: kernel, shape and argument values, usable with
// hipLaunchKernel or as a kernel graph node.
struct KernelDesc {
  enum Kind { kVector = 0, kElement = 1, kFused = 2 };
  Kind kind = kVector;
  const void* func = nullptr;
  dim3 grid, block;
  RankPtrs ptrs;
  const DevItem* items = nullptr;
  const FusedStep* steps = nullptr;  // plan kernel only
  uint32_t nsteps = 0;               // plan kernel only
  uint32_t phase = 0, xcd = 0;
  void* argv[5];  // filled by bind(); valid while this object lives
  void bind() {
    argv[0] = &ptrs;
    argv[1] = &items;
    if (kind == kFused) {
      argv[2] = &steps;
      argv[3] = &nsteps;
      argv[4] = &phase;
    } else {
      argv[2] = &phase;
      argv[3] = &xcd;
    }
  }
};

// The single-workgroup kernel running `nsteps` steps of a plan.
void describe_fused(int dtype, int op, const RankPtrs& ptrs, const DevItem* items, const FusedStep* steps,
                    uint32_t nsteps, uint32_t phase, KernelDesc* k);

// Choose the kernel and launch shape of one step.
hipError_t describe_step(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* out);

// Enqueue one step on `stream`; returns the launch's error state.
hipError_t launch_step(const StepLaunch& s, const RankPtrs& ptrs, hipStream_t stream);

}  // namespace hbmc
