// Host <-> kernel interface of one schedule step.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

#include "plan.hpp"
#include "regs.hpp"

namespace hbmc {

constexpr int kDevRanks = 64;

// Device addresses of every rank's buffer for one call (kernel argument).
struct RankPtrs {
  unsigned char* p[kDevRanks];
};

// A work item as the kernels read it from device memory: every destination's
// elements [begin, begin+count) receive the step's combination of the
// sources' same elements.  rank[0..nsrc) are sources, then ndst destinations.
// The ranks follow the shape words directly, so that one scalar load reads
// an item's range, shape and first eight ranks.
struct alignas(16) DevItem {
  uint64_t begin, count;
  uint32_t nsrc, ndst;
  uint8_t rank[2 * kDevRanks];
};
static_assert(offsetof(DevItem, rank) == 24 && sizeof(DevItem) == 160, "work item record");

struct StepLaunch {
  int dtype, op, mode;    // element type, reduce op, Mode of plan.hpp
  int nsrc, ndst;         // one item shape per step
  const DevItem* items;   // device table of the step's items
  const Item* host_items; // the same items on the host (nullptr: table only)
  int nitems;
  uint64_t max_count;     // largest item, elements
  bool aligned;           // every rank buffer has the same 16-byte phase
  uint32_t phase;         // that phase, bytes
  bool xcd_split;         // give each XCD one contiguous range of tiles
  uint64_t write_bytes;   // bytes the step writes, all items and destinations
};

// Step kernel flags.
constexpr uint32_t kFlagXcdSplit = 1u;

// A work item with its operands resolved on the host, passed in the kernel
// arguments: buf[i] is the address of element `begin` of the item's i-th
// operand (sources, then destinations).  A step of at most kArgItems items
// of a compile-time shape with plain stores travels this way: a workgroup
// then waits on one scalar load (its record in the kernel-argument segment)
// before its data loads, instead of two dependent ones (the item record,
// then the pointer table).  Measured on MI355X, same session: ring
// AllReduce of 16 x 16 MiB fp32 230 vs 235 us; of 8 x 256 MiB 347.5 vs
// 346.7 GB/s bus bandwidth.
constexpr int kArgItems = 16;
constexpr int kArgMaxBufs = 10;  // 9 sources and 1 destination
template <int NB>
struct ArgItem {
  unsigned char* buf[NB];
  uint64_t count;
};
template <int NB>
struct ArgItems {
  ArgItem<NB> it[kArgItems];
};
constexpr size_t kArgBytes = sizeof(ArgItems<kArgMaxBufs>);

// A step that writes more than the memory-side cache holds (MI355X: 256 MiB
// Infinity Cache) gets the step kernel whose stores carry the nontemporal
// hint; plain stores measured 2-10% slower there.  At or below it, plain
// stores measured 2-4% faster.  That gain is not reads served by the cache:
// a 256 MiB-per-step kernel timed alone after a 512 MiB read pass, which
// leaves the cache holding other data, runs as fast as back to back.
constexpr uint64_t kCacheBytes = uint64_t(256) << 20;

// A step of the single-workgroup plan kernel (device table).
constexpr uint32_t kFusedMaxItems = 256;
struct FusedStep {
  uint32_t first_item, nitems, mode, pad;
};

// A chunk of the column kernel (device table): elements [begin,
// begin+count) of item `item` in step `step`.
struct alignas(16) DevChunk {
  uint64_t begin;
  uint32_t count, item, mode, step, pad0, pad1;
};

// A chunk as the LDS-resident column kernel reads it (device table, one run
// per column, in the column's schedule order; copied into LDS as is): bytes
// [lo, hi) of the column, relative to its first element.
struct alignas(16) DevColChunk {
  uint32_t lo, hi, step;
  uint32_t shape;                  // mode | nsrc << 8 | ndst << 16
  uint64_t dst_mask;               // bit r set when rank r is a destination
  uint32_t batch;                  // see below
  uint32_t pad;
  uint8_t rank[2 * kDevRanks];     // sources, then destinations
};
// `batch`: on the first record of a run of 2, 4 or 8 consecutive records of
// one step with the same byte range and the same two-source-one-destination
// reduce or one-to-one copy shape, the run's length; 0 on the run's other
// records; 1 on every record outside such runs.  The chunks of one step never
// conflict, so a lane may apply a run's chunks together.
static_assert(sizeof(DevColChunk) == 160, "column chunk record");

// The end of a column in a launch of all of a call's steps (device table):
// the column's trailing copy chunks only move finished values between rank
// copies, so instead of running them the kernel writes each destination
// rank's bytes [lo, hi) of the column (relative to its first element)
// straight from the LDS copy of rank `src`, which holds them once the
// column's other chunks have run.
struct alignas(16) DevColStore {
  uint32_t lo, hi, dst, src;
};
static_assert(sizeof(DevColStore) == 16, "column store record");

// The flow kernel's tables (device; see flow.hpp).  A tile is the work of
// one step on one column of elements: chunks [c_lo, c_hi) of the chunk table,
// the seq-th tile of column `col`.  A chunk is elements [begin, begin+count)
// of one item: shape = mode | nsrc << 8 | ndst << 16, rank[] its sources then
// destinations.  The control block holds the ticket and exit counters and
// the launch's give-up flag; the last workgroup to leave resets it and the
// column counters for the next launch.
constexpr int kFlowOperands = 32;
struct alignas(16) FlowTile {
  uint32_t col, seq, c_lo, c_hi;
};
struct alignas(16) FlowChunk {
  uint64_t begin;
  uint32_t count, shape;
  uint8_t rank[kFlowOperands];
};
static_assert(sizeof(FlowTile) == 16 && sizeof(FlowChunk) == 48, "flow records");
struct alignas(16) FlowCtrl {
  uint32_t next, done, abort, pad;
};
// Flow kernel flags: every wait targets a count its column never reaches, so
// each tile with a predecessor gives up after the wait bound (a host-forced
// test of the give-up path).
constexpr uint32_t kFlowUnreachable = 1u;
// Host-side choice of the instantiation whose stores carry the nontemporal
// hint (steps that write more than the memory-side cache holds).
constexpr uint32_t kFlowNtStores = 2u;

// The register-form kernel's arguments (see regs.hpp), one record per region
// of elements (grid.y): the region's whole 16-byte positions [vec_lo, vec_hi)
// of the vector (position k holds the elements from head + k * 16 / e on,
// head the elements before the buffers' first 16-byte boundary), the
// region's elements outside them [el_lo[i], el_hi[i]), and the address of
// element 0 of every operand: for the fold ptr[0..n) in fold order, for the
// tree ptr[v] and ptr[16 + v] the two ranks of leaf v (nullptr for a leaf of
// one rank).  Every operand is also a destination, except in the node form,
// where leaf v's rank receives the tree node of level lvl[v] above it (0: it
// keeps its input).
constexpr int kRegThreads = 256;
template <int NP>
struct RegRegionArg {
  uint32_t vec_lo, vec_hi;
  uint32_t el_lo[2], el_hi[2];
  uint8_t lvl[kRegMaxLeaves];
  unsigned char* ptr[NP];
};
template <int NP, int NR>
struct RegCallT {
  uint32_t n, phase;
  uint64_t count;
  RegRegionArg<NP> r[NR];
};
using RegFoldCall = RegCallT<kRegMaxLeaves, kRegMaxFoldRegions>;
using RegTreeCall = RegCallT<2 * kRegMaxLeaves, kRegMaxTreeRegions>;
constexpr size_t kRegCallBytes = sizeof(RegFoldCall) > sizeof(RegTreeCall) ? sizeof(RegFoldCall) : sizeof(RegTreeCall);

// One kernel launch: kernel, shape and argument values, usable with
// hipLaunchKernel or as a kernel graph node.
struct KernelDesc {
  enum Kind { kVector = 0, kElement = 1, kFused = 2, kColumns = 3, kColumnsLds = 4, kVectorArgs = 5, kRegs = 6,
              kFlow = 7 };
  Kind kind = kVector;
  const void* func = nullptr;
  dim3 grid, block;
  // the call's buffer table, or for kVectorArgs the step's resolved items
  // (an ArgItems of the kernel's operand count), or for kRegs a RegFoldCall
  // or RegTreeCall
  union {
    RankPtrs ptrs;
    alignas(16) unsigned char args[kArgBytes > kRegCallBytes ? kArgBytes : kRegCallBytes];
  };
  const DevItem* items = nullptr;
  uint32_t nitems = 0;               // step kernels: items of the step
  const FusedStep* steps = nullptr;  // plan kernel only
  uint32_t nsteps = 0;               // plan kernel only
  uint32_t phase = 0;
  uint32_t flags = 0;  // step kernel: kFlagXcdSplit
  // column kernel only
  const DevChunk* chunks = nullptr;
  const uint32_t* col_list = nullptr;
  const uint32_t* col_off = nullptr;
  uint32_t ncols = 0, c_lo = 0, c_hi = 0;
  // LDS-resident column kernel only
  const DevColChunk* image = nullptr;
  uint64_t col_elems = 0, count = 0;
  uint32_t nranks = 0, slot_bytes = 0, s_lo = 0, s_hi = 0;
  // and in a launch of all steps with composed stores: column g runs its
  // first col_run[g] chunk records, then store records [st_off[g],
  // st_off[g+1]) (nullptr: every chunk runs, dirty ranks stored whole)
  const DevColStore* stores = nullptr;
  const uint32_t* col_run = nullptr;
  const uint32_t* st_off = nullptr;
  const uint64_t* col_load = nullptr;  // per column, the ranks whose copies are ever read
  // flow kernel only: tables, control block, column counters, timeout
  // counter (sticky, per communicator) and the wait bound in wall-clock ticks
  const FlowTile* ftiles = nullptr;
  const FlowChunk* fchunks = nullptr;
  FlowCtrl* fctrl = nullptr;
  uint32_t* fprog = nullptr;
  uint32_t* ftimeouts = nullptr;
  uint32_t ntiles = 0, fbatch = 1;
  uint64_t wait_ticks = 0;
  uint32_t shared_bytes = 0;  // dynamic LDS per workgroup
  void* argv[16];  // filled by bind(); valid while this object lives
  void bind() {
    argv[0] = &ptrs;
    argv[1] = &items;
    if (kind == kFused) {
      argv[2] = &steps;
      argv[3] = &nsteps;
      argv[4] = &phase;
    } else if (kind == kColumns) {
      argv[2] = &chunks;
      argv[3] = &col_list;
      argv[4] = &col_off;
      argv[5] = &ncols;
      argv[6] = &c_lo;
      argv[7] = &c_hi;
      argv[8] = &phase;
    } else if (kind == kColumnsLds) {
      argv[0] = &ptrs;
      argv[1] = &image;
      argv[2] = &col_off;
      argv[3] = &ncols;
      argv[4] = &s_lo;
      argv[5] = &s_hi;
      argv[6] = &phase;
      argv[7] = &col_elems;
      argv[8] = &count;
      argv[9] = &nranks;
      argv[10] = &slot_bytes;
      argv[11] = &stores;
      argv[12] = &col_run;
      argv[13] = &st_off;
      argv[14] = &col_load;
    } else if (kind == kVectorArgs) {
      argv[0] = &flags;
      argv[1] = args;
    } else if (kind == kRegs) {
      argv[0] = args;
    } else if (kind == kFlow) {
      argv[0] = &ptrs;
      argv[1] = &ftiles;
      argv[2] = &fchunks;
      argv[3] = &ntiles;
      argv[4] = &fctrl;
      argv[5] = &fprog;
      argv[6] = &ncols;
      argv[7] = &ftimeouts;
      argv[8] = &phase;
      argv[9] = &flags;
      argv[10] = &wait_ticks;
      argv[11] = &fbatch;
    } else {
      // step kernels: the small arguments first (preloaded into registers)
      argv[0] = &items;
      argv[1] = &phase;
      argv[2] = &flags;
      argv[3] = &ptrs;
      argv[4] = &nitems;
    }
  }
};

// The column kernel over chunks [c_lo, c_hi) of a plan: `grid` one-wave
// workgroups, workgroup w running columns w, w + grid, ...
void describe_columns(int dtype, int op, const RankPtrs& ptrs, const DevItem* items, const DevChunk* chunks,
                      const uint32_t* col_list, const uint32_t* col_off, uint32_t ncols, uint32_t c_lo,
                      uint32_t c_hi, uint32_t phase, uint32_t grid, KernelDesc* k);

// The dynamic LDS a workgroup of the LDS-resident column kernel needs:
// nranks column slots, then one record per entry of the longest column's
// chunk list.
uint32_t lds_slot_bytes(uint64_t col_elems, uint32_t e);
// Lanes per workgroup: about one per 16-byte position of a column (64, 128
// or 256).
uint32_t lds_threads(uint64_t col_elems, uint32_t e);
uint64_t lds_bytes(int nranks, uint64_t col_elems, uint32_t e, uint64_t max_chunks_per_col);

// The LDS-resident column kernel over steps [s_lo, s_hi) of a plan: `grid`
// workgroups, workgroup w running columns w, w + grid, ... of `col_elems`
// elements (the last one cut at `count`); column g's chunk records are
// image[col_off[g] .. col_off[g+1]).  With `stores` (a launch of all steps)
// column g loads the ranks in col_load[g], runs its first col_run[g] records
// and then its store records stores[st_off[g] .. st_off[g+1]).
// `meta_bytes`: the LDS after the rank copies that the records of the
// largest column need.
void describe_columns_lds(int dtype, int op, const RankPtrs& ptrs, const DevColChunk* image, const uint32_t* col_off,
                          uint32_t ncols, uint32_t s_lo, uint32_t s_hi, uint32_t phase, uint64_t col_elems,
                          uint64_t count, uint32_t nranks, uint64_t meta_bytes, uint32_t grid,
                          const DevColStore* stores, const uint32_t* col_run, const uint32_t* st_off,
                          const uint64_t* col_load, KernelDesc* k);

// The register-form kernel of a whole call of P ranks over `count` elements
// whose rank buffers share the 16-byte `phase` (rp.ok).
void describe_regs(int dtype, int op, const RankPtrs& ptrs, int P, const RegPlan& rp, uint64_t count,
                   uint32_t phase, KernelDesc* k);

// The flow kernel over a whole call's tiles: `grid` workgroups take tiles
// in ticket order until none is left (see flow_kernels.hip).
void describe_flow(int dtype, int op, const RankPtrs& ptrs, const FlowTile* tiles, const FlowChunk* chunks,
                   uint32_t ntiles, FlowCtrl* ctrl, uint32_t* progress, uint32_t ncols, uint32_t* timeouts,
                   uint32_t phase, uint32_t flags, uint64_t wait_ticks, uint32_t batch, uint32_t grid,
                   KernelDesc* k);
constexpr int kFlowThreads = 256;

// The single-workgroup kernel running `nsteps` steps of a plan.
void describe_fused(int dtype, int op, const RankPtrs& ptrs, const DevItem* items, const FusedStep* steps,
                    uint32_t nsteps, uint32_t phase, KernelDesc* k);

// Choose the kernel and launch shape of one step.
hipError_t describe_step(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* out);

// Enqueue one step on `stream`; returns the launch's error state.
hipError_t launch_step(const StepLaunch& s, const RankPtrs& ptrs, hipStream_t stream);

}  // namespace hbmc
