// Communicator internals shared by the C entry points and graph mode.
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <memory>
#include <tuple>
#include <vector>

#include "columns.hpp"
#include "flow.hpp"
#include "hbmcoll.h"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {

// How a call's steps are launched.
enum ExecMode : int {
  kExecAuto = 0, kExecSteps = 1, kExecFused = 2, kExecColumns = 3, kExecLds = 4, kExecRegs = 5, kExecFlow = 6
};

// Modelled time (us) of a range of steps in each launch form, fitted to
// measurements on MI355X (one launch per step, the single-workgroup kernel,
// the column kernel and the LDS-resident column kernel; see choose_exec).
// The LDS form's per-chunk cost was fitted on fp16 max, its slowest element
// op; cheaper ops run their chunks faster than modelled.
struct ExecModel {
  double launch_us = 4.2;       // host-side cost of one step launch (bounds eager small steps)
  double step_us = 3.0;         // fixed GPU cost of one step kernel
  double hbm_gbps = 6400.0;     // step kernels' streaming rate
  double fused_us = 2.0;        // single-workgroup kernel: launch
  double fused_step_us = 1.6;   //   per step (workgroup barrier, loads, stores)
  double fused_gbps = 33.0;     //   one compute unit's streaming rate
  double col_us = 4.0;          // column kernel: launch
  double col_hop_us = 0.85;     //   per chunk of the longest column (run one after another)
  double col_gbps = 6000.0;     //   streaming rate
  double lds_us = 4.0;          // LDS-resident column kernel: launch, load and store round trips
  double lds_chunk_us = 0.56;   //   per chunk of the longest column (one wave's pass over it)
  double lds_gbps = 5000.0;     //   loading and storing every rank buffer once
};

uint32_t elem_bytes(int dtype);
bool valid_coll(int c);
bool valid_op(int op);

// The LDS-resident column kernel's tables on the host, for the column
// length `built_col` (see upload_lds_tables): chunk records column after
// column, store records, per column the records run before the stores, the
// store records' offsets and the ranks loaded; the LDS their records need.
struct LdsHost {
  uint64_t built_col = 0;
  std::vector<DevColChunk> image;
  std::vector<DevColStore> stores;
  std::vector<uint32_t> col_run, st_off;
  std::vector<uint64_t> col_load;
  uint64_t meta_steps = 0, meta_whole = 0;
  bool any_tail = false;
  bool stores_fit = false;  // launches of all steps use the store records
};

// The flow kernel's state for one step range of a plan: its host table for
// the communicator's tile length, and one device allocation (on the plan's
// device) holding the control block, the count of waits that gave up, the
// column counters, the tiles and the chunks (built on first launch).
struct FlowSet {
  FlowTable table;
  bool built = false;
  bool ok = false;  // the steps fit the flow records
  void* mem = nullptr;
  FlowCtrl* ctrl = nullptr;
  uint32_t* timeouts = nullptr;
  uint32_t* prog = nullptr;
  FlowTile* tiles = nullptr;
  FlowChunk* chunks = nullptr;
};

// A cached schedule and its device item table (uploaded on first use).
struct Plan {
  Schedule sched;
  int coll = 0;                    // the collective it implements
  // the register form of the whole call, derived on first use
  bool regs_built = false;
  RegPlan regs;
  std::vector<size_t> first_item;  // offset of each step's items in the device table
  DevItem* dev = nullptr;          // all items, step after step
  FusedStep* dev_steps = nullptr;  // one entry per step, for the single-workgroup kernel
  int device = -1;
  // column kernel tables (one allocation), built on first use; the host table
  // also serves the launch-form choice
  ColumnTable cols;
  void* cols_mem = nullptr;
  DevChunk* dev_chunks = nullptr;
  uint32_t* dev_col_list = nullptr;
  uint32_t* dev_col_off = nullptr;
  // the LDS-resident column kernel: its column length, chosen per plan for
  // the communicator's column_bytes setting `lds_key`; the chunks of its
  // longest column; its own column table and, built on first launch, the
  // device chunk records and column offsets (one allocation)
  uint64_t lds_key = UINT64_MAX;
  uint64_t lds_col = 0;  // 0: no column length fits one workgroup's LDS
  uint64_t lds_chunks = 0;   // chunks of the longest column (its LDS records)
  double lds_longest = 0.0;  // serial chunk passes of the busiest column (for the cost model)
  double lds_longest_whole = 0.0;  // the same without the schedule's trailing copy steps
  double lds_whole_buffers = 0.0;  // rank buffers' worth of bytes a launch of all steps moves
  ColumnTable lds_cols;
  LdsHost lh;
  void* lds_mem = nullptr;
  DevColChunk* dev_image = nullptr;
  uint32_t* dev_lds_col_off = nullptr;
  // composed stores for launches of all steps (see DevColStore), built with
  // the tables: per column the chunk records to run and its store records;
  // the LDS the records of one column need at most (all chunks; leading
  // chunks and stores); stores used only when the latter fits
  DevColStore* dev_stores = nullptr;
  uint32_t* dev_col_run = nullptr;
  uint32_t* dev_st_off = nullptr;
  uint64_t* dev_col_load = nullptr;
  uint64_t lds_meta_steps = 0;
  uint64_t lds_meta_whole = 0;
  bool lds_stores = false;
  // the item table as the step kernels read it, kept on the host for the
  // no-allocation AllReduce, which copies it into its fixed device array on
  // every call
  std::vector<DevItem> host_table;
  bool host_table_built = false;
  // the flow kernel, per step range [first, last) launched in that form; and
  // the allocations of earlier tile lengths, whose counts are still read
  std::map<std::pair<int, int>, FlowSet> flow;
  std::vector<void*> flow_old;
  // device tables of earlier column lengths: graphs built or captured before
  // the length changed still point at them, so they are kept until the
  // communicator is destroyed
  std::vector<void*> retired;
};

}  // namespace hbmc

struct hbmc_comm {
  // One topology, or for AUTO the candidates the cost model chooses among.
  std::vector<hbmc::Topology> topos;
  bool auto_select = false;
  bool auto_rules = false;    // AUTO_RULES: topos = {ring, RHD, Flat}, picked by the pages' rules
  double alpha_us = 4.4;      // launch-to-launch cost of one step, measured eager on MI355X
  double beta_gbps = 6400.0;  // sustained HBM rate of the step kernels, measured
  int exec_mode = hbmc::kExecAuto;
  hbmc::ExecModel model;
  // eligibility: the single-workgroup kernel for step ranges moving at most
  // fused_limit algorithmic bytes, the column kernel for calls whose rank
  // buffers total at most columns_limit bytes (working sets the caches hold)
  uint64_t fused_limit = uint64_t(64) << 20;
  uint64_t columns_limit = uint64_t(64) << 20;
  uint64_t column_bytes = 0;   // column length in bytes; 0: chosen per call
  bool xcd_split = false;
  // the flow kernel: tile length per rank buffer (bytes), workgroups per
  // compute unit, wait bound, flags (kFlowUnreachable)
  uint64_t flow_tile_bytes = uint64_t(16) << 10;
  uint32_t flow_wgs_per_cu = 8;
  uint32_t flow_wait_us = 1000000;
  uint32_t flow_flags = 0;
  uint32_t flow_batch = 1;  // tiles per ticket
  // (topology index, coll, root, count, dtype) -> plan
  std::map<std::tuple<int, int, int, uint64_t, int>, std::unique_ptr<hbmc::Plan>> plans;
  // AUTO: (coll, root, count, dtype) -> chosen topology index
  std::map<std::tuple<int, int, uint64_t, int>, int> chosen;
};

namespace hbmc {

// Build (or fetch) the host schedule of (coll, root, count, dtype); the root
// matters only for Reduce and Broadcast.  For AUTO communicators this picks
// the candidate with the least modelled time first (see choose_topology).
hbmc_status_t get_plan(hbmc_comm* c, int coll, int root, size_t count, int dtype, Plan** out);
// AUTO: index into c->topos of the candidate with the least modelled time
// steps * alpha + hbm_bytes / beta (ties: fewer steps, then lower index).
// AUTO_RULES: Flat for an AllReduce below kFlatRuleBytes per rank, else RHD
// when P is a power of two and the ring otherwise; RHD for Reduce and
// Broadcast.
constexpr uint64_t kFlatRuleBytes = uint64_t(64) << 10;
hbmc_status_t choose_topology(hbmc_comm* c, int coll, int root, size_t count, int dtype, int* index);
// Copy the plan's item table to the current device (once per plan).
hbmc_status_t upload(Plan* p);
// Non-null, element-aligned, pairwise disjoint rank buffers of count elements.
hbmc_status_t check_bufs(int P, void* const bufs[], size_t count, uint32_t e);
// Validate a call and describe the launches of its steps [first, last) (all
// of them when `whole`): a single-workgroup kernel for the whole range when
// it moves no more than the communicator's fused limit; else one column
// kernel launch when the rank buffers' total size is within the
// communicator's column limit and the range has two or more busy steps; else
// one step kernel per non-empty step.  Both one-launch forms need buffers of
// one 16-byte phase.  Uploads the plan's device tables.  No launches for
// count == 0 or P == 1.
hbmc_status_t prepare(hbmc_comm* c, int coll, int root, void* const bufs[], size_t count, int dtype,
                      int op, int first, int last, bool whole, std::vector<KernelDesc>* launches);
// Column length in elements for `column_bytes` (a multiple of 16 bytes, at
// least 16) or, for 0, for a call of `count` elements: about four columns per
// compute unit, no shorter than 1 KiB (one 16-byte vector per lane of a wave).
uint64_t column_elems(uint64_t column_bytes, uint64_t count, uint32_t e, uint32_t compute_units);
// The plan's host column table for a column length of `chunk_elems` (built
// once per length, without dependency lists).
hbmc_status_t column_table(Plan* p, int P, uint64_t chunk_elems, const ColumnTable** out);
// Upload the plan's column table to the current device (again after the
// column length changed; the old tables are retired, not freed).
hbmc_status_t upload_columns(Plan* p);
// Column length of the LDS-resident column kernel for plan p (P ranks, count
// elements of e bytes), cached in the plan: the communicator's column_bytes
// when set; otherwise, of the lengths 16 B, 32 B, ... that fit one
// workgroup's LDS, the one of least modelled time (ties: the longer).
// Sets p->lds_col (0 when none fits), p->lds_chunks and p->lds_longest.
hbmc_status_t lds_layout(hbmc_comm* c, Plan* p, int P, uint64_t count, uint32_t e);
// Build and upload the LDS-resident kernel's tables for p->lds_col (count
// elements of e bytes): column g's chunks in order at [col_off[g],
// col_off[g+1]), each with its byte range relative to the column, step,
// shape, rank numbers and destination mask; and for launches of all steps
// the number of chunks before the column's trailing copies and the store
// records those copies compose into (see DevColStore).
hbmc_status_t upload_lds_tables(Plan* p, int P, uint64_t count, uint32_t e);
// The same tables built on the host only (p->lh), once per column length.
hbmc_status_t lds_host_tables(Plan* p, int P, uint64_t count, uint32_t e);
// The flow kernel's host table of steps [first, last) of plan p for the
// communicator's tile length (count elements of e bytes), built once per
// range and length; *out receives the range's state (ok: the steps fit).
hbmc_status_t flow_host(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, FlowSet** out);
// Upload a range's table to the plan's device with zeroed counters (again
// after the tile length changed; the old tables are retired, not freed).
hbmc_status_t upload_flow(Plan* p, FlowSet* f);
// The number of flow waits that gave up in all of the communicator's plans,
// then cleared (synchronous; 0 when no flow launch ran).
hbmc_status_t flow_timeouts(hbmc_comm* c, uint32_t* count);
// Bytes a launch of steps [first, last) in form `mode` moves between the
// compute units and memory (see hbmc_exec_bytes).
hbmc_status_t exec_bytes(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, int mode,
                         uint64_t* bytes);
// Launch form of steps [first, last) of plan `p` (count elements of e bytes,
// buffers of one 16-byte phase when `aligned`): the communicator's mode when
// not AUTO and the form is eligible; for AUTO the eligible form of least
// modelled time, where, for B algorithmic bytes in S non-empty steps,
//   steps:   sum over steps of max(launch_us, step_us + B_s / hbm)
//   fused:   fused_us + S * fused_step_us + B / fused_gbps
//   columns: col_us + H * col_hop_us + B / col_gbps, H the chunks of the
//            longest column, scaled to the range's share of the busy steps
// (ties: steps, then fused).  Fused needs <= 256 items per step and B within
// the fused limit; columns need two or more busy steps and P * count * e
// within the column limit; both need `aligned`.  Steps otherwise.
hbmc_status_t choose_exec(hbmc_comm* c, Plan* p, int first, int last, uint64_t count, uint32_t e, bool aligned,
                          int* mode);
// Enqueue one described launch on `stream`.
hbmc_status_t launch(KernelDesc& k, void* stream);
// Validate and enqueue steps [first, last) of a collective (all of them when
// `whole`) on `stream`, with the launches prepare() describes.
hbmc_status_t run(hbmc_comm* c, int coll, int root, void* const bufs[], size_t count, int dtype,
                  int op, int first, int last, bool whole, void* stream);
// Out-of-place: LocalCopy of send into recv where they differ (one copy
// launch per 32 ranks), then the collective in place on recv.
hbmc_status_t run_out_of_place(hbmc_comm* c, int coll, int root, const void* const send[],
                               void* const recv[], size_t count, int dtype, int op, void* stream);

// AllReduce with the step kernels' item tables in the library's fixed
// device array instead of allocated memory (see hbmc_allreduce_noalloc).
hbmc_status_t allreduce_noalloc(hbmc_comm* c, void* const bufs[], size_t count, int dtype, int op, void* stream);

// Runs an entry point's body so that no C++ exception crosses the C ABI.  The
// host code throws only when allocating its tables fails (std::bad_alloc,
// std::length_error), which is reported as HBMC_ERR_NOMEM; a plan is cached
// only once complete, so a failed call leaves the communicator usable.
template <typename F>
hbmc_status_t no_throw(F&& body) noexcept {
  try {
    return body();
  } catch (...) {
    return HBMC_ERR_NOMEM;
  }
}

}  // namespace hbmc
