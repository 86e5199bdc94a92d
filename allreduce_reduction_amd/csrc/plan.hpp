// Schedule builder: per-step work-item tables for ring, recursive
// halving-doubling and the two-level pipeline (host only, no HIP).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace hbmc {

constexpr int kMaxRanks = 64;

enum Mode : int32_t { kCopy = 0, kFold = 1, kRecvFold = 2 };
enum Algo : int32_t { kRing = 0, kRhd = 1, kPipeline = 2, kFlat = 4, kTree = 5, kHier = 6 };
enum Coll : int32_t { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2, kReduce = 3, kBroadcast = 4 };

// One unit of work: every destination's range [begin, begin+count) receives
// the combination (per Mode) of the sources' same range.
struct Item {
  uint64_t begin = 0, count = 0;
  int32_t nsrc = 0, ndst = 0;
  uint8_t rank[2 * kMaxRanks] = {};  // sources then destinations
};

struct Step {
  Mode mode = kCopy;
  int32_t nsrc = 0, ndst = 0;  // shared by every item of the step; 0 when items differ
  std::vector<Item> items;     // items with count == 0 are dropped
  uint64_t hbm_bytes = 0;      // (nsrc + ndst) * count * esize summed over items
  uint64_t max_count = 0;
};

struct Topology {
  int P = 1;
  Algo algo = kRing;
  int S = 1, M = 1;          // pipeline / hierarchical servers x ranks per server
  int K = 2;                 // tree arity
  uint64_t loop_bytes = 0;   // pipeline slice; 0 -> 32 MiB
};

struct Schedule {
  std::vector<Step> steps;
  uint64_t hbm_bytes = 0;
  uint64_t max_recv_bytes = 0;
};

enum BuildStatus { kBuilt = 0, kBadArg = 1, kUnsupported = 2 };

// Build the schedule of `coll` over `count` elements of `esize` bytes
// (`root`: the root rank of Reduce / Broadcast, ignored otherwise).
// Also verifies that no two items of a step touch overlapping ranges of one
// rank where either writes (so a step's items may run concurrently in place);
// a violation is reported as kBadArg.  Reduce and Broadcast exist for RHD only
// (kUnsupported otherwise).
BuildStatus build_schedule(const Topology& topo, Coll coll, uint64_t count, uint32_t esize, int root,
                           Schedule* out);

}  // namespace hbmc
