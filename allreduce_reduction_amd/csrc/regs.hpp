// The register form of a whole collective (host side).
//
// Every step combines operands at equal element offsets, so the value an
// element ends with on a rank is one expression over the P inputs at that
// offset, fixed by the schedule: which ranks' values each step combines, and
// in which grouping.  The host derives that expression by replaying the
// schedule symbolically over the intervals of elements that the same items
// cover.  Where, in every interval,
//   - every rank ends with one and the same expression, and it is a left
//     fold ((x_s0 op x_s1) op x_s2) op ... over all P ranks (the ring's
//     AllReduce, with the sequence rotated per segment; Flat), or a complete
//     binary tree of depth k whose 2^k leaves are single ranks or pairs
//     (x_a op x_b) (recursive halving-doubling, its merged pairs included),
//   - or every rank ends with one rank's input (an all-gather, a
//     broadcast: a copy),
//   - or the ranks end with the prefixes of one left fold over all P ranks,
//     each rank holding the prefix that ends with its own input (the ring's
//     reduce-scatter),
//   - or, for a complete pairwise tree over all P ranks (P a power of two),
//     every rank ends with its own input or with a node of that tree above
//     its own leaf (RHD's reduce-scatter and Reduce),
// one kernel evaluates it in registers: every operand loaded once, the
// operations in the schedule's grouping, and every rank's result stored.
// The element ops are commutative bit for bit (IEEE sum / product, wrapping
// integers, max / min with a canonical NaN), so only the grouping fixes the
// bits, and the kernel keeps it.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace hbmc {

constexpr int kRegMaxLeaves = 16;       // fold length / tree leaves
constexpr int kRegMaxFoldRegions = 16;  // intervals of distinct parameters, fold form
constexpr int kRegMaxTreeRegions = 8;   // and tree form (each region's addresses travel in
                                        // the kernel arguments)
enum RegForm : uint32_t { kRegFold = 0, kRegTree = 1, kRegCopy = 2, kRegPrefix = 3, kRegNodes = 6 };

// Elements [previous region's end, end) take: for kRegFold the left fold over
// a[0..n), stored to every rank; for kRegTree the tree over leaves v < n =
// 2^k, leaf v being rank a[v], or a[v] op b[v] when b[v] != 0xff, stored to
// every rank; for kRegCopy rank a[0]'s value, stored to ranks a[1..n); for
// kRegPrefix the left fold over a[0..n), rank a[i] (i >= 1) receiving the
// fold over a[0..i]; for kRegNodes the tree over leaves a[0..n) (n = 2^k),
// rank a[v] receiving the node of level lvl[v] whose leaves include v (the
// nodes of level l pair those of level l - 1: (0,1), (2,3), ...), or keeping
// its input when lvl[v] is 0.
struct RegRegion {
  uint64_t end;
  uint8_t a[kRegMaxLeaves];
  uint8_t b[kRegMaxLeaves];
  uint8_t lvl[kRegMaxLeaves];
};
static_assert(sizeof(RegRegion) == 56, "register-form region");

struct RegPlan {
  bool ok = false;  // the whole collective can run in the register form
  RegForm form = kRegFold;
  uint32_t n = 0;   // operands (fold length, tree leaves; one value for all regions)
  uint32_t loads = 0, stores = 0;  // per element position (kRegNodes: stores is the most of any region)
  std::vector<RegRegion> regions;
};

// Derive the register form of a whole schedule of P ranks over `count`
// elements; out->ok is false where the form does not apply.
void derive_regs(const Schedule& s, int P, uint64_t count, RegPlan* out);

}  // namespace hbmc
