// The register form of a whole AllReduce (host side).
//
// Every step combines operands at equal element offsets, so the value an
// element ends with on a rank is one expression over the P inputs at that
// offset, fixed by the schedule: which ranks' values each step combines, and
// in which grouping.  The host derives that expression by replaying the
// schedule symbolically over the intervals of elements that the same items
// cover.  Where every rank ends with one and the same expression, and that
// expression is
//   - a left fold  ((x_s0 op x_s1) op x_s2) op ... over all P ranks (the
//     ring, with the sequence rotated per segment; Flat), or
//   - a complete binary tree of depth k whose 2^k leaves are single ranks
//     or pairs (x_a op x_b) (recursive halving-doubling, its merged pairs
//     included),
// one kernel evaluates it in registers: every rank's value loaded once, the
// expression's operations in its grouping, the result stored to every rank.
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
enum RegForm : uint32_t { kRegFold = 0, kRegTree = 1 };

// Elements [previous region's end, end) take: for kRegFold the left fold over
// a[0..n); for kRegTree the tree over leaves v < n = 2^k, leaf v being rank
// a[v], or a[v] op b[v] when b[v] != 0xff.
struct RegRegion {
  uint64_t end;
  uint8_t a[kRegMaxLeaves];
  uint8_t b[kRegMaxLeaves];
};
static_assert(sizeof(RegRegion) == 40, "register-form region");

struct RegPlan {
  bool ok = false;  // the whole AllReduce can run in the register form
  RegForm form = kRegFold;
  uint32_t n = 0;   // fold length or tree leaves (one value for all regions)
  std::vector<RegRegion> regions;
};

// Derive the register form of an AllReduce schedule of P ranks over `count`
// elements; out->ok is false where the form does not apply.
void derive_regs(const Schedule& s, int P, uint64_t count, RegPlan* out);

}  // namespace hbmc
