// The register form of a whole call (see regs.hpp).  grid.y indexes the
// regions of elements that share one expression; a lane of region g takes
// one 16-byte position of the vector, loads every operand there into
// registers at once, evaluates the schedule's expression in its grouping --
// a left fold over a rank sequence, a complete pairwise tree over single
// ranks and merged pairs, a copy of one rank, the prefixes of a fold, or the
// nodes of a tree -- and stores every rank the schedule writes there.  A region's
// operand addresses travel in its record in the kernel arguments, so a
// workgroup waits on one round of scalar loads (its record) and one round of
// data loads: no table in device memory, no LDS, no barrier.  The region's
// elements outside its whole positions (where its edges cut a position, and
// the head / tail of the vector) are taken one by one by the lanes of its
// first workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>

#include "elemops.hpp"
#include "launch.hpp"
#include "regs.hpp"

namespace hbmc {
namespace {

using namespace dev;

// Kernel-side variants of the tree form, whose call records carry 16
// addresses as the fold's do (fewer scalar registers and record loads): trees
// whose leaves are all single ranks (P a power of two; no leaf tests for a
// pair), and trees of at most 8 leaves with pairs (the pair's second address
// at ptr[8 + v]).
constexpr int kRegTreeSingles = 4;
constexpr int kRegTreeSmall = 5;

// Leaves a form's kernel handles and where a leaf's pair address sits (0:
// no pairs).
template <int FORM>
struct RegShape {
  static constexpr int leaves = FORM == kRegTreeSmall ? 8 : kRegMaxLeaves;
  static constexpr int pair = FORM == kRegTree ? kRegMaxLeaves : (FORM == kRegTreeSmall ? 8 : 0);
  static constexpr int ptrs = FORM == kRegTree ? 2 * kRegMaxLeaves : kRegMaxLeaves;
};

// The expression of a region over values load(i) of its operands
// (addresses ptr[i]), combined by op.
template <int FORM, typename V, typename Load, typename Op>
__device__ __forceinline__ V eval(uint32_t n, const unsigned char* const* ptr, Load load, Op op) {
  V x[kRegMaxLeaves];
  if constexpr (FORM == kRegTreeSingles) {
#pragma unroll
    for (uint32_t v = 0; v < kRegMaxLeaves; ++v)
      if (v < n) x[v] = load(ptr[v]);
#pragma unroll
    for (uint32_t w = 1; w < kRegMaxLeaves; w *= 2)
#pragma unroll
      for (uint32_t v = 0; v + w < kRegMaxLeaves; v += 2 * w)
        if (v + w < n) x[v] = op(x[v], x[v + w]);
    return x[0];
  } else if constexpr (FORM == kRegFold) {
#pragma unroll
    for (uint32_t i = 0; i < kRegMaxLeaves; ++i)
      if (i < n) x[i] = load(ptr[i]);
    V acc = op(x[0], x[1]);
#pragma unroll
    for (uint32_t i = 2; i < kRegMaxLeaves; ++i)
      if (i < n) acc = op(acc, x[i]);
    return acc;
  } else {
    // leaves that may be pairs (x_a op x_b), then pairs (0,1), (2,3), ...,
    // then (0,2), (4,6), ...
    constexpr uint32_t NL = RegShape<FORM>::leaves, PO = RegShape<FORM>::pair;
    V y[NL];
#pragma unroll
    for (uint32_t v = 0; v < NL; ++v) {
      if (v < n) {
        x[v] = load(ptr[v]);
        if (ptr[PO + v]) y[v] = load(ptr[PO + v]);
      }
    }
#pragma unroll
    for (uint32_t v = 0; v < NL; ++v)
      if (v < n && ptr[PO + v]) x[v] = op(x[v], y[v]);
#pragma unroll
    for (uint32_t w = 1; w < NL; w *= 2)
#pragma unroll
      for (uint32_t v = 0; v + w < NL; v += 2 * w)
        if (v + w < n) x[v] = op(x[v], x[v + w]);
    return x[0];
  }
}

// Store v at byte offset off of every operand.
template <int FORM, typename Store>
__device__ __forceinline__ void store_all(uint32_t n, unsigned char* const* ptr, Store store) {
  constexpr uint32_t NL = RegShape<FORM>::leaves, PO = RegShape<FORM>::pair;
#pragma unroll
  for (uint32_t v = 0; v < NL; ++v) {
    if (v < n) {
      store(ptr[v]);
      if constexpr (PO > 0)
        if (ptr[PO + v]) store(ptr[PO + v]);
    }
  }
}

// One position (a 16-byte vector, or one element) of a region: the
// operands loaded, combined and stored as the form says (lvl: the node
// form's store levels).
template <int FORM, typename V, typename Load, typename Op, typename Store>
__device__ __forceinline__ void position(uint32_t n, unsigned char* const* ptr, const uint8_t* lvl, Load load,
                                         Op op, Store store) {
  if constexpr (FORM == kRegNodes) {
    // the tree level by level; after level l, every leaf whose rank holds
    // the level-l node above it stores that node
    // (fixed trip counts throughout, so that once unrolled every index is a
    // constant and x stays in registers)
    V x[kRegMaxLeaves];
#pragma unroll
    for (uint32_t v = 0; v < kRegMaxLeaves; ++v)
      if (v < n) x[v] = load(ptr[v]);
    constexpr uint32_t kLevels = __builtin_ctz(kRegMaxLeaves);
    static_assert((1u << kLevels) == kRegMaxLeaves, "leaves: a power of two");
#pragma unroll
    for (uint32_t l = 1; l <= kLevels; ++l) {
      const uint32_t w = 1u << (l - 1);
#pragma unroll
      for (uint32_t v = 0; v < kRegMaxLeaves; ++v)
        if ((v & (2 * w - 1)) == 0 && v + w < n) x[v] = op(x[v], x[v + w]);
#pragma unroll
      for (uint32_t v = 0; v < kRegMaxLeaves; ++v)
        if (v < n && lvl[v] == l) store(ptr[v], x[v & ~(2 * w - 1)]);
    }
  } else if constexpr (FORM == kRegCopy) {
    const V v = load(ptr[0]);
#pragma unroll
    for (uint32_t i = 1; i < kRegMaxLeaves; ++i)
      if (i < n) store(ptr[i], v);
  } else if constexpr (FORM == kRegPrefix) {
    V x[kRegMaxLeaves];
#pragma unroll
    for (uint32_t i = 0; i < kRegMaxLeaves; ++i)
      if (i < n) x[i] = load(ptr[i]);
    V acc = x[0];
#pragma unroll
    for (uint32_t i = 1; i < kRegMaxLeaves; ++i) {
      if (i < n) {
        acc = op(acc, x[i]);
        store(ptr[i], acc);
      }
    }
  } else {
    const V v = eval<FORM, V>(n, ptr, load, op);
    store_all<FORM>(n, ptr, [&](unsigned char* p) { store(p, v); });
  }
}

template <int DT, int OP, int FORM, typename Call>
__global__ void __launch_bounds__(kRegThreads)
plan_regs(Call c) {
  constexpr uint32_t E = Width<DT>::bytes;
  constexpr uint32_t EPV = 16 / E;
  constexpr int NP = RegShape<FORM>::ptrs;
  // the call's header and the region's record read whole before any branch
  // on them, so that their scalar loads go out together
  const uint32_t n = c.n, phase = c.phase;
  const uint64_t count = c.count;
  const auto& R0 = c.r[blockIdx.y];
  struct {
    uint32_t vec_lo, vec_hi, el_lo[2], el_hi[2];
    uint8_t lvl[kRegMaxLeaves];
    unsigned char* ptr[NP];
  } R;
  R.vec_lo = R0.vec_lo;
  R.vec_hi = R0.vec_hi;
  if constexpr (FORM == kRegNodes) {
#pragma unroll
    for (int i = 0; i < kRegMaxLeaves; ++i) R.lvl[i] = R0.lvl[i];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    R.el_lo[i] = R0.el_lo[i];
    R.el_hi[i] = R0.el_hi[i];
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) R.ptr[i] = R0.ptr[i];
  uint64_t head = ((16u - (phase & 15u)) & 15u) / E;
  if (head > count) head = count;
  const uint64_t k = uint64_t(R.vec_lo) + uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k < R.vec_hi) {
    const uint64_t off = (head + k * EPV) * E;
    position<FORM, u32x4>(
        n, R.ptr, R.lvl, [&](const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p + off); },
        [](u32x4 a, u32x4 b) { return op_vec<DT, OP>(a, b); },
        [&](unsigned char* p, u32x4 v) { store_vec(reinterpret_cast<u32x4*>(p + off), v); });
  }
  if (blockIdx.x == 0) {
    // the region's head and tail elements; the body written out twice (not
    // a loop over the two parts: int8's is too large to unroll, and an index
    // into R would move all of R, operand addresses included, to scratch)
    auto part = [&](uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
      const uint64_t e = uint64_t(lo) + threadIdx.x;
      if (e < hi) {
        const uint64_t off = e * E;
        position<FORM, uint32_t>(
            n, R.ptr, R.lvl, [&](const unsigned char* p) { return load_elem<E>(p + off); },
            [](uint32_t a, uint32_t b) { return op_word<DT, OP>(a, b); },
            [&](unsigned char* p, uint32_t v) { store_elem<E>(p + off, v); });
      }
    };
    part(R.el_lo[0], R.el_hi[0]);
    part(R.el_lo[1], R.el_hi[1]);
  }
}

template <int DT, int OP>
const void* regs_fn(uint32_t form) {
  switch (form) {
    case kRegTree: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegTree, RegTreeCall>);
    case kRegTreeSingles: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegTreeSingles, RegFoldCall>);
    case kRegTreeSmall: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegTreeSmall, RegFoldCall>);
    case kRegNodes: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegNodes, RegFoldCall>);
    case kRegCopy: return reinterpret_cast<const void*>(plan_regs<DT, kSum, kRegCopy, RegFoldCall>);
    case kRegPrefix: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegPrefix, RegFoldCall>);
    default: return reinterpret_cast<const void*>(plan_regs<DT, OP, kRegFold, RegFoldCall>);
  }
}

template <int DT>
const void* regs_op(int op, uint32_t form) {
  switch (op) {
    case kSum: return regs_fn<DT, kSum>(form);
    case kProd: return regs_fn<DT, kProd>(form);
    case kMax: return regs_fn<DT, kMax>(form);
    default: return regs_fn<DT, kMin>(form);
  }
}

// Fill a call's records from the derived regions; returns the largest
// number of whole positions in one region.
template <typename Call>
uint64_t fill(Call* c, const RankPtrs& ptrs, const RegPlan& rp, uint64_t count, uint32_t phase, uint32_t E,
              uint32_t pair) {
  std::memset(c, 0, sizeof(*c));
  c->n = rp.n;
  c->phase = phase;
  c->count = count;
  const uint64_t EPV = 16 / E;
  uint64_t head = ((16u - (phase & 15u)) & 15u) / E;
  if (head > count) head = count;
  const uint64_t nvec = (count - head) / EPV;
  uint64_t most = 0, start = 0;
  for (size_t g = 0; g < rp.regions.size(); ++g) {
    const RegRegion& q = rp.regions[g];
    auto& r = c->r[g];
    const uint64_t end = q.end;
    // whole positions inside [start, end)
    uint64_t lo = start <= head ? 0 : (start - head + EPV - 1) / EPV;
    uint64_t hi = end <= head ? 0 : (end - head) / EPV;
    lo = std::min(lo, nvec);
    hi = std::min(hi, nvec);
    if (hi < lo) hi = lo;
    r.vec_lo = static_cast<uint32_t>(lo);
    r.vec_hi = static_cast<uint32_t>(hi);
    if (hi > lo) {
      r.el_lo[0] = static_cast<uint32_t>(start);
      r.el_hi[0] = static_cast<uint32_t>(head + lo * EPV);
      r.el_lo[1] = static_cast<uint32_t>(head + hi * EPV);
      r.el_hi[1] = static_cast<uint32_t>(end);
    } else {
      r.el_lo[0] = static_cast<uint32_t>(start);
      r.el_hi[0] = static_cast<uint32_t>(end);
      r.el_lo[1] = r.el_hi[1] = 0;
    }
    for (uint32_t v = 0; v < rp.n; ++v) {
      r.ptr[v] = ptrs.p[q.a[v]];
      r.lvl[v] = q.lvl[v] == 0xff ? 0 : q.lvl[v];
      if (pair > 0 && q.b[v] != 0xff) r.ptr[pair + v] = ptrs.p[q.b[v]];
    }
    most = std::max<uint64_t>(most, hi - lo);
    start = end;
  }
  return most;
}

}  // namespace

void describe_regs(int dtype, int op, const RankPtrs& ptrs, int P, const RegPlan& rp, uint64_t count,
                   uint32_t phase, KernelDesc* k) {
  (void)P;
  const uint32_t E = dtype == kF32 || dtype == kI32 ? 4u : (dtype == kI8 ? 1u : 2u);
  uint64_t most = 0;
  uint32_t form = rp.form;
  if (form == kRegTree) {
    bool pairs = false;
    for (const RegRegion& q : rp.regions)
      for (uint32_t v = 0; v < rp.n; ++v) pairs = pairs || q.b[v] != 0xff;
    if (!pairs) form = kRegTreeSingles;
    else if (rp.n <= uint32_t(RegShape<kRegTreeSmall>::leaves)) form = kRegTreeSmall;
  }
  if (form == kRegTree) most = fill(new (k->args) RegTreeCall, ptrs, rp, count, phase, E, RegShape<kRegTree>::pair);
  else
    most = fill(new (k->args) RegFoldCall, ptrs, rp, count, phase, E,
                form == kRegTreeSmall ? uint32_t(RegShape<kRegTreeSmall>::pair) : 0u);
  // at least one lane per element a region takes one by one (fewer than 16
  // at each end of a region); one-wave workgroups, which measured as fast or
  // faster than 128 or 256 lanes everywhere (MI355X, graphs of ten calls:
  // 8-rank RHD bf16 at 4-64 KiB per rank 2.91-3.00 against 3.11-3.28 us,
  // 16-rank RHD fp16 at 16 KiB 3.06 against 3.52 us, 16-rank ring fp16 at
  // 4 MiB 21.9 against 23.5 us; a capped grid whose lanes walk several
  // positions was slower still)
  const uint64_t lanes = std::max<uint64_t>(most, 16);
  const uint32_t block = 64u;
  k->kind = KernelDesc::kRegs;
  k->grid = dim3(static_cast<uint32_t>((lanes + block - 1) / block), static_cast<uint32_t>(rp.regions.size()));
  k->block = dim3(block);
  k->shared_bytes = 0;
  switch (dtype) {
    case kF32: k->func = regs_op<kF32>(op, form); break;
    case kF16: k->func = regs_op<kF16>(op, form); break;
    case kBF16: k->func = regs_op<kBF16>(op, form); break;
    case kI32: k->func = regs_op<kI32>(op, form); break;
    default: k->func = regs_op<kI8>(op, form); break;
  }
  k->bind();
}

}  // namespace hbmc
