// gfx950 step kernels.  One launch executes one schedule step for all ranks:
// grid.x tiles an item's elements and grid.y indexes the step's work items;
// a step of more items than grid.y may hold (the device reports 65536) also
// spreads them over grid.z, item = z * grid.y + y, and the workgroups past
// the last item return at once.  A
// workgroup takes its item either from the plan's device item table
// (step_vec: the item's rank numbers index the call's pointer table) or, for
// steps of a few items, from the kernel arguments with its operand addresses
// already resolved by the host (step_arg).
//
// The reduce is the pages' reduce_op(recv, local) over a received block and
// the local block ([RING-RHD] "Ring AllReduce带宽最优的环形流水线" listing;
// the vector unit applies sum / product / maximum, section "Ascend950的AIVAICPU
// 通信引擎与图模式"); a copy is the all-gather's segment transfer.  On one GPU
// both become HBM streams: a step reads every source block once and writes
// every destination block once.
//
// Data path: every operand of an item sits at the same element offset, and
// when all rank buffers share one 16-byte phase the item's body is moved as
// 16-byte vectors (global_load_dwordx4 with the nontemporal hint;
// global_store_dwordx4, with that hint only in steps that write more than the
// memory-side cache holds): one wave per workgroup and one vector per lane per
// operand, i.e. 1 KiB tiles of every operand per workgroup, which measured
// fastest for streams far larger than the caches (copy steps that write at
// most 32 MiB and whose items reach 1 MiB take four vectors per lane, see
// arg_kernel); the few head / tail elements are done one by one.  Buffers with different phases take an
// element-wise kernel.
//
// Element ops: fp16 / bf16 lanes are widened to fp32, combined and rounded
// back to nearest even per operation; integers wrap; max / min order -0 below
// +0 and give the canonical quiet NaN when either operand is NaN.
#include <hip/hip_runtime.h>

#include <new>

#include "elemops.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace {

using namespace dev;

constexpr int kThreads = 64;        // vector kernel: one wave per workgroup
constexpr uint64_t kTileVecs = kThreads;  // one 16-byte vector per lane per operand
constexpr int kWideVecs = 4;  // vectors per lane of the small copy steps (arg_kernel)
constexpr uint64_t kWideMinItemBytes = uint64_t(1) << 20;  // ... whose items reach this size
constexpr int kElemThreads = 256;   // element-wise kernel
// Items per grid row when a step's items do not fit grid.y alone (below the
// device's reported grid.y and grid.z limits of 65536).
constexpr uint32_t kGridRows = 32768;
// Copy steps reading at most this many bytes take plain loads (see arg_kernel).
constexpr uint64_t kPlainLoadCopyBytes = uint64_t(32) << 20;
// Largest item a step kernel takes: grid.x times the workgroup size must stay
// below 2^32 work-items, so at most 2^26 one-wave tiles of 1 KiB.
constexpr uint64_t kMaxItemBytes = (uint64_t(1) << 26) * kTileVecs * 16;

// Resident workgroups per compute unit for steps of many items whose
// workgroups each keep many HBM streams open (the pipeline's steps: 512
// items of 1 MiB), capped by reserving LDS the kernel never touches
// (160 KiB per compute unit / cap).  Fewer resident workgroups keep the
// addresses in flight closer together in each stream.  Measured on MI355X
// (4 x 8 bf16 pipeline, 512 MiB per rank, same session; caps swept 6-32):
// - folds with all 8 or 9 sources' loads issued at once (the compile-time
//   shapes): 10 per CU, 6.2-6.3 TB/s against 6.0-6.1 at 16 and 5.8 at 24;
//   8 and 9 matched 10, 6 lost 7%;
// - copies to several destinations: 12 per CU; the closing one-to-seven
//   copy 6.1 TB/s against 5.7 at 20 and 5.8 at 10, the one-to-eight steps
//   5.8 TB/s at 10-20 and 5.45 at 28; the whole AllReduce 6514-6523 us
//   against 6652-6719 us at 16 / 20;
// - left uncapped, where a cap lost: folds that loop over a run-time source
//   count (one load at a time; 16 sources: 34% slower capped), Flat's
//   single-item fold and copy (the whole 8-rank AllReduce 2% slower with the
//   fold capped, the copy 5-9% slower), and the ring's 2-source reduce and
//   1-to-1 copy (every cap slower).
constexpr uint32_t kLdsPerCu = 160u * 1024u;
constexpr uint32_t kFoldWgPerCu = 10;
constexpr uint32_t kFanWgPerCu = 12;
constexpr int kCapMinItems = 64;  // above any tree level (at most 32 parents)

// ------------------------------------------------------------- kernels

// Vector kernels.  Workgroup -> (item, tile): grid.y is the item and grid.x the tile, and the
// hardware deals workgroups to the 8 XCDs round-robin by linear id.  With
// `xcd_split` each XCD instead walks one contiguous range of the step's tiles.
__device__ __forceinline__ void xcd_tile(uint32_t* item, uint32_t* tile) {
  uint32_t lin = blockIdx.y * gridDim.x + blockIdx.x;
  const uint32_t per = (gridDim.x * gridDim.y) / 8;
  lin = (lin % 8) * per + lin / 8;
  *item = lin / gridDim.x;
  *tile = lin % gridDim.x;
}

// One workgroup's tile of one item.  `bufs(i)` is the item's i-th operand
// (sources, then destinations) and element j of the item sits at byte
// (begin + j) * E from it; `phase` is the 16-byte phase the operand addresses
// share.  NS / ND > 0 fix the item shape at compile time (all loads of a tile
// issued before any combine); 0 takes ns / nd.
// NT: stores with the nontemporal hint (a compile-time choice: the compiler
// merges the two stores of a run-time branch into one plain store).  PL: the
// loads without the nontemporal hint.  VPL: 16-byte vectors per lane per
// operand, the tile being kThreads * VPL vectors.
// A 16-byte load: with the nontemporal hint, or plain (PL).
template <bool PL>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (PL) return *p;
  else return load_vec(p);
}

template <int DT, int OP, int MODE, int NS, int ND, bool NT, bool PL, int VPL, typename B>
__device__ __forceinline__ void vec_item(const B& bufs, uint64_t begin, uint64_t count, uint32_t phase,
                                         uint32_t tile, int ns, int nd) {
  constexpr uint32_t E = Width<DT>::bytes;
  // A fixed-shape item's buffer addresses, all taken before the first data
  // load: the scalar loads behind them are then issued together, and the
  // workgroup waits on one chain (kernel arguments, item record, addresses)
  // rather than on one address after another.
  constexpr int NB = NS > 0 && ND > 0 ? NS + ND : 1;
  unsigned char* buf[NB];
  if constexpr (NS > 0 && ND > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) buf[b] = bufs(b);
  }

  uint64_t head = ((16u - ((phase + begin * E) & 15u)) & 15u) / E;
  if (head > count) head = count;
  const uint64_t nvec = (count - head) * E / 16;
  const uint64_t body_end = head + nvec * (16 / E);

  constexpr uint64_t TV = kTileVecs * VPL;
  const uint64_t v0 = uint64_t(tile) * TV + threadIdx.x;
  if (uint64_t(tile) * TV < nvec) {
    const uint64_t base = (begin + head) * E;
    u32x4 acc[VPL];
    if constexpr (NS > 0) {
      // all loads of the tile first, then the combines in schedule order
      u32x4 x[NS][VPL];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const unsigned char* src;
        if constexpr (ND > 0) src = buf[s];
        else src = bufs(s);
        const u32x4* p = reinterpret_cast<const u32x4*>(src + base);
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kThreads;
          if (v < nvec) x[s][u] = ld<PL>(p + v);
        }
      }
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        if constexpr (MODE == kCopy || NS == 1) {
          acc[u] = x[0][u];
        } else if constexpr (MODE == kFold) {
          acc[u] = x[0][u];
#pragma unroll
          for (int s = 1; s < NS; ++s) acc[u] = op_vec<DT, OP>(acc[u], x[s][u]);
        } else {
          acc[u] = x[1][u];
#pragma unroll
          for (int s = 2; s < NS; ++s) acc[u] = op_vec<DT, OP>(acc[u], x[s][u]);
          acc[u] = op_vec<DT, OP>(x[0][u], acc[u]);
        }
      }
    } else {
      const int first = MODE == kRecvFold ? 1 : 0;
      {
        const u32x4* p = reinterpret_cast<const u32x4*>(bufs(first) + base);
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kThreads;
          if (v < nvec) acc[u] = ld<PL>(p + v);
        }
      }
      if constexpr (MODE != kCopy) {
        for (int s = first + 1; s < ns; ++s) {
          const u32x4* p = reinterpret_cast<const u32x4*>(bufs(s) + base);
#pragma unroll
          for (int u = 0; u < VPL; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(acc[u], ld<PL>(p + v));
          }
        }
        if constexpr (MODE == kRecvFold) {
          const u32x4* p = reinterpret_cast<const u32x4*>(bufs(0) + base);
#pragma unroll
          for (int u = 0; u < VPL; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(ld<PL>(p + v), acc[u]);
          }
        }
      }
    }
#pragma unroll
    for (int d = 0; d < (ND > 0 ? ND : nd); ++d) {
      unsigned char* dst;
      if constexpr (NS > 0 && ND > 0) dst = buf[NS + d];
      else dst = bufs(ns + d);
      u32x4* q = reinterpret_cast<u32x4*>(dst + base);
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const uint64_t v = v0 + uint64_t(u) * kThreads;
        if (v < nvec) {
          if constexpr (NT) store_vec_nt(q + v, acc[u]);
          else store_vec(q + v, acc[u]);
        }
      }
    }
  }

  // head and tail elements (fewer than 16 bytes each), by the item's first tile
  if (tile == 0) {
    const uint64_t t = threadIdx.x;
    if (t < head) do_elem<DT, OP, MODE>(bufs, ns, nd, begin + t);
    if (t >= 32 && t - 32 < count - body_end) do_elem<DT, OP, MODE>(bufs, ns, nd, begin + body_end + (t - 32));
  }
}

// Vector kernel, items from the device table.
template <int DT, int OP, int MODE, int NS, int ND, bool NT>
__global__ void __launch_bounds__(kThreads)
step_vec(const DevItem* __restrict__ items, uint32_t phase, uint32_t flags, RankPtrs ptrs, uint32_t nitems) {
  uint32_t item = blockIdx.y, tile = blockIdx.x;
  if (gridDim.z > 1) {
    item += blockIdx.z * gridDim.y;
    if (item >= nitems) return;
  } else if (flags & kFlagXcdSplit) {
    xcd_tile(&item, &tile);
  }
  const DevItem* it = items + item;
  const int ns = NS > 0 ? NS : static_cast<int>(it->nsrc);
  const int nd = ND > 0 ? ND : static_cast<int>(it->ndst);
  vec_item<DT, OP, MODE, NS, ND, NT, false, 1>(ItemBufs{ptrs, it}, it->begin, it->count, phase, tile, ns, nd);
}

// Vector kernel, items resolved into the kernel arguments (compile-time
// shapes, plain stores): the operand addresses already point at the item's
// first element, whose 16-byte phase they carry.  VPL vectors per lane.
template <int DT, int OP, int MODE, int NS, int ND, bool PL, int VPL>
__global__ void __launch_bounds__(kThreads)
step_arg(uint32_t flags, ArgItems<NS + ND> args) {
  uint32_t item = blockIdx.y, tile = blockIdx.x;
  if (flags & kFlagXcdSplit) xcd_tile(&item, &tile);
  const ArgItem<NS + ND>* a = &args.it[item];
  const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a->buf[0]) & 15u);
  vec_item<DT, OP, MODE, NS, ND, false, PL, VPL>(ArgBufs<NS + ND>{a}, 0, a->count, phase, tile, NS, ND);
}

// Element-wise kernel for buffers whose 16-byte phases differ.
template <int DT, int OP, int MODE>
__global__ void __launch_bounds__(kElemThreads)
step_elem(const DevItem* __restrict__ items, uint32_t, uint32_t, RankPtrs ptrs, uint32_t nitems) {
  const uint32_t item = blockIdx.z * gridDim.y + blockIdx.y;
  if (item >= nitems) return;
  const DevItem* it = items + item;
  const uint64_t begin = it->begin, count = it->count;
  const int ns = static_cast<int>(it->nsrc), nd = static_cast<int>(it->ndst);
  const uint64_t stride = uint64_t(gridDim.x) * kElemThreads;
  for (uint64_t i = uint64_t(blockIdx.x) * kElemThreads + threadIdx.x; i < count; i += stride)
    do_elem<DT, OP, MODE>(ptrs, it, ns, nd, begin + i);
}

// ------------------------------------------------------------- dispatch

template <typename F>
const void* fn(F* f) {
  return reinterpret_cast<const void*>(f);
}

// The vector kernel for one step shape.  Item shapes of the schedules get
// compile-time source counts: ring / RHD (2 sources) and the pipeline with 1,
// 2, 4 or 8 ranks per server; any other shape takes the runtime-count kernel.
template <int DT, int OP, bool NT>
const void* vector_kernel(const StepLaunch& s) {
  if (s.mode == kRecvFold) {
    switch (s.nsrc) {
      case 2: return fn(step_vec<DT, OP, kRecvFold, 2, 1, NT>);
      case 3: return fn(step_vec<DT, OP, kRecvFold, 3, 1, NT>);
      case 5: return fn(step_vec<DT, OP, kRecvFold, 5, 1, NT>);
      case 9: return fn(step_vec<DT, OP, kRecvFold, 9, 1, NT>);
      default: return fn(step_vec<DT, OP, kRecvFold, 0, 1, NT>);
    }
  }
  if (s.mode == kFold) {
    switch (s.nsrc) {
      case 2: return fn(step_vec<DT, OP, kFold, 2, 1, NT>);
      case 4: return fn(step_vec<DT, OP, kFold, 4, 1, NT>);
      case 8: return fn(step_vec<DT, OP, kFold, 8, 1, NT>);
      default: return fn(step_vec<DT, OP, kFold, 0, 1, NT>);
    }
  }
  // several destinations: the runtime-count store loop, which fetches each
  // destination's address just before its store, measured faster than
  // compile-time counts that fetch all addresses first (1 read, 8 writes:
  // 5.8 vs 5.4 TB/s; 1 read, 7 writes of 256 MiB: 389 vs 410 us)
  if (s.ndst == 1) return fn(step_vec<DT, kSum, kCopy, 1, 1, NT>);
  return fn(step_vec<DT, kSum, kCopy, 1, 0, NT>);
}

// Kernel-argument form of a compile-time shape: write the step's items,
// operands resolved, into k->args and return the kernel (plain loads for
// `plain`; for a copy, kWideVecs vectors per lane for `wide`).
template <int DT, int OP, int MODE, int NS, int ND>
const void* arg_items(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* k, bool plain, bool wide) {
  constexpr int NB = NS + ND;
  constexpr uint32_t E = Width<DT>::bytes;
  static_assert(NB <= kArgMaxBufs && sizeof(ArgItems<NB>) <= kArgBytes, "argument items");
  ArgItems<NB>* a = new (k->args) ArgItems<NB>;
  for (int i = 0; i < s.nitems; ++i) {
    const Item& it = s.host_items[i];
    for (int b = 0; b < NB; ++b) a->it[i].buf[b] = ptrs.p[it.rank[b]] + it.begin * E;
    a->it[i].count = it.count;
  }
  if constexpr (MODE == kCopy) {
    if (wide) return fn(step_arg<DT, OP, MODE, NS, ND, true, kWideVecs>);
  }
  return plain ? fn(step_arg<DT, OP, MODE, NS, ND, true, 1>) : fn(step_arg<DT, OP, MODE, NS, ND, false, 1>);
}

// The kernel-argument form for a step of at most kArgItems items of a
// compile-time shape whose stores take no hint; nullptr otherwise.  A copy
// step that reads at most kPlainLoadCopyBytes takes plain loads: at these
// sizes it reads blocks the step before has just written with plain stores.
// Measured on MI355X, one launch per step, same session, us per AllReduce
// (nontemporal loads everywhere / plain loads in copy steps of up to 32 MiB):
// 16-rank fp16 ring at 16 MiB per rank 234.9 / 224.8, RHD 202.6 / 201.3;
// 8-rank fp32 ring at 16 MiB 109.0 / 102.7, RHD 99.3 / 96.7; at 64 MiB per
// rank no change (ring 790.0 / 790.1, RHD 754.4 / 753.9).  A limit of 64 MiB
// made the 16-rank ring at 64 MiB 1% slower; plain loads in the reduce steps
// as well gained at 8 ranks and lost at 16.
// Such a copy of items of at least 1 MiB also moves kWideVecs vectors per
// lane (4 KiB tiles): its one-wave workgroups of 1 KiB are so short that the
// rate at which the hardware starts workgroups (about 3.3 per ns) bounds it.
// Measured on MI355X, one launch per step, fp16 max, same session, three
// runs each, us per AllReduce (1 KiB tiles / 4 KiB tiles): 16-rank ring at
// 16 MiB per rank 235.7-235.8 / 224.0-226.3, 8-rank fp32 ring at 16 MiB
// 101.9-102.4 / 100.8-100.9; RHD lost a little (16 ranks at 16 MiB
// 199.7-200.2 / 201.1-201.8, at 4 MiB 58.0-58.3 / 59.7-59.8), 2 KiB tiles
// lost more, and copies of smaller items lost 0.8-1.4 us per step, hence
// the item bound.  The 2-read reduce gained nothing from wider tiles, and
// at 8 items of 32 MiB 1 KiB tiles stay fastest.  `*tile_vecs` receives the
// kernel's vectors per tile.
template <int DT, int OP>
const void* arg_kernel(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* k, uint64_t* tile_vecs) {
  *tile_vecs = kTileVecs;
  if (!s.host_items || s.nitems > kArgItems || s.write_bytes > kCacheBytes || s.ndst != 1) return nullptr;
  const bool pl = s.mode == kCopy && s.write_bytes <= kPlainLoadCopyBytes;  // a copy reads what it writes
  const bool wide = pl && s.max_count * Width<DT>::bytes >= kWideMinItemBytes;
  if (s.mode == kRecvFold) {
    switch (s.nsrc) {
      case 2: return arg_items<DT, OP, kRecvFold, 2, 1>(s, ptrs, k, pl, false);
      case 3: return arg_items<DT, OP, kRecvFold, 3, 1>(s, ptrs, k, pl, false);
      case 5: return arg_items<DT, OP, kRecvFold, 5, 1>(s, ptrs, k, pl, false);
      case 9: return arg_items<DT, OP, kRecvFold, 9, 1>(s, ptrs, k, pl, false);
      default: return nullptr;
    }
  }
  if (s.mode == kFold) {
    switch (s.nsrc) {
      case 2: return arg_items<DT, OP, kFold, 2, 1>(s, ptrs, k, pl, false);
      case 4: return arg_items<DT, OP, kFold, 4, 1>(s, ptrs, k, pl, false);
      case 8: return arg_items<DT, OP, kFold, 8, 1>(s, ptrs, k, pl, false);
      default: return nullptr;
    }
  }
  if (s.nsrc != 1) return nullptr;
  if (wide) *tile_vecs = kTileVecs * kWideVecs;  // the grid follows the kernel's tile
  return arg_items<DT, kSum, kCopy, 1, 1>(s, ptrs, k, pl, wide);
}

// Grid of `gx` tiles by `nitems` items: items along y, and along z as well
// when there are more than kGridRows.
dim3 item_grid(uint32_t gx, int nitems) {
  const uint32_t n = static_cast<uint32_t>(nitems);
  if (n <= kGridRows) return dim3(gx, n, 1);
  return dim3(gx, kGridRows, (n + kGridRows - 1) / kGridRows);
}

template <int DT, int OP>
void describe_typed(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* k) {
  constexpr uint32_t E = Width<DT>::bytes;
  k->ptrs = ptrs;
  k->items = s.items;
  k->phase = s.phase;
  k->nitems = static_cast<uint32_t>(s.nitems);
  if (!s.aligned) {
    uint64_t gx = (s.max_count + kElemThreads - 1) / kElemThreads;
    if (gx > 2048) gx = 2048;
    if (gx < 1) gx = 1;
    k->grid = item_grid(static_cast<uint32_t>(gx), s.nitems);
    k->block = dim3(kElemThreads);
    k->kind = KernelDesc::kElement;
    switch (s.mode) {
      case kCopy: k->func = fn(step_elem<DT, OP, kCopy>); break;
      case kFold: k->func = fn(step_elem<DT, OP, kFold>); break;
      default: k->func = fn(step_elem<DT, OP, kRecvFold>); break;
    }
    return;
  }
  // body vectors of the largest item (a head of fewer than 16 bytes only
  // shortens the body); tile 0 of each item also takes the head and tail
  uint64_t tv = kTileVecs;
  const void* af = arg_kernel<DT, OP>(s, ptrs, k, &tv);
  const uint64_t vecs = s.max_count * E / 16;
  const uint64_t gx = vecs > tv ? (vecs + tv - 1) / tv : 1;
  k->grid = item_grid(static_cast<uint32_t>(gx), s.nitems);
  k->block = dim3(kThreads);
  k->flags = (s.xcd_split && k->grid.z == 1 && (gx * s.nitems) % 8 == 0) ? kFlagXcdSplit : 0u;
  if (af) {
    k->kind = KernelDesc::kVectorArgs;
    k->func = af;
    return;
  }
  k->kind = KernelDesc::kVector;
  k->func = s.write_bytes > kCacheBytes ? vector_kernel<DT, OP, true>(s) : vector_kernel<DT, OP, false>(s);
  if (s.nitems >= kCapMinItems) {
    if ((s.mode == kFold && s.nsrc == 8) || (s.mode == kRecvFold && s.nsrc == 9))
      k->shared_bytes = kLdsPerCu / kFoldWgPerCu;
    else if (s.mode == kCopy && s.ndst > 1)
      k->shared_bytes = kLdsPerCu / kFanWgPerCu;
  }
}

template <int DT>
void describe_op(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* k) {
  switch (s.op) {
    case kSum: describe_typed<DT, kSum>(s, ptrs, k); break;
    case kProd: describe_typed<DT, kProd>(s, ptrs, k); break;
    case kMax: describe_typed<DT, kMax>(s, ptrs, k); break;
    default: describe_typed<DT, kMin>(s, ptrs, k); break;
  }
}

}  // namespace

hipError_t describe_step(const StepLaunch& s, const RankPtrs& ptrs, KernelDesc* k) {
  if (s.nitems <= 0) return hipErrorInvalidValue;
  if (s.ndst > 1 && s.mode != kCopy) return hipErrorInvalidValue;  // no such schedule step
  // grid.x * workgroup size must stay below 2^32 work-items: at most 2^26
  // one-wave tiles of 1 KiB, i.e. items of at most 64 GiB
  const uint32_t e = s.dtype == kF32 || s.dtype == kI32 ? 4u : (s.dtype == kI8 ? 1u : 2u);
  if (s.max_count > kMaxItemBytes / e) return hipErrorInvalidValue;
  if (static_cast<uint64_t>(s.nitems) > uint64_t(kGridRows) * kGridRows) return hipErrorInvalidValue;
  switch (s.dtype) {
    case kF32: describe_op<kF32>(s, ptrs, k); break;
    case kF16: describe_op<kF16>(s, ptrs, k); break;
    case kBF16: describe_op<kBF16>(s, ptrs, k); break;
    case kI32: describe_op<kI32>(s, ptrs, k); break;
    default: describe_op<kI8>(s, ptrs, k); break;
  }
  k->bind();
  return hipSuccess;
}

hipError_t launch_step(const StepLaunch& s, const RankPtrs& ptrs, hipStream_t stream) {
  if (s.nitems <= 0) return hipSuccess;
  KernelDesc k;
  const hipError_t e = describe_step(s, ptrs, &k);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(k.func, k.grid, k.block, k.argv, k.shared_bytes, stream);
}

}  // namespace hbmc
