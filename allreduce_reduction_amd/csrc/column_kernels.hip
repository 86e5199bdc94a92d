// Column kernel: one launch runs a whole range of schedule steps, for calls
// whose working set the caches hold, where time goes to the fixed per-step
// cost ([RHD] "耗时计算": every step pays alpha) rather than to HBM.
//
// Every step combines operands at equal element offsets, so the elements
// [g*C, (g+1)*C) of all rank buffers (column g, C the chunk length) evolve
// independently of every other column: cutting each item at multiples of C,
// the chunks of a column depend only on earlier chunks of the same column.
// One wave therefore runs a column's chunks in schedule order (step after
// step, each step's chunks in item order) with no synchronisation with other
// waves: no flags, no atomics, no barriers, and a wave never waits on another.
// Between steps the wave orders its own stores before its next loads with a
// workgroup-scope fence (program order of one wave through its compute
// unit's memory pipeline).  Same items, element ops and order as the step
// kernels: bit-identical results.  In the spirit of the pipelined segments of
// [RING-RHD] "Ring AllReduce带宽最优的环形流水线", each column runs the
// schedule on its own, so no step waits for the whole previous step.
#include <hip/hip_runtime.h>

#include "elemops.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace {

using namespace dev;

constexpr int kColThreads = 64;  // one wave per workgroup
constexpr int kColUnroll = 4;    // 16-byte vectors per lane per operand in flight

// Elements [begin, begin+count) of one item by one wave.  NS / ND > 0 fix the
// item shape at compile time.
template <int DT, int OP, int MODE, int NS, int ND>
__device__ __forceinline__ void column_body(const RankPtrs& ptrs, const DevItem* it, uint64_t begin,
                                          uint64_t count, uint32_t phase) {
  constexpr uint32_t E = Width<DT>::bytes;
  const uint32_t lane = threadIdx.x;
  const int ns = NS > 0 ? NS : static_cast<int>(it->nsrc);
  const int nd = ND > 0 ? ND : static_cast<int>(it->ndst);
  uint64_t head = ((16u - ((phase + begin * E) & 15u)) & 15u) / E;
  if (head > count) head = count;
  const uint64_t nvec = (count - head) * E / 16;
  const uint64_t body_end = head + nvec * (16 / E);
  const uint64_t base = (begin + head) * E;

  for (uint64_t v0 = lane; v0 < nvec; v0 += uint64_t(kColThreads) * kColUnroll) {
    u32x4 acc[kColUnroll];
    if constexpr (NS > 0) {
      u32x4 x[NS][kColUnroll];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4* p = reinterpret_cast<const u32x4*>(rank_buf(ptrs, it, s) + base);
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kColThreads;
          if (v < nvec) x[s][u] = load_vec(p + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u) {
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
        const u32x4* p = reinterpret_cast<const u32x4*>(rank_buf(ptrs, it, first) + base);
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kColThreads;
          if (v < nvec) acc[u] = load_vec(p + v);
        }
      }
      if constexpr (MODE != kCopy) {
        for (int s = first + 1; s < ns; ++s) {
          const u32x4* p = reinterpret_cast<const u32x4*>(rank_buf(ptrs, it, s) + base);
#pragma unroll
          for (int u = 0; u < kColUnroll; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kColThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(acc[u], load_vec(p + v));
          }
        }
        if constexpr (MODE == kRecvFold) {
          const u32x4* p = reinterpret_cast<const u32x4*>(rank_buf(ptrs, it, 0) + base);
#pragma unroll
          for (int u = 0; u < kColUnroll; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kColThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(load_vec(p + v), acc[u]);
          }
        }
      }
    }
    for (int d = 0; d < (ND > 0 ? ND : nd); ++d) {
      u32x4* q = reinterpret_cast<u32x4*>(rank_buf(ptrs, it, ns + d) + base);
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u) {
        const uint64_t v = v0 + uint64_t(u) * kColThreads;
        if (v < nvec) store_vec(q + v, acc[u]);
      }
    }
  }
  // head and tail elements (fewer than 16 bytes each)
  if (lane < head) do_elem<DT, OP, MODE>(ptrs, it, ns, nd, begin + lane);
  if (lane >= 32 && lane - 32 < count - body_end) do_elem<DT, OP, MODE>(ptrs, it, ns, nd, begin + body_end + (lane - 32));
}

template <int DT, int OP>
__device__ __forceinline__ void column_chunk(const RankPtrs& ptrs, const DevItem* it, uint64_t begin,
                                           uint64_t count, uint32_t mode, uint32_t phase) {
  const uint32_t ns = it->nsrc, nd = it->ndst;
  if (mode == kRecvFold) {
    if (ns == 2 && nd == 1) column_body<DT, OP, kRecvFold, 2, 1>(ptrs, it, begin, count, phase);
    else column_body<DT, OP, kRecvFold, 0, 0>(ptrs, it, begin, count, phase);
  } else if (mode == kFold) {
    column_body<DT, OP, kFold, 0, 0>(ptrs, it, begin, count, phase);
  } else {
    if (ns == 1 && nd == 1) column_body<DT, kSum, kCopy, 1, 1>(ptrs, it, begin, count, phase);
    else column_body<DT, kSum, kCopy, 0, 0>(ptrs, it, begin, count, phase);
  }
}

// Workgroup w runs columns w, w + gridDim.x, ...; of each column only the
// chunks with index in [c_lo, c_hi) (steps of this launch; the column list is
// ascending, so they are contiguous in it).  All branches are uniform: the
// column and chunk indices and the chunk records are the same for all lanes.
template <int DT, int OP>
__global__ void __launch_bounds__(kColThreads)
plan_columns(RankPtrs ptrs, const DevItem* __restrict__ items, const DevChunk* __restrict__ chunks,
             const uint32_t* __restrict__ col_list, const uint32_t* __restrict__ col_off, uint32_t ncols,
             uint32_t c_lo, uint32_t c_hi, uint32_t phase) {
  for (uint32_t g = blockIdx.x; g < ncols; g += gridDim.x) {
    const uint32_t k0 = col_off[g], k1 = col_off[g + 1];
    uint32_t prev_step = UINT32_MAX;
    for (uint32_t k = k0; k < k1; ++k) {
      const uint32_t c = col_list[k];
      if (c < c_lo) continue;
      if (c >= c_hi) break;
      const DevChunk ch = chunks[c];
      // this column's chunks of the previous step are done before any of this step
      if (ch.step != prev_step && prev_step != UINT32_MAX) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      prev_step = ch.step;
      column_chunk<DT, OP>(ptrs, items + ch.item, ch.begin, ch.count, ch.mode, phase);
    }
  }
}

template <int DT>
const void* columns_fn(int op) {
  switch (op) {
    case kSum: return reinterpret_cast<const void*>(plan_columns<DT, kSum>);
    case kProd: return reinterpret_cast<const void*>(plan_columns<DT, kProd>);
    case kMax: return reinterpret_cast<const void*>(plan_columns<DT, kMax>);
    default: return reinterpret_cast<const void*>(plan_columns<DT, kMin>);
  }
}

}  // namespace

void describe_columns(int dtype, int op, const RankPtrs& ptrs, const DevItem* items, const DevChunk* chunks,
                      const uint32_t* col_list, const uint32_t* col_off, uint32_t ncols, uint32_t c_lo,
                      uint32_t c_hi, uint32_t phase, uint32_t grid, KernelDesc* k) {
  switch (dtype) {
    case kF32: k->func = columns_fn<kF32>(op); break;
    case kF16: k->func = columns_fn<kF16>(op); break;
    case kBF16: k->func = columns_fn<kBF16>(op); break;
    case kI32: k->func = columns_fn<kI32>(op); break;
    default: k->func = columns_fn<kI8>(op); break;
  }
  k->kind = KernelDesc::kColumns;
  k->grid = dim3(grid);
  k->block = dim3(kColThreads);
  k->ptrs = ptrs;
  k->items = items;
  k->chunks = chunks;
  k->col_list = col_list;
  k->col_off = col_off;
  k->ncols = ncols;
  k->c_lo = c_lo;
  k->c_hi = c_hi;
  k->phase = phase;
  k->bind();
}

}  // namespace hbmc
