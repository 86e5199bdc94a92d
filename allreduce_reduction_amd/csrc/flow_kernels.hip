// Flow kernel: all steps of a call in one launch, for calls too large for the
// one-launch forms whose working set the caches hold, so that consecutive
// steps overlap instead of meeting at a kernel boundary ([RING-RHD] "Ring
// AllReduce带宽最优的环形流水线": the ring pipelines its segments so that no
// rank waits for a whole step; "Ascend950的AIVAICPU通信引擎与图模式": tasks
// issued ahead and ordered by their data dependencies).
//
// Every step combines operands at equal element offsets, so column g
// (elements [g*C, (g+1)*C) of every rank buffer) evolves on its own: the work
// of step s on column g (a tile: the step's items cut to the column) depends
// only on the column's tiles of earlier steps.  Tiles are numbered step after
// step and handed out by one atomic ticket counter; a workgroup that takes
// the seq-th tile of column g waits until the column's counter reads seq,
// runs the tile (every operand read from and every result written to the
// rank buffers, exactly as the step kernel does: each step still moves its
// own bytes), and sets the counter to seq + 1.
//
// Progress: a tile waits only on a tile of its column with a smaller ticket,
// which a running workgroup already holds (tickets are taken by running
// workgroups only, at most one ahead of the tile a workgroup runs), so the
// smallest unfinished ticket can always proceed.  Every wait is bounded in
// wall-clock time all the same: a wait past the bound counts a timeout in the
// plan's counter, raises the launch's give-up flag and skips its
// tile; waits that see the flag give up at once, so every workgroup reaches
// the exit.  The last workgroup to leave resets the ticket and column
// counters for the next launch.
//
// Memory ordering across compute units (and XCDs, whose L2s are separate):
// every wave waits for its own stores before the workgroup barrier, then one
// lane releases at agent scope and stores the column counter; the waiting
// lane reads the counter at agent scope and acquires at agent scope before
// the workgroup barrier that lets the tile's loads go.  Same items, element
// ops and order as the step kernels: bit-identical results.
#include <hip/hip_runtime.h>

#include "elemops.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace {

using namespace dev;

constexpr int kFlowUnroll = 4;  // 16-byte vectors per lane per operand in flight

// Operand i of a chunk: the buffer of its i-th rank (rank bytes read as
// aligned words, which the scalar unit loads).
struct ChunkBufs {
  const RankPtrs& ptrs;
  const FlowChunk* ch;
  __device__ __forceinline__ unsigned char* operator()(int i) const {
    const uint32_t w = reinterpret_cast<const uint32_t*>(ch->rank)[i >> 2];
    return ptrs.p[(w >> ((i & 3) * 8)) & 0xffu];
  }
};

// Elements [begin, begin+count) of one item by the whole workgroup.  NS / ND
// > 0 fix the item shape at compile time (all loads of a pass issued before
// any combine); 0 takes ns / nd.
template <int DT, int OP, int MODE, int NS, int ND, bool NT>
__device__ __forceinline__ void flow_body(const ChunkBufs& bufs, uint64_t begin, uint64_t count, uint32_t phase,
                                          int ns, int nd) {
  constexpr uint32_t E = Width<DT>::bytes;
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
  const uint64_t base = (begin + head) * E;

  for (uint64_t v0 = threadIdx.x; v0 < nvec; v0 += uint64_t(kFlowThreads) * kFlowUnroll) {
    u32x4 acc[kFlowUnroll];
    if constexpr (NS > 0) {
      u32x4 x[NS][kFlowUnroll];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4* p = reinterpret_cast<const u32x4*>((ND > 0 ? buf[s] : bufs(s)) + base);
#pragma unroll
        for (int u = 0; u < kFlowUnroll; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kFlowThreads;
          if (v < nvec) x[s][u] = load_vec(p + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kFlowUnroll; ++u) {
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
        for (int u = 0; u < kFlowUnroll; ++u) {
          const uint64_t v = v0 + uint64_t(u) * kFlowThreads;
          if (v < nvec) acc[u] = load_vec(p + v);
        }
      }
      if constexpr (MODE != kCopy) {
        for (int s = first + 1; s < ns; ++s) {
          const u32x4* p = reinterpret_cast<const u32x4*>(bufs(s) + base);
#pragma unroll
          for (int u = 0; u < kFlowUnroll; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kFlowThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(acc[u], load_vec(p + v));
          }
        }
        if constexpr (MODE == kRecvFold) {
          const u32x4* p = reinterpret_cast<const u32x4*>(bufs(0) + base);
#pragma unroll
          for (int u = 0; u < kFlowUnroll; ++u) {
            const uint64_t v = v0 + uint64_t(u) * kFlowThreads;
            if (v < nvec) acc[u] = op_vec<DT, OP>(load_vec(p + v), acc[u]);
          }
        }
      }
    }
    for (int d = 0; d < (ND > 0 ? ND : nd); ++d) {
      u32x4* q = reinterpret_cast<u32x4*>((NS > 0 && ND > 0 ? buf[NS + d] : bufs(ns + d)) + base);
#pragma unroll
      for (int u = 0; u < kFlowUnroll; ++u) {
        const uint64_t v = v0 + uint64_t(u) * kFlowThreads;
        if (v < nvec) {
          if constexpr (NT) store_vec_nt(q + v, acc[u]);
          else store_vec(q + v, acc[u]);
        }
      }
    }
  }
  // head and tail elements (fewer than 16 bytes each)
  const uint32_t t = threadIdx.x;
  if (t < head) do_elem<DT, OP, MODE>(bufs, ns, nd, begin + t);
  if (t >= 128 && t - 128 < count - body_end) do_elem<DT, OP, MODE>(bufs, ns, nd, begin + body_end + (t - 128));
}

template <int DT, int OP, bool NT>
__device__ __forceinline__ void flow_chunk(const RankPtrs& ptrs, const FlowChunk* ch, uint32_t phase) {
  const uint32_t shape = ch->shape;
  const uint32_t mode = shape & 0xffu;
  const int ns = static_cast<int>((shape >> 8) & 0xffu), nd = static_cast<int>(shape >> 16);
  const ChunkBufs b{ptrs, ch};
  const uint64_t begin = ch->begin, count = ch->count;
  if (mode == kRecvFold) {
    if (ns == 2 && nd == 1) flow_body<DT, OP, kRecvFold, 2, 1, NT>(b, begin, count, phase, ns, nd);
    else flow_body<DT, OP, kRecvFold, 0, 0, NT>(b, begin, count, phase, ns, nd);
  } else if (mode == kFold) {
    if (ns == 2 && nd == 1) flow_body<DT, OP, kFold, 2, 1, NT>(b, begin, count, phase, ns, nd);
    else flow_body<DT, OP, kFold, 0, 0, NT>(b, begin, count, phase, ns, nd);
  } else {
    if (ns == 1 && nd == 1) flow_body<DT, kSum, kCopy, 1, 1, NT>(b, begin, count, phase, ns, nd);
    else flow_body<DT, kSum, kCopy, 0, 0, NT>(b, begin, count, phase, ns, nd);
  }
}

__device__ __forceinline__ uint32_t take_tickets(FlowCtrl* ctrl, uint32_t n) {
  return __hip_atomic_fetch_add(&ctrl->next, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *counter reads `target` (1), or give up (0): at once when the
// launch's give-up flag is raised, else after `wait_ticks` of the wall clock,
// counting a timeout and raising the flag.
__device__ __forceinline__ uint32_t wait_turn(uint32_t* counter, uint32_t target, FlowCtrl* ctrl,
                                              uint32_t* timeouts, uint64_t wait_ticks) {
  if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target) return 1;
  const uint64_t t0 = static_cast<uint64_t>(wall_clock64());
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target) return 1;
    if (__hip_atomic_load(&ctrl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return 0;
    if (static_cast<uint64_t>(wall_clock64()) - t0 > wait_ticks) {
      __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return 0;
    }
  }
}

// Every memory operation this wave issued has completed: its stores are
// acknowledged (before the barrier after which one lane releases the
// workgroup's results), and a cache write-back or invalidate it issued is
// done (after the release and acquire fences, whose code the compiler may
// leave without a wait of its own when no load or store is outstanding).
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int DT, int OP, bool NT>
__global__ void __launch_bounds__(kFlowThreads)
plan_flow(RankPtrs ptrs, const FlowTile* __restrict__ tiles, const FlowChunk* __restrict__ chunks, uint32_t ntiles,
          FlowCtrl* ctrl, uint32_t* progress, uint32_t ncols, uint32_t* timeouts, uint32_t phase, uint32_t flags,
          uint64_t wait_ticks, uint32_t batch) {
  __shared__ uint32_t s_ticket, s_ok, s_last;
  const uint32_t tid = threadIdx.x;
  uint32_t next = 0;
  // tickets are taken `batch` at a time: a workgroup runs tiles [t0, t0 +
  // batch) in order, and takes its next batch as it starts this one
  if (tid == 0) s_ticket = take_tickets(ctrl, batch);
  __syncthreads();
  for (;;) {
    const uint32_t t0 = __builtin_amdgcn_readfirstlane(s_ticket);
    if (t0 >= ntiles) break;
    if (tid == 0) next = take_tickets(ctrl, batch);
    const uint32_t t1 = ntiles - t0 < batch ? ntiles : t0 + batch;
    for (uint32_t t = t0; t < t1; ++t) {
      const FlowTile tile = tiles[t];
      if (tid == 0) {
        uint32_t ok = 1;
        if (tile.seq > 0)
          ok = wait_turn(progress + tile.col, (flags & kFlowUnreachable) ? UINT32_MAX : tile.seq, ctrl, timeouts,
                         wait_ticks);
        if (ok) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          wait_memory();
        }
        s_ok = ok;
      }
      __syncthreads();
      const uint32_t ok = __builtin_amdgcn_readfirstlane(s_ok);
      if (ok)
        for (uint32_t c = tile.c_lo; c < tile.c_hi; ++c) flow_chunk<DT, OP, NT>(ptrs, chunks + c, phase);
      wait_memory();
      __syncthreads();
      if (tid == 0 && ok) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        wait_memory();
        __hip_atomic_store(progress + tile.col, tile.seq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (tid == 0) s_ticket = next;
    __syncthreads();
  }
  // every workgroup has taken exactly one batch past the last tile; the
  // last one out resets the counters
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&ctrl->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    for (uint32_t i = tid; i < ncols; i += kFlowThreads)
      __hip_atomic_store(progress + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(&ctrl->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->abort, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int DT, int OP>
const void* flow_nt(bool nt) {
  return nt ? reinterpret_cast<const void*>(plan_flow<DT, OP, true>)
            : reinterpret_cast<const void*>(plan_flow<DT, OP, false>);
}

template <int DT>
const void* flow_fn(int op, bool nt) {
  switch (op) {
    case kSum: return flow_nt<DT, kSum>(nt);
    case kProd: return flow_nt<DT, kProd>(nt);
    case kMax: return flow_nt<DT, kMax>(nt);
    default: return flow_nt<DT, kMin>(nt);
  }
}

}  // namespace

void describe_flow(int dtype, int op, const RankPtrs& ptrs, const FlowTile* tiles, const FlowChunk* chunks,
                   uint32_t ntiles, FlowCtrl* ctrl, uint32_t* progress, uint32_t ncols, uint32_t* timeouts,
                   uint32_t phase, uint32_t flags, uint64_t wait_ticks, uint32_t batch, uint32_t grid,
                   KernelDesc* k) {
  const bool nt = (flags & kFlowNtStores) != 0;
  switch (dtype) {
    case kF32: k->func = flow_fn<kF32>(op, nt); break;
    case kF16: k->func = flow_fn<kF16>(op, nt); break;
    case kBF16: k->func = flow_fn<kBF16>(op, nt); break;
    case kI32: k->func = flow_fn<kI32>(op, nt); break;
    default: k->func = flow_fn<kI8>(op, nt); break;
  }
  k->kind = KernelDesc::kFlow;
  k->grid = dim3(grid);
  k->block = dim3(kFlowThreads);
  k->shared_bytes = 0;
  k->ptrs = ptrs;
  k->ftiles = tiles;
  k->fchunks = chunks;
  k->ntiles = ntiles;
  k->fctrl = ctrl;
  k->fprog = progress;
  k->ncols = ncols;
  k->ftimeouts = timeouts;
  k->phase = phase;
  k->flags = flags & kFlowUnreachable;
  k->wait_ticks = wait_ticks;
  k->fbatch = batch;
  k->bind();
}

}  // namespace hbmc
