// LDS-resident column kernel: one launch runs a range of schedule steps for
// calls whose rank buffers the caches hold, where time goes to the fixed cost
// of every step ([RHD] "耗时计算": each step pays alpha) rather than to HBM.
//
// As in the column kernel, every step combines operands at equal element
// offsets, so the elements [g*C, (g+1)*C) of all rank buffers (column g)
// evolve on their own.  Here one workgroup takes a whole column into LDS and
// runs the column's chunks in schedule order on the LDS copies, then writes
// back the rank buffers some chunk wrote.  Same items, element ops and order
// as the step kernels: bit-identical results.
//
// No barrier between steps: the column's bytes are cut into 16-byte
// positions (aligned like the global addresses), and lane t of the workgroup
// owns positions t, t + blockDim.x, ... of every rank's copy for the whole
// launch: it loads them, applies every chunk to the elements of its
// positions (whole-vector ops where a chunk covers a position, element ops
// where a chunk edge cuts it), and stores them back.  Every element is only
// ever touched by its owning lane, so a step's results are ordered before the
// next step's reads by the lane's own program order.  The one barrier makes
// the chunk records (copied into LDS by wave 0 while the lanes load their
// data) visible to every wave.
//
// In a launch of all of a call's steps, a column whose chunk list ends in
// copies over three or more steps (the ring's all-gather, RHD's doubling and
// restore, a stand-alone all-gather) does not run those copies: they only
// pass finished values from one rank's copy to another's, so the host
// composes them into store records (DevColStore) that write each rank's
// final bytes from the LDS copy holding them.  The bits are the same; the
// column's chain of dependent chunk passes is shorter (ring: P - 1 instead
// of 2 (P - 1)), and ranks that neither a remaining chunk nor a store record
// reads are not loaded (a stand-alone all-gather loads only the owners).
//
// LDS layout (dynamic): nranks slots of slot_bytes (element col_begin + i of
// rank r at slot r + phase + i*E, so LDS and global 16-byte phases agree),
// then one DevColChunk record per chunk the column runs, then its store
// records.
//
// A chunk's cost is a short dependent chain (record words, then its data,
// then the op and the store), so the loop is kept lean: ONE marks launches
// in which every lane owns at most one position (lane t takes position t,
// no position loop), and the two single-chunk shapes the schedules mostly
// use, a two-source reduce and a one-to-one copy, are tested right after
// the batches and run without the generic shape dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "elemops.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace {

using namespace dev;

constexpr int kLdsMaxThreads = 256;
constexpr int kLdsUnroll = 8;  // ranks whose 16-byte loads a lane has in flight while filling LDS

__device__ __forceinline__ uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Rank number s of a chunk: the first 16 from the scalar words `rw`, the
// rest from the record in LDS.
__device__ __forceinline__ uint32_t rank_of(const uint32_t* rw, const uint8_t* lds_ranks, int s) {
  return s < 16 ? (rw[s >> 2] >> (8 * (s & 3))) & 0xffu : uni(lds_ranks[s]);
}

// One 16-byte position (slot offset o) of one chunk, whole vector.
template <int DT, int OP, int MODE, int NS, int ND>
__device__ __forceinline__ void pos_vec(unsigned char* lds, uint32_t slot_bytes, uint32_t o, int ns, int nd,
                                        const uint32_t* rw, const uint8_t* lr) {
  auto at = [&](int s) { return reinterpret_cast<u32x4*>(lds + rank_of(rw, lr, s) * slot_bytes + o); };
  u32x4 acc;
  if constexpr (MODE == kCopy) {
    acc = *at(0);
  } else if constexpr (MODE == kFold) {
    acc = *at(0);
    for (int s = 1; s < ns; ++s) acc = op_vec<DT, OP>(acc, *at(s));
  } else {
    acc = *at(1);
    for (int s = 2; s < ns; ++s) acc = op_vec<DT, OP>(acc, *at(s));
    acc = op_vec<DT, OP>(*at(0), acc);
  }
  for (int d = 0; d < nd; ++d) *at(ns + d) = acc;
}

// Elements of one chunk inside one position: slot offsets [lo, hi).
template <int DT, int OP, int MODE, int NS, int ND>
__device__ __forceinline__ void pos_elems(unsigned char* lds, uint32_t slot_bytes, uint32_t lo, uint32_t hi,
                                          int ns, int nd, const uint32_t* rw, const uint8_t* lr) {
  constexpr uint32_t E = Width<DT>::bytes;
  auto at = [&](int s, uint32_t o) { return lds + rank_of(rw, lr, s) * slot_bytes + o; };
  for (uint32_t o = lo; o < hi; o += E) {
    uint32_t acc;
    if constexpr (MODE == kCopy) {
      acc = load_elem<E>(at(0, o));
    } else if constexpr (MODE == kFold) {
      acc = load_elem<E>(at(0, o));
      for (int s = 1; s < ns; ++s) acc = op_word<DT, OP>(acc, load_elem<E>(at(s, o)));
    } else {
      acc = load_elem<E>(at(1, o));
      for (int s = 2; s < ns; ++s) acc = op_word<DT, OP>(acc, load_elem<E>(at(s, o)));
      acc = op_word<DT, OP>(load_elem<E>(at(0, o)), acc);
    }
    for (int d = 0; d < nd; ++d) store_elem<E>(at(ns + d, o), acc);
  }
}

// This lane's positions of one chunk covering slot bytes [lo, hi).
template <int DT, int OP, int MODE, int NS, int ND, bool ONE>
__device__ __forceinline__ void lds_chunk(unsigned char* lds, uint32_t slot_bytes, uint32_t lo, uint32_t hi,
                                          int ns_rt, int nd_rt, const uint32_t* rw, const uint8_t* lr) {
  const int ns = NS > 0 ? NS : ns_rt;
  const int nd = ND > 0 ? ND : nd_rt;
  const uint32_t p_lo = lo >> 4, p_hi = (hi + 15) >> 4;
  auto one = [&](uint32_t p) {
    const uint32_t a = p * 16, b = a + 16;
    if (a >= lo && b <= hi) pos_vec<DT, OP, MODE, NS, ND>(lds, slot_bytes, a, ns, nd, rw, lr);
    else pos_elems<DT, OP, MODE, NS, ND>(lds, slot_bytes, a > lo ? a : lo, b < hi ? b : hi, ns, nd, rw, lr);
  };
  if constexpr (ONE) {
    // lane t owns position t only
    if (threadIdx.x >= p_lo && threadIdx.x < p_hi) one(threadIdx.x);
  } else {
    const uint32_t nthr = blockDim.x;  // a power of two
    // first position >= p_lo owned by this lane
    for (uint32_t p = p_lo + ((threadIdx.x - p_lo) & (nthr - 1)); p < p_hi; p += nthr) one(p);
  }
}

// This lane's positions of a batch of NB chunks of one step that share the
// byte range [lo, hi) and a shape: two-source reduce (MODE kRecvFold:
// rank[k] = src0 | src1 << 8 | dst << 16) or copy (kCopy: src | dst << 8).
// The chunks are independent, so every load of the batch is issued before
// any result is combined; the element-wise edges go chunk by chunk.
template <int DT, int OP, int MODE, int NB>
__device__ __forceinline__ void lds_batch(unsigned char* lds, uint32_t slot_bytes, uint32_t lo, uint32_t hi,
                                          const uint32_t* rank) {
  constexpr uint32_t E = Width<DT>::bytes;
  const uint32_t nthr = blockDim.x;  // a power of two
  const uint32_t p_lo = lo >> 4, p_hi = (hi + 15) >> 4;
  uint32_t p = p_lo + ((threadIdx.x - p_lo) & (nthr - 1));
  auto slot = [&](int k, int which) { return lds + ((rank[k] >> (8 * which)) & 0xffu) * slot_bytes; };
  for (; p < p_hi; p += nthr) {
    const uint32_t a = p * 16, b = a + 16;
    if (a >= lo && b <= hi) {
      u32x4 x[NB], y[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        x[k] = *reinterpret_cast<const u32x4*>(slot(k, 0) + a);
        if constexpr (MODE == kRecvFold) y[k] = *reinterpret_cast<const u32x4*>(slot(k, 1) + a);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if constexpr (MODE == kRecvFold) *reinterpret_cast<u32x4*>(slot(k, 2) + a) = op_vec<DT, OP>(x[k], y[k]);
        else *reinterpret_cast<u32x4*>(slot(k, 1) + a) = x[k];
      }
    } else {
      const uint32_t l = a > lo ? a : lo, h = b < hi ? b : hi;
      for (uint32_t o = l; o < h; o += E) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          if constexpr (MODE == kRecvFold)
            store_elem<E>(slot(k, 2) + o, op_word<DT, OP>(load_elem<E>(slot(k, 0) + o), load_elem<E>(slot(k, 1) + o)));
          else
            store_elem<E>(slot(k, 1) + o, load_elem<E>(slot(k, 0) + o));
        }
      }
    }
  }
}

template <int DT, int OP, int NB>
__device__ __forceinline__ void run_batch(unsigned char* lds, uint32_t slot_bytes, uint32_t lo, uint32_t hi,
                                          uint32_t mode, const uint32_t* rank) {
  if (mode == kRecvFold) lds_batch<DT, OP, kRecvFold, NB>(lds, slot_bytes, lo, hi, rank);
  else lds_batch<DT, kSum, kCopy, NB>(lds, slot_bytes, lo, hi, rank);
}

// Global <-> LDS for this lane's positions of every rank in `mask`: the
// column's bytes are slot offsets [phase, phase + n*E); whole positions move
// as 16-byte vectors, the cut first / last positions element by element.
template <int DT, bool TO_LDS>
__device__ __forceinline__ void move_positions(unsigned char* lds, uint32_t slot_bytes, const RankPtrs& ptrs,
                                               uint64_t col_byte, uint64_t mask, uint32_t nranks, uint32_t phase,
                                               uint32_t n) {
  constexpr uint32_t E = Width<DT>::bytes;
  const uint32_t lo = phase, hi = phase + n * E;
  const uint32_t nthr = blockDim.x;
  for (uint32_t p = threadIdx.x; p < ((hi + 15) >> 4); p += nthr) {
    const uint32_t a = p * 16, b = a + 16;
    if (a >= lo && b <= hi) {
      for (uint32_t r0 = 0; r0 < nranks; r0 += kLdsUnroll) {
        u32x4 x[kLdsUnroll];
#pragma unroll
        for (int u = 0; u < kLdsUnroll; ++u) {
          const uint32_t r = r0 + u;
          if (r < nranks && ((mask >> r) & 1u)) {
            // global address of slot byte a of rank r
            const u32x4* g = reinterpret_cast<const u32x4*>(ptrs.p[r] + col_byte - phase + a);
            if constexpr (TO_LDS) x[u] = load_vec(g);
            else x[u] = *reinterpret_cast<const u32x4*>(lds + r * slot_bytes + a);
          }
        }
#pragma unroll
        for (int u = 0; u < kLdsUnroll; ++u) {
          const uint32_t r = r0 + u;
          if (r < nranks && ((mask >> r) & 1u)) {
            if constexpr (TO_LDS) *reinterpret_cast<u32x4*>(lds + r * slot_bytes + a) = x[u];
            else store_vec(reinterpret_cast<u32x4*>(ptrs.p[r] + col_byte - phase + a), x[u]);
          }
        }
      }
    } else {
      const uint32_t l = a > lo ? a : lo, h = b < hi ? b : hi;
      for (uint32_t r = 0; r < nranks; ++r) {
        if (!((mask >> r) & 1u)) continue;
        for (uint32_t o = l; o < h; o += E) {
          unsigned char* g = ptrs.p[r] + col_byte - phase + o;
          unsigned char* s = lds + r * slot_bytes + o;
          if constexpr (TO_LDS) store_elem<E>(s, load_elem<E>(g));
          else store_elem<E>(g, load_elem<E>(s));
        }
      }
    }
  }
}

// This lane's positions of slot bytes [lo, hi) of one LDS copy (`src`) into
// a rank's global buffer (`g`: the global address of slot byte 0).
template <int DT, bool ONE>
__device__ __forceinline__ void store_range(const unsigned char* src, unsigned char* g, uint32_t lo, uint32_t hi) {
  constexpr uint32_t E = Width<DT>::bytes;
  const uint32_t p_lo = lo >> 4, p_hi = (hi + 15) >> 4;
  auto one = [&](uint32_t p) {
    const uint32_t a = p * 16, b = a + 16;
    if (a >= lo && b <= hi) {
      store_vec(reinterpret_cast<u32x4*>(g + a), *reinterpret_cast<const u32x4*>(src + a));
    } else {
      const uint32_t l = a > lo ? a : lo, h = b < hi ? b : hi;
      for (uint32_t o = l; o < h; o += E) store_elem<E>(g + o, load_elem<E>(src + o));
    }
  };
  if constexpr (ONE) {
    if (threadIdx.x >= p_lo && threadIdx.x < p_hi) one(threadIdx.x);
  } else {
    const uint32_t nthr = blockDim.x;  // a power of two
    for (uint32_t p = p_lo + ((threadIdx.x - p_lo) & (nthr - 1)); p < p_hi; p += nthr) one(p);
  }
}

// Workgroup w runs columns w, w + gridDim.x, ...; of each column only the
// chunks of steps [s_lo, s_hi).  Chunk headers are read into scalar
// registers, so every branch on them is uniform.
template <int DT, int OP, bool ONE>
__global__ void __launch_bounds__(kLdsMaxThreads)
plan_columns_lds(RankPtrs ptrs, const DevColChunk* __restrict__ image, const uint32_t* __restrict__ col_off,
                 uint32_t ncols, uint32_t s_lo, uint32_t s_hi, uint32_t phase, uint64_t col_elems, uint64_t count,
                 uint32_t nranks, uint32_t slot_bytes, const DevColStore* __restrict__ stores,
                 const uint32_t* __restrict__ col_run, const uint32_t* __restrict__ st_off,
                 const uint64_t* __restrict__ col_load) {
  constexpr uint32_t E = Width<DT>::bytes;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  DevColChunk* meta = reinterpret_cast<DevColChunk*>(lds + nranks * slot_bytes);
  const uint64_t all = nranks >= 64 ? ~uint64_t(0) : ((uint64_t(1) << nranks) - 1);

  for (uint32_t g = blockIdx.x; g < ncols; g += gridDim.x) {
    const uint64_t col_begin = uint64_t(g) * col_elems;
    const uint32_t n = static_cast<uint32_t>(count - col_begin < col_elems ? count - col_begin : col_elems);
    const uint32_t k0 = col_off[g];
    const uint32_t nk = stores ? col_run[g] : col_off[g + 1] - k0;
    const uint32_t st0 = stores ? st_off[g] : 0, nst = stores ? st_off[g + 1] - st0 : 0;
    const DevColStore* st_lds = reinterpret_cast<const DevColStore*>(meta + nk);
    if (threadIdx.x < 64) {
      // the column's chunk records into LDS (ten 16-byte words each), then
      // its store records (one word each)
      const u32x4* src = reinterpret_cast<const u32x4*>(image + k0);
      u32x4* dst = reinterpret_cast<u32x4*>(meta);
      for (uint32_t w = threadIdx.x; w < nk * 10; w += 64) dst[w] = src[w];
      const u32x4* ssrc = reinterpret_cast<const u32x4*>(stores + st0);
      u32x4* sdst = reinterpret_cast<u32x4*>(meta + nk);
      for (uint32_t w = threadIdx.x; w < nst; w += 64) sdst[w] = ssrc[w];
    }
    move_positions<DT, true>(lds, slot_bytes, ptrs, col_begin * E, stores ? col_load[g] : all, nranks, phase, n);
    __syncthreads();
    uint64_t dirty = 0;
    for (uint32_t j = 0; j < nk; ++j) {
      // the record's three 16-byte words together: one LDS round trip
      const u32x4 h = *reinterpret_cast<const u32x4*>(&meta[j]);
      const u32x4 mv = *reinterpret_cast<const u32x4*>(&meta[j].dst_mask);
      const u32x4 rv = *reinterpret_cast<const u32x4*>(meta[j].rank);
      const uint32_t step = uni(h.z);
      const uint32_t lo = phase + uni(h.x), hi = phase + uni(h.y), shape = uni(h.w);
      const uint32_t m0 = uni(mv.x), m1 = uni(mv.y), nb = uni(mv.z);
      const uint32_t rw[4] = {uni(rv.x), uni(rv.y), uni(rv.z), uni(rv.w)};
      if (step < s_lo || step >= s_hi) continue;
      dirty |= uint64_t(m0) | (uint64_t(m1) << 32);
      if (nb > 1) {
        // a batch: the same step, range and shape; its first ranks and masks
        uint32_t rank[8];
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
          if (k >= nb) break;
          rank[k] = k == 0 ? rw[0] : uni(*reinterpret_cast<const uint32_t*>(meta[j + k].rank));
          if (k > 0) {
            const u32x4 mk = *reinterpret_cast<const u32x4*>(&meta[j + k].dst_mask);
            dirty |= uint64_t(uni(mk.x)) | (uint64_t(uni(mk.y)) << 32);
          }
        }
        const uint32_t mode = shape & 0xffu;
        if (nb == 8) run_batch<DT, OP, 8>(lds, slot_bytes, lo, hi, mode, rank);
        else if (nb == 4) run_batch<DT, OP, 4>(lds, slot_bytes, lo, hi, mode, rank);
        else run_batch<DT, OP, 2>(lds, slot_bytes, lo, hi, mode, rank);
        j += nb - 1;
        continue;
      }
      // the common single chunks: a two-source reduce, a one-to-one copy
      if (shape == (kRecvFold | 2u << 8 | 1u << 16)) {
        lds_chunk<DT, OP, kRecvFold, 2, 1, ONE>(lds, slot_bytes, lo, hi, 2, 1, rw, meta[j].rank);
        continue;
      }
      if (shape == (kCopy | 1u << 8 | 1u << 16)) {
        lds_chunk<DT, kSum, kCopy, 1, 1, ONE>(lds, slot_bytes, lo, hi, 1, 1, rw, meta[j].rank);
        continue;
      }
      const uint8_t* lr = meta[j].rank;
      const uint32_t mode = shape & 0xffu;
      const int ns = static_cast<int>((shape >> 8) & 0xffu), nd = static_cast<int>(shape >> 16);
      if (mode == kRecvFold) {
        if (ns == 2 && nd == 1) lds_chunk<DT, OP, kRecvFold, 2, 1, ONE>(lds, slot_bytes, lo, hi, ns, nd, rw, lr);
        else lds_chunk<DT, OP, kRecvFold, 0, 0, ONE>(lds, slot_bytes, lo, hi, ns, nd, rw, lr);
      } else if (mode == kFold) {
        lds_chunk<DT, OP, kFold, 0, 0, ONE>(lds, slot_bytes, lo, hi, ns, nd, rw, lr);
      } else {
        if (ns == 1 && nd == 1) lds_chunk<DT, kSum, kCopy, 1, 1, ONE>(lds, slot_bytes, lo, hi, ns, nd, rw, lr);
        else lds_chunk<DT, kSum, kCopy, 0, 0, ONE>(lds, slot_bytes, lo, hi, ns, nd, rw, lr);
      }
    }
    if (nst > 0) {
      // four records at a time: their LDS reads go out together
      for (uint32_t i = 0; i < nst; i += 4) {
        uint32_t lo[4], hi[4], dst[4], src[4];
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          const u32x4 r = i + q < nst ? *reinterpret_cast<const u32x4*>(st_lds + i + q) : u32x4{0, 0, 0, 0};
          lo[q] = phase + uni(r.x);
          hi[q] = phase + uni(r.y);
          dst[q] = uni(r.z);
          src[q] = uni(r.w);
        }
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
          if (i + q < nst)
            store_range<DT, ONE>(lds + src[q] * slot_bytes, ptrs.p[dst[q]] + col_begin * E - phase, lo[q], hi[q]);
      }
    } else {
      move_positions<DT, false>(lds, slot_bytes, ptrs, col_begin * E, dirty, nranks, phase, n);
    }
    __syncthreads();  // the chunk records are refilled for the next column
  }
}

template <int DT, bool ONE>
const void* lds_fn(int op) {
  switch (op) {
    case kSum: return reinterpret_cast<const void*>(plan_columns_lds<DT, kSum, ONE>);
    case kProd: return reinterpret_cast<const void*>(plan_columns_lds<DT, kProd, ONE>);
    case kMax: return reinterpret_cast<const void*>(plan_columns_lds<DT, kMax, ONE>);
    default: return reinterpret_cast<const void*>(plan_columns_lds<DT, kMin, ONE>);
  }
}

template <int DT>
const void* lds_fn(int op, bool one) {
  return one ? lds_fn<DT, true>(op) : lds_fn<DT, false>(op);
}

}  // namespace

uint32_t lds_threads(uint64_t col_elems, uint32_t e) {
  // a column's buffers of phase > 0 touch one more position, which a lane
  // takes as its second; whole waves, a power of two (the lanes' position
  // arithmetic relies on it)
  const uint64_t positions = std::max<uint64_t>(1, col_elems * e / 16);
  return positions <= 64 ? 64 : (positions <= 128 ? 128 : 256);
}

uint32_t lds_slot_bytes(uint64_t col_elems, uint32_t e) {
  return static_cast<uint32_t>((col_elems * e + 16 + 15) / 16 * 16);
}

uint64_t lds_bytes(int nranks, uint64_t col_elems, uint32_t e, uint64_t max_chunks_per_col) {
  return uint64_t(nranks) * lds_slot_bytes(col_elems, e) + max_chunks_per_col * sizeof(DevColChunk);
}

void describe_columns_lds(int dtype, int op, const RankPtrs& ptrs, const DevColChunk* image, const uint32_t* col_off,
                          uint32_t ncols, uint32_t s_lo, uint32_t s_hi, uint32_t phase, uint64_t col_elems,
                          uint64_t count, uint32_t nranks, uint64_t meta_bytes, uint32_t grid,
                          const DevColStore* stores, const uint32_t* col_run, const uint32_t* st_off,
                          const uint64_t* col_load, KernelDesc* k) {
  const uint32_t e = dtype == kF32 || dtype == kI32 ? 4 : (dtype == kI8 ? 1 : 2);
  // every lane owns at most one 16-byte position of the column
  const bool one = (phase + col_elems * e + 15) / 16 <= lds_threads(col_elems, e);
  switch (dtype) {
    case kF32: k->func = lds_fn<kF32>(op, one); break;
    case kF16: k->func = lds_fn<kF16>(op, one); break;
    case kBF16: k->func = lds_fn<kBF16>(op, one); break;
    case kI32: k->func = lds_fn<kI32>(op, one); break;
    default: k->func = lds_fn<kI8>(op, one); break;
  }
  k->kind = KernelDesc::kColumnsLds;
  k->grid = dim3(grid);
  k->block = dim3(lds_threads(col_elems, e));
  k->ptrs = ptrs;
  k->image = image;
  k->col_off = col_off;
  k->ncols = ncols;
  k->s_lo = s_lo;
  k->s_hi = s_hi;
  k->phase = phase;
  k->col_elems = col_elems;
  k->count = count;
  k->nranks = nranks;
  k->slot_bytes = lds_slot_bytes(col_elems, e);
  k->shared_bytes = static_cast<uint32_t>(uint64_t(nranks) * k->slot_bytes + meta_bytes);
  k->stores = stores;
  k->col_run = col_run;
  k->st_off = st_off;
  k->col_load = col_load;
  k->bind();
}

}  // namespace hbmc
