// Device element ops shared by every kernel family (step, single-workgroup,
// column and LDS-resident kernels): fp16 / bf16 sums and products widen to
// fp32, combine and round back to nearest even per operation; integers wrap;
// max / min order -0 below +0 and give the canonical quiet NaN when either
// operand is NaN.  Floating max / min compare order keys: the bit pattern
// with all bits flipped when the sign bit is set, else with the sign bit
// set, which sorts negative values below positive ones and -0 under +0.
#pragma once

#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "plan.hpp"

namespace hbmc {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { kF32 = 0, kF16 = 1, kBF16 = 2, kI32 = 3, kI8 = 4 };
enum { kSum = 0, kProd = 1, kMax = 2, kMin = 3 };

template <int DT>
struct Width {
  static constexpr uint32_t bytes = (DT == kF32 || DT == kI32) ? 4 : (DT == kI8 ? 1 : 2);
};

// ------------------------------------------------------------- element ops

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

template <int OP>
__device__ __forceinline__ uint32_t op_f32(uint32_t a, uint32_t b) {
  if constexpr (OP == kSum) {
    return f2u(u2f(a) + u2f(b));
  } else if constexpr (OP == kProd) {
    return f2u(u2f(a) * u2f(b));
  } else {
    // order keys without a branch (an arithmetic shift spreads the sign),
    // the unsigned max / min of the keys, and the winner's key turned back
    const uint32_t ka = a ^ (static_cast<uint32_t>(static_cast<int32_t>(a) >> 31) | 0x80000000u);
    const uint32_t kb = b ^ (static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u);
    const uint32_t k = OP == kMax ? (ka > kb ? ka : kb) : (ka < kb ? ka : kb);
    const uint32_t r = k ^ (~static_cast<uint32_t>(static_cast<int32_t>(k) >> 31) | 0x80000000u);
    const uint32_t ma = a & 0x7fffffffu, mb = b & 0x7fffffffu;
    return (ma > mb ? ma : mb) > 0x7f800000u ? 0x7fc00000u : r;
  }
}

__device__ __forceinline__ float widen_f16(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
__device__ __forceinline__ uint32_t narrow_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // v_cvt_f16_f32, nearest even
}
// fp16 sum / product of one 16-bit lane (value in the low half of the word).
template <int OP>
__device__ __forceinline__ uint32_t op_f16(uint32_t a, uint32_t b) {
  static_assert(OP == kSum || OP == kProd, "fp16 max / min take minmax_h16x2");
  const float x = widen_f16(a), y = widen_f16(b);
  return narrow_f16(OP == kSum ? x + y : x * y);
}

template <int OP>
__device__ __forceinline__ int op_int(int x, int y) {
  if constexpr (OP == kSum) return static_cast<int>(static_cast<uint32_t>(x) + static_cast<uint32_t>(y));
  if constexpr (OP == kProd) return static_cast<int>(static_cast<uint32_t>(x) * static_cast<uint32_t>(y));
  if constexpr (OP == kMax) return x >= y ? x : y;
  return x <= y ? x : y;
}

// bf16 sum / product of both halves of a word: each half widened exactly
// to fp32, combined in fp32, and both rounded to nearest even by one packed
// conversion (v_cvt_pk_bf16_f32: a NaN keeps its sign and payload, quieted).
template <int OP>
__device__ __forceinline__ uint32_t op_bf16x2(uint32_t a, uint32_t b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const float xl = u2f(a << 16), xh = u2f(a & 0xffff0000u);
  const float yl = u2f(b << 16), yh = u2f(b & 0xffff0000u);
  const f32x2 z = OP == kSum ? f32x2{xl + yl, xh + yh} : f32x2{xl * yl, xh * yh};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(z, bf16x2));
}

// fp16 / bf16 max or min of both halves of a word at once: each half's order
// key, the packed unsigned max / min of the keys, the winning
// key turned back into its bits, and the canonical quiet NaN in every half
// where either operand is a NaN (a saturating subtract of the infinity
// pattern is nonzero exactly there).
template <int DT, int OP>
__device__ __forceinline__ uint32_t minmax_h16x2(uint32_t a, uint32_t b) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
  constexpr uint16_t inf = DT == kF16 ? 0x7c00u : 0x7f80u;
  constexpr uint32_t qnan2 = DT == kF16 ? 0x7e007e00u : 0x7fc07fc0u;
  const u16x2 top = {0x8000u, 0x8000u}, low = {0x7fffu, 0x7fffu}, lim = {inf, inf}, one = {1u, 1u};
  const u16x2 A = __builtin_bit_cast(u16x2, a), B = __builtin_bit_cast(u16x2, b);
  const u16x2 ka = A ^ (__builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, A) >> 15) | top);
  const u16x2 kb = B ^ (__builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, B) >> 15) | top);
  const u16x2 k = OP == kMax ? __builtin_elementwise_max(ka, kb) : __builtin_elementwise_min(ka, kb);
  const u16x2 r = k ^ (~__builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, k) >> 15) | top);
  const u16x2 d = __builtin_elementwise_sub_sat(__builtin_elementwise_max(A & low, B & low), lim);
  const u16x2 zero = {0u, 0u};
  const uint32_t mask = __builtin_bit_cast(uint32_t, u16x2(zero - __builtin_elementwise_min(d, one)));
  return (__builtin_bit_cast(uint32_t, r) & ~mask) | (qnan2 & mask);
}

// The op on one 32-bit word of packed elements.
template <int DT, int OP>
__device__ __forceinline__ uint32_t op_word(uint32_t a, uint32_t b) {
  if constexpr (DT == kF32) {
    return op_f32<OP>(a, b);
  } else if constexpr (DT == kBF16 && (OP == kSum || OP == kProd)) {
    return op_bf16x2<OP>(a, b);
  } else if constexpr ((DT == kF16 || DT == kBF16) && (OP == kMax || OP == kMin)) {
    return minmax_h16x2<DT, OP>(a, b);
  } else if constexpr (DT == kF16) {
    return op_f16<OP>(a & 0xffffu, b & 0xffffu) | (op_f16<OP>(a >> 16, b >> 16) << 16);
  } else if constexpr (DT == kI32) {
    return static_cast<uint32_t>(op_int<OP>(static_cast<int>(a), static_cast<int>(b)));
  } else if constexpr (OP == kSum) {
    // four wrapping int8 adds: the low 7 bits of each byte cannot carry into
    // the next byte, and each byte's top bit is its carry-in xor both top bits
    return ((a & 0x7f7f7f7fu) + (b & 0x7f7f7f7fu)) ^ ((a ^ b) & 0x80808080u);
  } else {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
      const int x = static_cast<int8_t>(a >> k), y = static_cast<int8_t>(b >> k);
      r |= (static_cast<uint32_t>(op_int<OP>(x, y)) & 0xffu) << k;
    }
    return r;
  }
}

template <int DT, int OP>
__device__ __forceinline__ u32x4 op_vec(u32x4 a, u32x4 b) {
  u32x4 r;
  r.x = op_word<DT, OP>(a.x, b.x);
  r.y = op_word<DT, OP>(a.y, b.y);
  r.z = op_word<DT, OP>(a.z, b.z);
  r.w = op_word<DT, OP>(a.w, b.w);
  return r;
}

// 16-byte vector access.  Loads carry the nontemporal hint.  Stores are plain
// write-back stores, or nontemporal ones (`store_vec_nt`) where the step
// kernel is told that a step writes more than the memory-side cache holds.
__device__ __forceinline__ u32x4 load_vec(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_vec(u32x4* p, u32x4 v) { *p = v; }
__device__ __forceinline__ void store_vec_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

template <uint32_t E>
__device__ __forceinline__ uint32_t load_elem(const unsigned char* p) {
  if constexpr (E == 4) return *reinterpret_cast<const uint32_t*>(p);
  if constexpr (E == 2) return *reinterpret_cast<const uint16_t*>(p);
  return *p;
}
template <uint32_t E>
__device__ __forceinline__ void store_elem(unsigned char* p, uint32_t v) {
  if constexpr (E == 4) *reinterpret_cast<uint32_t*>(p) = v;
  else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v);
  else *p = static_cast<unsigned char>(v);
}

// Buffer of an item's i-th rank.  The rank index is read as part of its
// aligned 32-bit word: gfx950 has no scalar byte load, and a byte read becomes
// a vector load that waits behind the streaming traffic before any data load
// of the workgroup can be addressed.
__device__ __forceinline__ unsigned char* rank_buf(const RankPtrs& ptrs, const DevItem* it, int i) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(it->rank)[i >> 2];
  return ptrs.p[(w >> ((i & 3) * 8)) & 0xffu];
}

// An item's operands read from the device item table: the i-th is the
// buffer of the item's i-th rank, element offsets count from its start.
struct ItemBufs {
  const RankPtrs& ptrs;
  const DevItem* it;
  __device__ __forceinline__ unsigned char* operator()(int i) const { return rank_buf(ptrs, it, i); }
};

// An item's operands resolved on the host (kernel arguments): the i-th is
// the address of the item's first element in that operand.
template <int NB>
struct ArgBufs {
  const ArgItem<NB>* a;
  __device__ __forceinline__ unsigned char* operator()(int i) const { return a->buf[i]; }
};

// Combination of an item's sources at one element (byte offset `off` from
// each operand address `b(i)`).
template <int DT, int OP, int MODE, typename B>
__device__ __forceinline__ uint32_t combine_elem(const B& b, int ns, uint64_t off) {
  constexpr uint32_t E = Width<DT>::bytes;
  if constexpr (MODE == kCopy) {
    return load_elem<E>(b(0) + off);
  } else if constexpr (MODE == kFold) {
    uint32_t acc = load_elem<E>(b(0) + off);
    for (int s = 1; s < ns; ++s) acc = op_word<DT, OP>(acc, load_elem<E>(b(s) + off));
    return acc;
  } else {
    uint32_t acc = load_elem<E>(b(1) + off);
    for (int s = 2; s < ns; ++s) acc = op_word<DT, OP>(acc, load_elem<E>(b(s) + off));
    return op_word<DT, OP>(load_elem<E>(b(0) + off), acc);
  }
}

template <int DT, int OP, int MODE, typename B>
__device__ __forceinline__ void do_elem(const B& b, int ns, int nd, uint64_t elem) {
  constexpr uint32_t E = Width<DT>::bytes;
  const uint64_t off = elem * E;
  const uint32_t v = combine_elem<DT, OP, MODE>(b, ns, off);
  for (int d = 0; d < nd; ++d) store_elem<E>(b(ns + d) + off, v);
}

template <int DT, int OP, int MODE>
__device__ __forceinline__ void do_elem(const RankPtrs& ptrs, const DevItem* it, int ns, int nd,
                                        uint64_t elem) {
  do_elem<DT, OP, MODE>(ItemBufs{ptrs, it}, ns, nd, elem);
}

}  // namespace dev
}  // namespace hbmc
