/*
 * CPU oracle for the AllReduce dataflow -- TEST INFRASTRUCTURE ONLY.
 * (Only the tests, the smoke check and the bench's CPU-baseline leg use it.)
 *
 * What it computes, and from which passage (page titles as in oracle.h):
 *
 *  - The reduction's definition, Y[j] = op over ranks i of X_i[j]
 *    ([RING-RHD], section "AllReduce的数学抽象与问题定义"): orc_direct.
 *  - Ring AllReduce = ring reduce-scatter (P-1 steps) + ring all-gather
 *    (P-1 steps), each rank sending to rank+1 and receiving from rank-1
 *    ([RING-RHD], section "Ring AllReduce带宽最优的环形流水线"; [TOPO],
 *    section "AllReduce算法实现").  Segments are the ceiling split of the
 *    [TOPO] Python listing (chunk = ceil(numel / size)).  Rank r ends the
 *    reduce-scatter owning segment r, so at step t rank i sends segment
 *    (i-1-t) mod P; page [TOPO] states this ownership, page [RING-RHD]'s code
 *    is offset by one and its Python listing is inconsistent (see DESIGN).
 *  - Recursive halving-doubling ([RHD], sections "算法描述" (the 5-rank
 *    example), "耗时计算" and its Table 1; [RING-RHD], section "Recursive
 *    Halving-Doubling短消息场景的延迟优势"): r = P - 2^floor(log2 P); the
 *    first 2r ranks are merged pairwise (rank 2i+1 into rank 2i), the
 *    remaining 2^k ranks run halving (partner v xor 2^j, j = 0,1,..) then
 *    doubling in reverse, and rank 2i finally copies its result to 2i+1.
 *    Stand-alone reduce-scatter / all-gather for P = 2^k use the
 *    order-preserving variant (distance halving for reduce-scatter, so rank v
 *    ends with segment v; distance doubling for all-gather), Table 1 of [RHD].
 *  - Two-level pipeline ([PIPE], sections "AllGather 算子的 Pipeline 时序编排",
 *    "Rank0 视角的传输任务编排", "源码中的流水执行印证" and Table 1): ranks
 *    g = s*M + m; inter-server ring over servers for each local index m,
 *    intra-server full mesh; the data is sliced into loops of at most
 *    loop_bytes, each split into P blocks (block g owned by rank g).
 *    All-gather: at ring step t rank (s,m) receives block ((s-1-t)M+m) from
 *    (s-1,m) and passes block ((s-t)M+m) to the other ranks of its server;
 *    after the last ring step one more intra-server pass.  Reduce-scatter is
 *    the time reverse: one intra-server step, then S-1 ring steps that each
 *    fold the server's M contributions into the received partial.
 *  - Flat, tree and hierarchical AllReduce ([TOPO] "AllReduce算法实现": Flat
 *    below a size threshold has every device talk directly to the root; Tree
 *    reduces from the leaves of a K-ary tree to the root and broadcasts back
 *    down, 2 log_K N rounds; [PIPE] "与其它分级算法的关系": the non-pipelined
 *    hierarchical AllReduce is an intra-server reduce-scatter, an
 *    inter-server AllReduce and an intra-server all-gather).
 *  - Element ops: sum / prod / max / min; binary16 and bfloat16 are widened
 *    to binary32, combined, and rounded back to nearest even after every
 *    operation; integers wrap ([RING-RHD], section "Ascend950的AIVAICPU通信
 *    引擎与图模式", which lists addition, multiplication and maximum as the
 *    reductions the vector unit performs).
 *
 * Every step is replayed as the pages describe it: all blocks a step sends are
 * first copied into receive buffers (so every read of a step sees the state
 * before the step), then each destination combines or copies.  Two actions of
 * one step that write overlapping ranges of one rank are reported as an error.
 */
#include "oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------ */
/* floating-point environment: IEEE round-to-nearest, no flush-to-zero       */

typedef struct {
  unsigned csr;
  int round;
} fpenv_t;

static fpenv_t env_enter(void) {
  fpenv_t s;
  s.csr = _mm_getcsr();
  s.round = fegetround();
  /* clear flush-to-zero (bit 15) and denormals-are-zero (bit 6); nearest */
  _mm_setcsr((s.csr & ~(0x8000u | 0x0040u | 0x6000u)));
  fesetround(FE_TONEAREST);
  return s;
}

static void env_leave(fpenv_t s) {
  fesetround(s.round);
  _mm_setcsr(s.csr);
}

/* ------------------------------------------------------------------------ */
/* conversions, from the IEEE 754 formats' definitions                       */

static float u2f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t ex = (h >> 10) & 0x1fu, fr = h & 0x3ffu;
  if (ex == 0) { /* zero or subnormal: fr * 2^-24, exact in binary32 */
    float v = ldexpf((float)fr, -24);
    return (h & 0x8000u) ? -v : v;
  }
  if (ex == 31) return u2f(sign | 0x7f800000u | (fr << 13) | (fr ? 0x00400000u : 0u));
  return u2f(sign | ((ex - 15u + 127u) << 23) | (fr << 13));
}

uint16_t orc_f32_to_f16(float x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return sign | 0x7e00u;
  float a = fabsf(x);
  if (isinf(a) || a >= 65520.0f) return sign | 0x7c00u; /* 65520 is the tie above 65504 */
  if (a < 0x1p-14f) { /* subnormal range: count units of 2^-24 */
    float q = rintf(a * 0x1p24f);   /* exact scaling, then nearest-even */
    return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the least normal */
  }
  int ex;
  (void)frexpf(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;
  float m = rintf(ldexpf(a, 10 - E)); /* significand in [1024, 2048] */
  if (m >= 2048.0f) {
    m = 1024.0f;
    E += 1;
  }
  if (E > 15) return sign | 0x7c00u;
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024));
}

float orc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

uint16_t orc_f32_to_bf16(float x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return sign | 0x7fc0u;
  float a = fabsf(x);
  if (isinf(a)) return sign | 0x7f80u;
  if (a < 0x1p-126f) { /* subnormal range: units of 2^-133 */
    double q = rint((double)a * 0x1p133);
    return (uint16_t)(sign | (uint16_t)q);
  }
  int ex;
  (void)frexpf(a, &ex);
  int E = ex - 1;
  double m = rint(ldexp((double)a, 7 - E)); /* significand in [128, 256] */
  if (m >= 256.0) {
    m = 128.0;
    E += 1;
  }
  if (E > 127) return sign | 0x7f80u;
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)m - 128));
}

int orc_round_f32(int dtype, const float* in, uint16_t* out, size_t n) {
  if (dtype != ORC_FP16 && dtype != ORC_BF16) return ORC_EINVAL;
  fpenv_t s = env_enter();
  for (size_t i = 0; i < n; ++i) out[i] = dtype == ORC_FP16 ? orc_f32_to_f16(in[i]) : orc_f32_to_bf16(in[i]);
  env_leave(s);
  return ORC_OK;
}

int orc_widen(int dtype, const uint16_t* in, float* out, size_t n) {
  if (dtype != ORC_FP16 && dtype != ORC_BF16) return ORC_EINVAL;
  for (size_t i = 0; i < n; ++i) out[i] = dtype == ORC_FP16 ? orc_f16_to_f32(in[i]) : orc_bf16_to_f32(in[i]);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* element ops                                                                */

static size_t esize(int dtype) {
  switch (dtype) {
    case ORC_FP32: return 4;
    case ORC_FP16: return 2;
    case ORC_BF16: return 2;
    case ORC_INT32: return 4;
    case ORC_INT8: return 1;
    default: return 0;
  }
}

/* max / min over binary32: NaN in either operand gives the quiet NaN
 * 0x7FC00000; -0 orders below +0. */
static float fmax_ord(float a, float b) {
  if (isnan(a) || isnan(b)) return u2f(0x7fc00000u);
  if (a > b) return a;
  if (b > a) return b;
  if (a == 0.0f && signbit(a) != signbit(b)) return 0.0f;
  return a;
}
static float fmin_ord(float a, float b) {
  if (isnan(a) || isnan(b)) return u2f(0x7fc00000u);
  if (a < b) return a;
  if (b < a) return b;
  if (a == 0.0f && signbit(a) != signbit(b)) return -0.0f;
  return a;
}

static float fop(int op, float a, float b) {
  switch (op) {
    case ORC_SUM: return a + b;
    case ORC_PROD: return a * b;
    case ORC_MAX: return fmax_ord(a, b);
    default: return fmin_ord(a, b);
  }
}

static uint32_t uop32(int op, uint32_t a, uint32_t b) {
  int32_t sa = (int32_t)a, sb = (int32_t)b;
  switch (op) {
    case ORC_SUM: return a + b;
    case ORC_PROD: return a * b;
    case ORC_MAX: return sa >= sb ? a : b;
    default: return sa <= sb ? a : b;
  }
}

static uint8_t uop8(int op, uint8_t a, uint8_t b) {
  int8_t sa = (int8_t)a, sb = (int8_t)b;
  switch (op) {
    case ORC_SUM: return (uint8_t)(a + b);
    case ORC_PROD: return (uint8_t)(a * b);
    case ORC_MAX: return sa >= sb ? a : b;
    default: return sa <= sb ? a : b;
  }
}

static void combine_raw(int dtype, int op, const void* a, const void* b, void* out, size_t n) {
  switch (dtype) {
    case ORC_FP32: {
      const float* x = (const float*)a;
      const float* y = (const float*)b;
      float* z = (float*)out;
      for (size_t i = 0; i < n; ++i) z[i] = fop(op, x[i], y[i]);
      break;
    }
    case ORC_FP16: {
      const uint16_t* x = (const uint16_t*)a;
      const uint16_t* y = (const uint16_t*)b;
      uint16_t* z = (uint16_t*)out;
      for (size_t i = 0; i < n; ++i)
        z[i] = orc_f32_to_f16(fop(op, orc_f16_to_f32(x[i]), orc_f16_to_f32(y[i])));
      break;
    }
    case ORC_BF16: {
      const uint16_t* x = (const uint16_t*)a;
      const uint16_t* y = (const uint16_t*)b;
      uint16_t* z = (uint16_t*)out;
      for (size_t i = 0; i < n; ++i)
        z[i] = orc_f32_to_bf16(fop(op, orc_bf16_to_f32(x[i]), orc_bf16_to_f32(y[i])));
      break;
    }
    case ORC_INT32: {
      const uint32_t* x = (const uint32_t*)a;
      const uint32_t* y = (const uint32_t*)b;
      uint32_t* z = (uint32_t*)out;
      for (size_t i = 0; i < n; ++i) z[i] = uop32(op, x[i], y[i]);
      break;
    }
    default: {
      const uint8_t* x = (const uint8_t*)a;
      const uint8_t* y = (const uint8_t*)b;
      uint8_t* z = (uint8_t*)out;
      for (size_t i = 0; i < n; ++i) z[i] = uop8(op, x[i], y[i]);
      break;
    }
  }
}

int orc_combine(int dtype, int op, const void* a, const void* b, void* out, size_t n) {
  if (esize(dtype) == 0 || op < ORC_SUM || op > ORC_MIN) return ORC_EINVAL;
  if (n && (!a || !b || !out)) return ORC_EINVAL;
  fpenv_t s = env_enter();
  combine_raw(dtype, op, a, b, out, n);
  env_leave(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* the definition                                                             */

static double load_f64(int dtype, const void* p, size_t j) {
  switch (dtype) {
    case ORC_FP32: return ((const float*)p)[j];
    case ORC_FP16: return orc_f16_to_f32(((const uint16_t*)p)[j]);
    default: return orc_bf16_to_f32(((const uint16_t*)p)[j]);
  }
}

int orc_direct(int dtype, int op, int P, const void* const* srcs, size_t n, double* fp_out,
               int64_t* int_out) {
  if (esize(dtype) == 0 || op < ORC_SUM || op > ORC_MIN || P < 1 || !srcs) return ORC_EINVAL;
  int is_int = dtype == ORC_INT32 || dtype == ORC_INT8;
  if (n && ((is_int && !int_out) || (!is_int && !fp_out))) return ORC_EINVAL;
  fpenv_t s = env_enter();
  for (size_t j = 0; j < n; ++j) {
    if (is_int) {
      uint64_t acc = 0;
      for (int r = 0; r < P; ++r) {
        int64_t v = dtype == ORC_INT32 ? (int64_t)((const int32_t*)srcs[r])[j]
                                       : (int64_t)((const int8_t*)srcs[r])[j];
        if (r == 0) {
          acc = (uint64_t)v;
        } else if (op == ORC_SUM) {
          acc += (uint64_t)v;
        } else if (op == ORC_PROD) {
          acc *= (uint64_t)v;
        } else if (op == ORC_MAX) {
          if (v > (int64_t)acc) acc = (uint64_t)v;
        } else {
          if (v < (int64_t)acc) acc = (uint64_t)v;
        }
      }
      /* wrap to the element width */
      if (dtype == ORC_INT32)
        int_out[j] = (int64_t)(int32_t)(uint32_t)acc;
      else
        int_out[j] = (int64_t)(int8_t)(uint8_t)acc;
    } else {
      double acc = 0.0;
      int any_nan = 0;
      for (int r = 0; r < P; ++r) {
        double v = load_f64(dtype, srcs[r], j);
        if (isnan(v)) any_nan = 1;
        if (r == 0) {
          acc = v;
        } else if (op == ORC_SUM) {
          acc += v;
        } else if (op == ORC_PROD) {
          acc *= v;
        } else if (op == ORC_MAX) {
          if (v > acc || (v == 0.0 && acc == 0.0 && !signbit(v))) acc = v;
        } else {
          if (v < acc || (v == 0.0 && acc == 0.0 && signbit(v))) acc = v;
        }
      }
      fp_out[j] = any_nan ? NAN : acc;
    }
  }
  env_leave(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* segments: ceiling split of n elements into m parts ([TOPO] "AllReduce算法实现") */

static size_t seg_begin(size_t n, size_t m, size_t k) {
  size_t q = (n + m - 1) / m;
  size_t b = k * q;
  return b < n ? b : n;
}

static int imod(long a, long m) {
  long r = a % m;
  return (int)(r < 0 ? r + m : r);
}

static int floor_log2(int p) {
  int k = 0;
  while ((1 << (k + 1)) <= p) ++k;
  return k;
}

/* ------------------------------------------------------------------------ */
/* step replay                                                                */

#define MAX_SRC 72

typedef struct {
  int kind, dst, nsrc;
  int src[MAX_SRC];
  size_t b, n; /* element range in the full vector */
} act_t;

typedef struct {
  int P;
  void* const* bufs;
  size_t w0, w1;
  int dtype, op;
  size_t e;
  long step, first, last;
  act_t* acts;
  size_t nacts, cap;
  unsigned char* scratch;
  size_t scratch_cap;
  orc_trace_t* trace;
  size_t trace_cap, trace_len;
  int err;
} run_t;

static int in_range(const run_t* R) {
  return R->step >= R->first && (R->last < 0 || R->step < R->last);
}

static void step_begin(run_t* R) { R->nacts = 0; }

static void add_action(run_t* R, int kind, int dst, const int* src, int nsrc, size_t b, size_t n) {
  if (R->err) return;
  if (nsrc > MAX_SRC) {
    R->err = ORC_EINVAL;
    return;
  }
  if (R->nacts == R->cap) {
    size_t nc = R->cap ? 2 * R->cap : 64;
    act_t* na = (act_t*)realloc(R->acts, nc * sizeof(act_t));
    if (!na) {
      R->err = ORC_ENOMEM;
      return;
    }
    R->acts = na;
    R->cap = nc;
  }
  act_t* a = &R->acts[R->nacts++];
  a->kind = kind;
  a->dst = dst;
  a->nsrc = nsrc;
  for (int i = 0; i < nsrc; ++i) a->src[i] = src[i];
  a->b = b;
  a->n = n;
  if (in_range(R) && R->trace) {
    for (int i = 0; i < nsrc; ++i) {
      if (R->trace_len < R->trace_cap) {
        orc_trace_t* t = &R->trace[R->trace_len];
        t->step = (int32_t)R->step;
        t->kind = kind;
        t->dst = dst;
        t->src = src[i];
        t->slot = i;
        t->pad = 0;
        t->begin = b;
        t->count = n;
      }
      R->trace_len++;
    }
  }
}

static unsigned char* scratch(run_t* R, size_t bytes) {
  if (bytes > R->scratch_cap) {
    unsigned char* p = (unsigned char*)realloc(R->scratch, bytes);
    if (!p) {
      R->err = ORC_ENOMEM;
      return NULL;
    }
    R->scratch = p;
    R->scratch_cap = bytes;
  }
  return R->scratch;
}

static void clip(const run_t* R, const act_t* a, size_t* cb, size_t* ce) {
  size_t b = a->b, e = a->b + a->n;
  *cb = b > R->w0 ? b : R->w0;
  *ce = e < R->w1 ? e : R->w1;
  if (*ce < *cb) *ce = *cb;
}

/* Execute the collected actions with "send, then combine" semantics. */
static void step_end(run_t* R) {
  if (R->err) return;
  if (!in_range(R)) {
    R->step++;
    return;
  }
  /* two writes to overlapping ranges of one rank within one step are an error */
  for (size_t i = 0; i < R->nacts; ++i)
    for (size_t k = i + 1; k < R->nacts; ++k) {
      const act_t* a = &R->acts[i];
      const act_t* c = &R->acts[k];
      if (a->dst == c->dst && a->n && c->n && a->b < c->b + c->n && c->b < a->b + a->n) {
        R->err = ORC_ECONFLICT;
        return;
      }
    }
  /* receive buffers: one copy of every block read in this step (for REDUCE
   * the local block too), taken before anything is written */
  size_t total = 0;
  for (size_t i = 0; i < R->nacts; ++i) {
    size_t cb, ce;
    clip(R, &R->acts[i], &cb, &ce);
    int nread = R->acts[i].nsrc + (R->acts[i].kind == ORC_REDUCE ? 1 : 0);
    total += (ce - cb) * R->e * (size_t)(nread + 1);
  }
  unsigned char* base = scratch(R, total ? total : 1);
  if (!base) return;
  unsigned char* p = base;
  unsigned char** recv = (unsigned char**)malloc(R->nacts * sizeof(unsigned char*) + 1);
  if (!recv) {
    R->err = ORC_ENOMEM;
    return;
  }
  for (size_t i = 0; i < R->nacts; ++i) {
    const act_t* a = &R->acts[i];
    size_t cb, ce;
    clip(R, a, &cb, &ce);
    size_t bytes = (ce - cb) * R->e;
    recv[i] = p;
    for (int s = 0; s < a->nsrc; ++s) {
      memcpy(p, (const unsigned char*)R->bufs[a->src[s]] + (cb - R->w0) * R->e, bytes);
      p += bytes;
    }
    if (a->kind == ORC_REDUCE) {
      memcpy(p, (const unsigned char*)R->bufs[a->dst] + (cb - R->w0) * R->e, bytes);
      p += bytes;
    }
    p += bytes; /* room for the result */
  }
  for (size_t i = 0; i < R->nacts; ++i) {
    const act_t* a = &R->acts[i];
    size_t cb, ce;
    clip(R, a, &cb, &ce);
    size_t n = ce - cb, bytes = n * R->e;
    if (!n) continue;
    unsigned char* in = recv[i];
    unsigned char* res = in + bytes * (size_t)(a->nsrc + (a->kind == ORC_REDUCE ? 1 : 0));
    switch (a->kind) {
      case ORC_COPY:
        memcpy(res, in, bytes);
        break;
      case ORC_REDUCE: /* reduce_op(recv, local) */
        combine_raw(R->dtype, R->op, in, in + bytes, res, n);
        break;
      case ORC_FOLD:
        memcpy(res, in, bytes);
        for (int s = 1; s < a->nsrc; ++s) combine_raw(R->dtype, R->op, res, in + s * bytes, res, n);
        break;
      default: /* FOLD_RECV: op(recv, fold of slots 1..) */
        memcpy(res, in + bytes, bytes);
        for (int s = 2; s < a->nsrc; ++s) combine_raw(R->dtype, R->op, res, in + s * bytes, res, n);
        combine_raw(R->dtype, R->op, in, res, res, n);
        break;
    }
    memcpy((unsigned char*)R->bufs[a->dst] + (cb - R->w0) * R->e, res, bytes);
  }
  free(recv);
  R->step++;
}

/* ------------------------------------------------------------------------ */
/* ring ([RING-RHD] "Ring AllReduce带宽最优的环形流水线"; [TOPO] "AllReduce算法实现") */

static void ring_reduce_scatter(run_t* R, size_t L) {
  int P = R->P;
  for (int t = 0; t < P - 1; ++t) {
    step_begin(R);
    for (int i = 0; i < P; ++i) { /* rank i sends segment (i-1-t) to rank i+1 */
      int c = imod((long)i - 1 - t, P), to = (i + 1) % P;
      size_t b = seg_begin(L, (size_t)P, (size_t)c), e = seg_begin(L, (size_t)P, (size_t)c + 1);
      add_action(R, ORC_REDUCE, to, &i, 1, b, e - b);
    }
    step_end(R);
  }
}

static void ring_all_gather(run_t* R, size_t L) {
  int P = R->P;
  for (int t = 0; t < P - 1; ++t) {
    step_begin(R);
    for (int i = 0; i < P; ++i) { /* rank i forwards segment (i-t) to rank i+1 */
      int c = imod((long)i - t, P), to = (i + 1) % P;
      size_t b = seg_begin(L, (size_t)P, (size_t)c), e = seg_begin(L, (size_t)P, (size_t)c + 1);
      add_action(R, ORC_COPY, to, &i, 1, b, e - b);
    }
    step_end(R);
  }
}

/* ------------------------------------------------------------------------ */
/* recursive halving-doubling ([RHD] "算法描述", "耗时计算" Table 1)          */

/* real rank of virtual rank v when the first 2r ranks were merged in pairs */
static int rhd_real(int v, int r) { return v < r ? 2 * v : v + r; }

static void rhd_allreduce(run_t* R, size_t L) {
  int P = R->P, k = floor_log2(P), pp = 1 << k, r = P - pp;
  /* merge part1: rank 2i+1 sends everything to rank 2i, which reduces */
  if (r > 0) {
    step_begin(R);
    for (int i = 0; i < r; ++i) {
      int odd = 2 * i + 1;
      add_action(R, ORC_REDUCE, 2 * i, &odd, 1, 0, L);
    }
    step_end(R);
  }
  /* halving: distance 1, 2, 4, ...; windows are ranges of the pp-segment split */
  int lo[64], hi[64];
  for (int v = 0; v < pp; ++v) {
    lo[v] = 0;
    hi[v] = pp;
  }
  for (int j = 0; j < k; ++j) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < pp; ++v) {
      int u = v ^ (1 << j), mid = (lo[v] + hi[v]) / 2;
      int keep_low = ((v >> j) & 1) == 0;
      nlo[v] = keep_low ? lo[v] : mid;
      nhi[v] = keep_low ? mid : hi[v];
      size_t b = seg_begin(L, (size_t)pp, (size_t)nlo[v]), e = seg_begin(L, (size_t)pp, (size_t)nhi[v]);
      int src = rhd_real(u, r);
      add_action(R, ORC_REDUCE, rhd_real(v, r), &src, 1, b, e - b);
    }
    for (int v = 0; v < pp; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
  /* doubling: reverse order, each rank copies its partner's window */
  for (int j = k - 1; j >= 0; --j) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < pp; ++v) {
      int u = v ^ (1 << j);
      size_t b = seg_begin(L, (size_t)pp, (size_t)lo[u]), e = seg_begin(L, (size_t)pp, (size_t)hi[u]);
      int src = rhd_real(u, r);
      add_action(R, ORC_COPY, rhd_real(v, r), &src, 1, b, e - b);
      nlo[v] = lo[v] < lo[u] ? lo[v] : lo[u];
      nhi[v] = hi[v] > hi[u] ? hi[v] : hi[u];
    }
    for (int v = 0; v < pp; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
  /* restore part1: rank 2i sends the result to rank 2i+1 */
  if (r > 0) {
    step_begin(R);
    for (int i = 0; i < r; ++i) {
      int even = 2 * i;
      add_action(R, ORC_COPY, 2 * i + 1, &even, 1, 0, L);
    }
    step_end(R);
  }
}

/* order-preserving reduce-scatter, P = 2^k: distances P/2, P/4, ..., 1 */
static void rhd_reduce_scatter(run_t* R, size_t L) {
  int P = R->P;
  int lo[64], hi[64];
  for (int v = 0; v < P; ++v) {
    lo[v] = 0;
    hi[v] = P;
  }
  for (int d = P / 2; d >= 1; d /= 2) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < P; ++v) {
      int u = v ^ d, mid = (lo[v] + hi[v]) / 2;
      int keep_low = v < mid; /* keep the half that holds segment v */
      nlo[v] = keep_low ? lo[v] : mid;
      nhi[v] = keep_low ? mid : hi[v];
      size_t b = seg_begin(L, (size_t)P, (size_t)nlo[v]), e = seg_begin(L, (size_t)P, (size_t)nhi[v]);
      add_action(R, ORC_REDUCE, v, &u, 1, b, e - b);
    }
    for (int v = 0; v < P; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
}

/* order-preserving all-gather, P = 2^k: distances 1, 2, ..., P/2 */
static void rhd_all_gather(run_t* R, size_t L) {
  int P = R->P;
  int lo[64], hi[64];
  for (int v = 0; v < P; ++v) {
    lo[v] = v;
    hi[v] = v + 1;
  }
  for (int d = 1; d < P; d *= 2) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < P; ++v) {
      int u = v ^ d;
      size_t b = seg_begin(L, (size_t)P, (size_t)lo[u]), e = seg_begin(L, (size_t)P, (size_t)hi[u]);
      add_action(R, ORC_COPY, v, &u, 1, b, e - b);
      nlo[v] = lo[v] < lo[u] ? lo[v] : lo[u];
      nhi[v] = hi[v] > hi[u] ? hi[v] : hi[u];
    }
    for (int v = 0; v < P; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
}

/* ------------------------------------------------------------------------ */
/* RHD with P not a power of two, stand-alone ([RHD] "耗时计算", Table 1).
 * Reduce-scatter: (1) Reduce: each two-share pair merges into one rank;
 * (2) a non-uniform reduce-scatter over the 2^k virtual ranks, distance
 * halving, in which some virtual ranks hold two shares; (3) Scatter: the
 * merged rank hands the second share to its partner.  The two-share virtual
 * ranks are those whose k-bit reversal is below r, which makes the largest
 * exchange of halving step i equal to ceil(p / 2^i) shares, the table's n_i.
 * Shares (segments of the P-way split) lie in order along the virtual ranks,
 * so rank g ends owning segment g.  All-gather is the mirror image: Gather of
 * the second share, distance doubling, and a final copy of everything to the
 * partner. */

static int bitrev(int v, int k) {
  int out = 0;
  for (int i = 0; i < k; ++i)
    if ((v >> i) & 1) out |= 1 << (k - 1 - i);
  return out;
}

typedef struct {
  int k, pp, r;
  int first[65]; /* first share (= real rank) of virtual rank v; first[pp] = P */
  int two[64];   /* virtual rank v holds two shares */
} shares_t;

static void share_layout(int P, shares_t* S) {
  S->k = floor_log2(P);
  S->pp = 1 << S->k;
  S->r = P - S->pp;
  int s = 0;
  for (int v = 0; v < S->pp; ++v) {
    S->two[v] = bitrev(v, S->k) < S->r;
    S->first[v] = s;
    s += S->two[v] ? 2 : 1;
  }
  S->first[S->pp] = s;
}

static void rhd_reduce_scatter_np2(run_t* R, size_t L) {
  int P = R->P;
  shares_t S;
  share_layout(P, &S);
  /* (1) Reduce: share first+1 is folded into the rank owning share first */
  step_begin(R);
  for (int v = 0; v < S.pp; ++v)
    if (S.two[v]) {
      int odd = S.first[v] + 1;
      add_action(R, ORC_REDUCE, S.first[v], &odd, 1, 0, L);
    }
  step_end(R);
  /* (2) non-uniform halving over virtual ranks; v keeps the half holding v */
  int lo[64], hi[64];
  for (int v = 0; v < S.pp; ++v) {
    lo[v] = 0;
    hi[v] = S.pp;
  }
  for (int d = S.pp / 2; d >= 1; d /= 2) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < S.pp; ++v) {
      int u = v ^ d, mid = (lo[v] + hi[v]) / 2;
      nlo[v] = v < mid ? lo[v] : mid;
      nhi[v] = v < mid ? mid : hi[v];
      size_t b = seg_begin(L, (size_t)P, (size_t)S.first[nlo[v]]);
      size_t e = seg_begin(L, (size_t)P, (size_t)S.first[nhi[v]]);
      int src = S.first[u];
      add_action(R, ORC_REDUCE, S.first[v], &src, 1, b, e - b);
    }
    for (int v = 0; v < S.pp; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
  /* (3) Scatter: the second share goes to its own rank */
  step_begin(R);
  for (int v = 0; v < S.pp; ++v)
    if (S.two[v]) {
      int g = S.first[v] + 1, src = S.first[v];
      size_t b = seg_begin(L, (size_t)P, (size_t)g), e = seg_begin(L, (size_t)P, (size_t)g + 1);
      add_action(R, ORC_COPY, g, &src, 1, b, e - b);
    }
  step_end(R);
}

static void rhd_all_gather_np2(run_t* R, size_t L) {
  int P = R->P;
  shares_t S;
  share_layout(P, &S);
  /* (1) Gather: the partner's share comes to the merged rank */
  step_begin(R);
  for (int v = 0; v < S.pp; ++v)
    if (S.two[v]) {
      int g = S.first[v] + 1;
      size_t b = seg_begin(L, (size_t)P, (size_t)g), e = seg_begin(L, (size_t)P, (size_t)g + 1);
      add_action(R, ORC_COPY, S.first[v], &g, 1, b, e - b);
    }
  step_end(R);
  /* (2) distance doubling over virtual ranks */
  int lo[64], hi[64];
  for (int v = 0; v < S.pp; ++v) {
    lo[v] = v;
    hi[v] = v + 1;
  }
  for (int d = 1; d < S.pp; d *= 2) {
    step_begin(R);
    int nlo[64], nhi[64];
    for (int v = 0; v < S.pp; ++v) {
      int u = v ^ d;
      size_t b = seg_begin(L, (size_t)P, (size_t)S.first[lo[u]]);
      size_t e = seg_begin(L, (size_t)P, (size_t)S.first[hi[u]]);
      int src = S.first[u];
      add_action(R, ORC_COPY, S.first[v], &src, 1, b, e - b);
      nlo[v] = lo[v] < lo[u] ? lo[v] : lo[u];
      nhi[v] = hi[v] > hi[u] ? hi[v] : hi[u];
    }
    for (int v = 0; v < S.pp; ++v) {
      lo[v] = nlo[v];
      hi[v] = nhi[v];
    }
    step_end(R);
  }
  /* (3) the merged rank copies everything to its partner */
  step_begin(R);
  for (int v = 0; v < S.pp; ++v)
    if (S.two[v]) {
      int src = S.first[v];
      add_action(R, ORC_COPY, S.first[v] + 1, &src, 1, 0, L);
    }
  step_end(R);
}

/* ------------------------------------------------------------------------ */
/* RHD Reduce and Broadcast with a root ([RHD] Table 1).  For P not a power
 * of two the ranks 0..2r-1 pair up (2i, 2i+1); in each pair the rank with the
 * root's parity (even when the root is outside part1) takes part in the 2^k
 * block.  Reduce = merge of part1 + order-preserving reduce-scatter over the
 * 2^k-way split (distance halving) + gather to the root (distance doubling,
 * each rank sending the block it has collected).  Broadcast = distance
 * halving from the root over the block, then one send to each part1 partner. */

typedef struct {
  int k, pp, r, odd, vroot;
} rooted_t;

static rooted_t rooted(int P, int root) {
  rooted_t t;
  t.k = floor_log2(P);
  t.pp = 1 << t.k;
  t.r = P - t.pp;
  t.odd = (root < 2 * t.r) && (root & 1);
  t.vroot = root < 2 * t.r ? root / 2 : root - t.r;
  return t;
}
static int rooted_real(const rooted_t* t, int v) { return v < t->r ? 2 * v + t->odd : v + t->r; }
static int rooted_partner(const rooted_t* t, int i) { return 2 * i + 1 - t->odd; }

static void rhd_reduce(run_t* R, size_t L, int root) {
  rooted_t t = rooted(R->P, root);
  if (t.r > 0) {
    step_begin(R);
    for (int i = 0; i < t.r; ++i) {
      int from = rooted_partner(&t, i);
      add_action(R, ORC_REDUCE, rooted_real(&t, i), &from, 1, 0, L);
    }
    step_end(R);
  }
  /* reduce-scatter: virtual rank v ends with segment v of the pp-way split */
  for (int d = t.pp / 2; d >= 1; d /= 2) {
    step_begin(R);
    for (int v = 0; v < t.pp; ++v) {
      int a = v & ~(d - 1); /* aligned block of d segments holding v */
      size_t b = seg_begin(L, (size_t)t.pp, (size_t)a), e = seg_begin(L, (size_t)t.pp, (size_t)(a + d));
      int src = rooted_real(&t, v ^ d);
      add_action(R, ORC_REDUCE, rooted_real(&t, v), &src, 1, b, e - b);
    }
    step_end(R);
  }
  /* gather to the root: at distance d the rank whose offset from the root
   * has lowest set bit d sends its collected block of d segments */
  for (int d = 1; d < t.pp; d *= 2) {
    step_begin(R);
    for (int v = 0; v < t.pp; ++v) {
      int rel = v ^ t.vroot;
      if ((rel & d) && !(rel & (d - 1))) {
        int a = v & ~(d - 1), src = rooted_real(&t, v);
        size_t b = seg_begin(L, (size_t)t.pp, (size_t)a), e = seg_begin(L, (size_t)t.pp, (size_t)(a + d));
        add_action(R, ORC_COPY, rooted_real(&t, v ^ d), &src, 1, b, e - b);
      }
    }
    step_end(R);
  }
}

static void rhd_broadcast(run_t* R, size_t L, int root) {
  rooted_t t = rooted(R->P, root);
  for (int d = t.pp / 2; d >= 1; d /= 2) {
    step_begin(R);
    for (int v = 0; v < t.pp; ++v)
      if (((v ^ t.vroot) & (2 * d - 1)) == 0) {
        int src = rooted_real(&t, v);
        add_action(R, ORC_COPY, rooted_real(&t, v ^ d), &src, 1, 0, L);
      }
    step_end(R);
  }
  if (t.r > 0) {
    step_begin(R);
    for (int i = 0; i < t.r; ++i) {
      int src = rooted_real(&t, i);
      add_action(R, ORC_COPY, rooted_partner(&t, i), &src, 1, 0, L);
    }
    step_end(R);
  }
}

/* ------------------------------------------------------------------------ */
/* two-level pipeline ([PIPE] "AllGather 算子的 Pipeline 时序编排", Table 1)  */

typedef struct {
  int S, M;
  size_t lb, n; /* loop's first element and length */
} pipe_t;

static void blk(const run_t* R, const pipe_t* pl, int g, size_t* b, size_t* n) {
  size_t bb = seg_begin(pl->n, (size_t)R->P, (size_t)g), ee = seg_begin(pl->n, (size_t)R->P, (size_t)g + 1);
  *b = pl->lb + bb;
  *n = ee - bb;
}

static void pipe_reduce_scatter(run_t* R, const pipe_t* pl) {
  int S = pl->S, M = pl->M;
  int src[MAX_SRC];
  size_t b, n;
  /* intra-server step: (s,m) folds its server's contributions to the block
   * that its ring neighbour expects first */
  step_begin(R);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      for (int l = 0; l < M; ++l) src[l] = s * M + l;
      blk(R, pl, imod((long)s - 1, S) * M + m, &b, &n);
      add_action(R, ORC_FOLD, s * M + m, src, M, b, n);
    }
  step_end(R);
  /* ring steps: receive the partial from (s-1,m), fold in the server's own */
  for (int t = 0; t < S - 1; ++t) {
    step_begin(R);
    for (int s = 0; s < S; ++s)
      for (int m = 0; m < M; ++m) {
        src[0] = imod((long)s - 1, S) * M + m;
        for (int l = 0; l < M; ++l) src[1 + l] = s * M + l;
        blk(R, pl, imod((long)s - t - 2, S) * M + m, &b, &n);
        add_action(R, ORC_FOLD_RECV, s * M + m, src, M + 1, b, n);
      }
    step_end(R);
  }
}

static void pipe_all_gather(run_t* R, const pipe_t* pl) {
  int S = pl->S, M = pl->M;
  size_t b, n;
  for (int t = 0; t < S - 1; ++t) {
    step_begin(R);
    for (int s = 0; s < S; ++s)
      for (int m = 0; m < M; ++m) {
        int g = s * M + m, from = imod((long)s - 1, S) * M + m;
        blk(R, pl, imod((long)s - 1 - t, S) * M + m, &b, &n);
        add_action(R, ORC_COPY, g, &from, 1, b, n);
        blk(R, pl, imod((long)s - t, S) * M + m, &b, &n);
        for (int l = 0; l < M; ++l)
          if (l != m) add_action(R, ORC_COPY, s * M + l, &g, 1, b, n);
      }
    step_end(R);
  }
  /* closing intra-server pass of the block received in the last ring step */
  step_begin(R);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      int g = s * M + m;
      blk(R, pl, imod((long)s + 1, S) * M + m, &b, &n);
      for (int l = 0; l < M; ++l)
        if (l != m) add_action(R, ORC_COPY, s * M + l, &g, 1, b, n);
    }
  step_end(R);
}

/* ------------------------------------------------------------------------ */
/* Flat, tree and hierarchical AllReduce                                      */

/* Flat: rank 0 receives every rank's vector and reduces them in rank order,
 * then sends the result to every rank. */
static void flat_allreduce(run_t* R, size_t L) {
  int P = R->P, all[64];
  for (int r = 0; r < P; ++r) all[r] = r;
  step_begin(R);
  add_action(R, ORC_FOLD, 0, all, P, 0, L);
  step_end(R);
  step_begin(R);
  for (int r = 1; r < P; ++r) {
    int root = 0;
    add_action(R, ORC_COPY, r, &root, 1, 0, L);
  }
  step_end(R);
}

/* Tree: K-ary tree in heap order (parent of i is (i-1)/K).  Reduce rounds go
 * from the deepest level of parents up to the root, each parent folding its
 * own vector and its children's (in rank order); broadcast rounds go back
 * down, each parent copying the result to its children. */
static int tree_depth(int i, int K) {
  int d = 0;
  while (i > 0) {
    i = (i - 1) / K;
    ++d;
  }
  return d;
}

static void tree_allreduce(run_t* R, size_t L, int K) {
  int P = R->P, maxd = tree_depth(P - 1, K);
  for (int lvl = maxd - 1; lvl >= 0; --lvl) {
    step_begin(R);
    for (int p = 0; p < P; ++p) {
      if (tree_depth(p, K) != lvl || K * p + 1 >= P) continue;
      int src[MAX_SRC], n = 0;
      src[n++] = p;
      for (int c = K * p + 1; c <= K * p + K && c < P; ++c) src[n++] = c;
      add_action(R, ORC_FOLD, p, src, n, 0, L);
    }
    step_end(R);
  }
  for (int lvl = 0; lvl < maxd; ++lvl) {
    step_begin(R);
    for (int p = 0; p < P; ++p) {
      if (tree_depth(p, K) != lvl) continue;
      for (int c = K * p + 1; c <= K * p + K && c < P; ++c) add_action(R, ORC_COPY, c, &p, 1, 0, L);
    }
    step_end(R);
  }
}

/* Hierarchical (not pipelined), S servers x M ranks, rank g = s*M + m:
 * (1) intra-server reduce-scatter by full mesh: (s,m) folds block m (M-way
 *     ceiling split) of its server's M vectors, in local-rank order;
 * (2) inter-server ring AllReduce of block m among (0,m) .. (S-1,m), with the
 *     ring's S-way ceiling split of the block and its step rules;
 * (3) intra-server all-gather by full mesh: (s,m) sends block m to its peers. */
static void hier_allreduce(run_t* R, size_t L, int S, int M) {
  int src[MAX_SRC];
  step_begin(R);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      for (int l = 0; l < M; ++l) src[l] = s * M + l;
      size_t b = seg_begin(L, (size_t)M, (size_t)m), e = seg_begin(L, (size_t)M, (size_t)m + 1);
      add_action(R, ORC_FOLD, s * M + m, src, M, b, e - b);
    }
  step_end(R);
  for (int phase = 0; phase < 2; ++phase)
    for (int t = 0; t < S - 1; ++t) {
      step_begin(R);
      for (int m = 0; m < M; ++m) {
        size_t b0 = seg_begin(L, (size_t)M, (size_t)m), n = seg_begin(L, (size_t)M, (size_t)m + 1) - b0;
        for (int i = 0; i < S; ++i) { /* server i sends to server i+1 */
          int c = phase == 0 ? imod((long)i - 1 - t, S) : imod((long)i - t, S);
          size_t b = b0 + seg_begin(n, (size_t)S, (size_t)c), e = b0 + seg_begin(n, (size_t)S, (size_t)c + 1);
          int from = i * M + m, to = ((i + 1) % S) * M + m;
          add_action(R, phase == 0 ? ORC_REDUCE : ORC_COPY, to, &from, 1, b, e - b);
        }
      }
      step_end(R);
    }
  step_begin(R);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      int g = s * M + m;
      size_t b = seg_begin(L, (size_t)M, (size_t)m), e = seg_begin(L, (size_t)M, (size_t)m + 1);
      for (int l = 0; l < M; ++l)
        if (l != m) add_action(R, ORC_COPY, s * M + l, &g, 1, b, e - b);
    }
  step_end(R);
}

/* ------------------------------------------------------------------------ */
/* entry points                                                               */

static size_t loop_elems(size_t loop_bytes, int dtype) {
  if (loop_bytes == 0) loop_bytes = (size_t)32 << 20;
  size_t c = loop_bytes / esize(dtype);
  return c ? c : 1;
}

long orc_num_steps(int coll, int algo, int P, int S, int M, size_t L, int dtype,
                   size_t loop_bytes) {
  (void)L;
  (void)dtype;
  (void)loop_bytes;
  (void)M;
  if (P <= 1) return 0;
  const int pow2 = (P & (P - 1)) == 0, k = floor_log2(P);
  if (algo == ORC_RHD) {
    switch (coll) {
      case ORC_ALLREDUCE: return 2 * k + (pow2 ? 0 : 2);
      case ORC_REDUCE_SCATTER:
      case ORC_ALL_GATHER: return k + (pow2 ? 0 : 2);
      case ORC_ROOT_REDUCE: return 2 * k + (pow2 ? 0 : 1);
      default: return k + (pow2 ? 0 : 1);
    }
  }
  if (algo == ORC_FLAT) return 2;
  if (algo == ORC_TREE) {
    int d = 0;
    for (int i = P - 1; i > 0; i = (i - 1) / (M < 2 ? 2 : M)) ++d;
    return 2 * d;
  }
  if (algo == ORC_HIER) return 2 * S;
  long half = algo == ORC_RING ? P - 1 : S;
  return coll == ORC_ALLREDUCE ? 2 * half : half;
}

int orc_collective(int coll, int algo, int P, int S, int M, size_t loop_bytes, int root,
                   void* const* bufs, size_t L, size_t w0, size_t w1, int dtype, int op,
                   long first_step, long last_step, orc_trace_t* trace, size_t trace_cap,
                   size_t* trace_len) {
  if (trace_len) *trace_len = 0;
  if (P < 1 || P > 64 || esize(dtype) == 0 || op < ORC_SUM || op > ORC_MIN) return ORC_EINVAL;
  if (coll < ORC_ALLREDUCE || coll > ORC_BROADCAST || algo < ORC_RING || algo > ORC_HIER)
    return ORC_EINVAL;
  if (w0 > w1 || w1 > L || (w1 > w0 && !bufs)) return ORC_EINVAL;
  if ((algo == ORC_PIPELINE || algo == ORC_HIER) && (S < 1 || M < 1 || S * M != P || M + 1 > MAX_SRC))
    return ORC_EINVAL;
  if (algo == ORC_TREE && (M < 2 || M + 1 > MAX_SRC)) return ORC_EINVAL;
  if (algo >= ORC_FLAT && coll != ORC_ALLREDUCE) return ORC_EUNSUPPORTED;
  if ((coll == ORC_ROOT_REDUCE || coll == ORC_BROADCAST) && (root < 0 || root >= P)) return ORC_EINVAL;
  if ((coll == ORC_ROOT_REDUCE || coll == ORC_BROADCAST) && algo != ORC_RHD) return ORC_EUNSUPPORTED;
  if (w1 > w0)
    for (int r = 0; r < P; ++r)
      if (!bufs[r]) return ORC_EINVAL;

  run_t R;
  memset(&R, 0, sizeof(R));
  R.P = P;
  R.bufs = bufs;
  R.w0 = w0;
  R.w1 = w1;
  R.dtype = dtype;
  R.op = op;
  R.e = esize(dtype);
  R.first = first_step;
  R.last = last_step;
  R.trace = trace;
  R.trace_cap = trace ? trace_cap : 0;

  fpenv_t s = env_enter();
  if (P > 1) {
    if (algo == ORC_RING) {
      if (coll != ORC_ALL_GATHER) ring_reduce_scatter(&R, L);
      if (coll != ORC_REDUCE_SCATTER) ring_all_gather(&R, L);
    } else if (algo == ORC_RHD) {
      const int pow2 = (P & (P - 1)) == 0;
      switch (coll) {
        case ORC_ALLREDUCE: rhd_allreduce(&R, L); break;
        case ORC_REDUCE_SCATTER: pow2 ? rhd_reduce_scatter(&R, L) : rhd_reduce_scatter_np2(&R, L); break;
        case ORC_ALL_GATHER: pow2 ? rhd_all_gather(&R, L) : rhd_all_gather_np2(&R, L); break;
        case ORC_ROOT_REDUCE: rhd_reduce(&R, L, root); break;
        default: rhd_broadcast(&R, L, root); break;
      }
    } else if (algo == ORC_FLAT) {
      flat_allreduce(&R, L);
    } else if (algo == ORC_TREE) {
      tree_allreduce(&R, L, M);
    } else if (algo == ORC_HIER) {
      hier_allreduce(&R, L, S, M);
    } else {
      size_t C = loop_elems(loop_bytes, dtype);
      for (size_t lb = 0; lb < L && !R.err; lb += C) {
        pipe_t pl;
        pl.S = S;
        pl.M = M;
        pl.lb = lb;
        pl.n = (L - lb) < C ? (L - lb) : C;
        /* a loop outside the replayed window changes nothing there */
        if (!trace && (lb + pl.n <= w0 || lb >= w1)) continue;
        R.step = 0; /* steps are numbered within a loop; all loops share them */
        if (coll != ORC_ALL_GATHER) pipe_reduce_scatter(&R, &pl);
        if (coll != ORC_REDUCE_SCATTER) pipe_all_gather(&R, &pl);
      }
    }
  }
  env_leave(s);
  if (trace_len) *trace_len = R.trace_len;
  free(R.acts);
  free(R.scratch);
  return R.err;
}
