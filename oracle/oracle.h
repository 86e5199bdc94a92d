/*
 * CPU oracle for the AllReduce dataflow -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, single-threaded C.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load it; the product path never does.  It shares no
 * code, header, table or constant generator with the GPU library.
 *
 * Pages cited (titles as printed; no line numbers):
 *   [RING-RHD]  "HCCL Ring AllReduce 与 Recursive Halving-Doubling 对比"
 *               (mhpn.cn/news/973985)
 *   [TOPO]      HCCL topology-aware routing article
 *               (hwcomputing.csdn.net/6a38a89e10ee7a33f280a3ac.html)
 *   [RHD]       "HCCL RHD（Recursive Halving-Doubling）算法深度解析"
 *               (mhpn.cn/news/2258316)
 *   [PIPE]      "HCCL Pipeline分级流水算法深度解析：原理、时序编排与耗时模型"
 *               (lpnh.cn/news/2272425)
 *
 * Parity status: every function here is pinned by the CPU tests (brute-force
 * direct sums, library conversions, closed-order evaluators, the RHD 5-rank
 * example, step counts and byte closed forms), except the intra-server
 * reduction order inside the pipeline, which the pages leave open; that order
 * is pinned only through its special cases (one server = left fold, one rank
 * per server = ring).
 */
#ifndef ALLREDUCE_ORACLE_H
#define ALLREDUCE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types, reduce ops, algorithms, collectives (numeric codes) */
enum { ORC_FP32 = 0, ORC_FP16 = 1, ORC_BF16 = 2, ORC_INT32 = 3, ORC_INT8 = 4 };
enum { ORC_SUM = 0, ORC_PROD = 1, ORC_MAX = 2, ORC_MIN = 3 };
enum { ORC_RING = 0, ORC_RHD = 1, ORC_PIPELINE = 2, ORC_FLAT = 3, ORC_TREE = 4, ORC_HIER = 5 };
enum { ORC_ALLREDUCE = 0, ORC_REDUCE_SCATTER = 1, ORC_ALL_GATHER = 2, ORC_ROOT_REDUCE = 3, ORC_BROADCAST = 4 };

/* action kinds of one step, as recorded in a trace */
enum {
  ORC_COPY = 0,      /* dst[range] <- received block                          */
  ORC_REDUCE = 1,    /* dst[range] <- op(received, dst[range])                */
  ORC_FOLD = 2,      /* dst[range] <- left fold of op over the source ranks   */
  ORC_FOLD_RECV = 3  /* dst[range] <- op(received, left fold over the peers)  */
};

/* return codes */
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_EUNSUPPORTED = -2, ORC_ENOMEM = -3, ORC_ECONFLICT = -4 };

/* One (action, source) pair of a step.  For FOLD_RECV slot 0 is the ring
 * receive and slots 1.. the intra-server sources in fold order. */
typedef struct {
  int32_t step, kind, dst, src, slot, pad;
  uint64_t begin, count;
} orc_trace_t;

/* IEEE 754 conversions, round to nearest even. */
uint16_t orc_f32_to_f16(float x);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
/* the same conversions over arrays (dtype ORC_FP16 or ORC_BF16) */
int orc_round_f32(int dtype, const float* in, uint16_t* out, size_t n);
int orc_widen(int dtype, const uint16_t* in, float* out, size_t n);

/* out[i] = a[i] (op) b[i] for n elements of type dtype. */
int orc_combine(int dtype, int op, const void* a, const void* b, void* out, size_t n);

/* Reduction by its definition: out[j] = op over ranks of srcs[r][j], computed
 * in binary64 for float types (fp_out) and in wrapping two's complement of the
 * element width for integer types (int_out). */
int orc_direct(int dtype, int op, int P, const void* const* srcs, size_t n, double* fp_out,
               int64_t* int_out);

/* Number of steps of a collective. */
long orc_num_steps(int coll, int algo, int P, int S, int M, size_t L, int dtype,
                   size_t loop_bytes);

/*
 * Replay a collective step by step on host buffers, in place.
 *   bufs[r] holds elements [w0, w1) of rank r's vector of L elements
 *   (w0 = 0, w1 = L replays everything); only steps with index in
 *   [first_step, last_step) run (pass 0, -1 for all); the trace, if given,
 *   receives up to trace_cap records and *trace_len the number produced.
 *   S, M describe the pipeline's (and the hierarchical AllReduce's) servers
 *   and ranks per server (S*M == P); for the tree M is the arity K (>= 2);
 *   loop_bytes is the pipeline's per-loop slice (0 selects 32 MiB); root is
 *   the root rank of Reduce and Broadcast (RHD only; others ignore it).
 */
int orc_collective(int coll, int algo, int P, int S, int M, size_t loop_bytes, int root,
                   void* const* bufs, size_t L, size_t w0, size_t w1, int dtype, int op,
                   long first_step, long last_step, orc_trace_t* trace, size_t trace_cap,
                   size_t* trace_len);

#ifdef __cplusplus
}
#endif
#endif
