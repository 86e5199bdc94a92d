/*
 * hbmcoll -- AllReduce dataflow of P logical ranks kept as P buffers in one
 * GPU's HBM (gfx950).  C ABI: plain pointers and sizes, no C++ or torch types.
 *
 * Pages cited (titles as printed):
 *   [RING-RHD]  "HCCL Ring AllReduce 与 Recursive Halving-Doubling 对比" (mhpn.cn/news/973985)
 *   [TOPO]      HCCL topology-aware routing article (hwcomputing.csdn.net)
 *   [RHD]       "HCCL RHD（Recursive Halving-Doubling）算法深度解析" (mhpn.cn/news/2258316)
 *   [PIPE]      "HCCL Pipeline分级流水算法深度解析：原理、时序编排与耗时模型" (lpnh.cn/news/2272425)
 *
 * Common rules for every call below:
 *   - Return HBMC_OK on success, otherwise an error code; outputs come back
 *     through out-parameters (the pages' result-code convention, [RING-RHD]
 *     section "Ascend950的AIVAICPU通信引擎与图模式", HcclGraphBuild listing).
 *   - Collectives are in place: bufs[r] is rank r's device buffer of `count`
 *     elements of `dtype` on the current device; the P buffers must not
 *     overlap and must be aligned to the element size.  Buffers whose 16-byte
 *     phases differ are accepted and take a slower element-wise path.
 *   - Collectives are asynchronous and ordered on `stream` (a hipStream_t;
 *     NULL is the default stream), like the pages' stream-ordered operations
 *     with wait/event completion ([TOPO] section "梯度同步与计算重叠").  They
 *     return after enqueueing; a device fault surfaces at the caller's next
 *     synchronisation of that stream.
 *   - The caller owns the buffers and the stream; the communicator owns its
 *     cached schedules and their device tables.  A communicator is not
 *     thread-safe; calls that overlap on one communicator from several host
 *     threads race.
 *   - The first call of a (collective, root, count, dtype) builds its schedule
 *     and uploads its device tables with hipMalloc and blocking copies (and
 *     so does the first call in the LDS or column form, and one after the
 *     column length changes; the tables of the earlier length are kept until
 *     hbmc_comm_destroy, so launches still queued and graphs built or
 *     captured before the change stay valid); later calls with the same
 *     shape only enqueue kernels.  Tables live on the device current at that first call: a
 *     communicator serves one device, and a call made with another device
 *     current returns HBMC_ERR_INVALID_ARG.  Cached schedules are kept until
 *     hbmc_comm_destroy.  A later call of a cached shape allocates, copies and
 *     synchronises nothing; it only enqueues kernels on `stream`, so a caller
 *     may capture it into a graph (the first call of a shape, and the first in
 *     a new launch form or column length, must not be made while capturing).
 * *   - count == 0 and P == 1 are valid and enqueue nothing.
 *   - No C++ exception leaves the library: a host allocation that fails while
 *     building schedules, tables or graphs returns HBMC_ERR_NOMEM, and the
 *     communicator (or graph) stays usable, with nothing half-built cached.
 */
#ifndef HBMCOLL_H
#define HBMCOLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hbmc_comm* hbmc_comm_t;

typedef enum {
  HBMC_OK = 0,
  HBMC_ERR_INVALID_ARG = 1, /* null / aliased / misaligned buffers, bad P, count*e overflow,
                               S*M != P, enum out of range, step range out of bounds      */
  HBMC_ERR_UNSUPPORTED = 2, /* collective not offered by the algorithm: Reduce / Broadcast
                               other than RHD; anything but AllReduce for Flat, tree,
                               hierarchical                                               */
  HBMC_ERR_HIP = 3,         /* a HIP call or kernel launch failed                          */
  HBMC_ERR_NOMEM = 4,       /* host or device allocation failed                            */
  HBMC_ERR_SCRATCH = 5      /* hbmc_allreduce_noalloc: the schedule's work-item table
                               exceeds the library's fixed device array                   */
} hbmc_status_t;

/* element types (the pages' HcclDataType) */
typedef enum { HBMC_FP32 = 0, HBMC_FP16 = 1, HBMC_BF16 = 2, HBMC_INT32 = 3, HBMC_INT8 = 4 } hbmc_dtype_t;

/* reduce ops (the pages' HcclReduceOp: addition, multiplication, maximum;
 * minimum added).  fp16/bf16 are widened to fp32, combined and rounded back to
 * nearest even after every operation; integers wrap; max/min order -0 below
 * +0 and return the canonical quiet NaN if either operand is NaN. */
typedef enum { HBMC_SUM = 0, HBMC_PROD = 1, HBMC_MAX = 2, HBMC_MIN = 3 } hbmc_op_t;

/* algorithms.  RING: [RING-RHD] "Ring AllReduce带宽最优的环形流水线".
 * RHD: [RHD] "算法描述" and Table 1 (non-power-of-two P merges the first 2r
 * ranks into r, r = P - 2^floor(log2 P), and restores them at the end).
 * PIPELINE: [PIPE] -- S servers x M ranks, inter-server ring, intra-server
 * full mesh, sliced into loops.  FLAT: every rank talks directly to rank 0,
 * which reduces and sends the result back ([TOPO] "AllReduce算法实现").
 * TREE: K-ary tree in heap order, reduce up then broadcast down, 2 x height
 * steps ([TOPO] "AllReduce算法实现").  HIER: S servers x M ranks,
 * intra-server reduce-scatter, inter-server ring AllReduce, intra-server
 * all-gather, not pipelined ([PIPE] "与其它分级算法的关系").  FLAT, TREE and
 * HIER offer AllReduce only.  AUTO: per call, the candidate schedule with
 * the least modelled time (see hbmc_comm_set_cost_model).  AUTO_RULES: per
 * call, the pages' default rules instead of the cost model: an AllReduce of
 * fewer than 64 KiB per rank takes Flat ([TOPO] "拓扑感知路由": below the
 * 64 KB threshold every device talks to the root directly); otherwise RHD
 * when P is a power of two and the ring when it is not ([RHD] "RHD 在 HCCL
 * 中的定位与启用方式": ring by default for a rank count that is not a power
 * of two, H-D_R otherwise); Reduce and Broadcast take RHD.  ENV: take the
 * algorithm from the environment variable HBMC_ALGO ("ring", "rhd" or
 * "H-D_R", "pipeline", "flat", "tree", "hier", "auto", "auto_rules"), the
 * way the pages' HCCL_ALGO selects an algorithm ([RHD] "RHD 在 HCCL 中的定位
 * 与启用方式"). */
typedef enum {
  HBMC_ALGO_RING = 0,
  HBMC_ALGO_RHD = 1,
  HBMC_ALGO_PIPELINE = 2,
  HBMC_ALGO_ENV = 3,
  HBMC_ALGO_FLAT = 4,
  HBMC_ALGO_TREE = 5,
  HBMC_ALGO_HIER = 6,
  HBMC_ALGO_AUTO = 7,
  HBMC_ALGO_AUTO_RULES = 8
} hbmc_algo_t;

typedef enum {
  HBMC_COLL_ALLREDUCE = 0,
  HBMC_COLL_REDUCE_SCATTER = 1,
  HBMC_COLL_ALL_GATHER = 2,
  HBMC_COLL_REDUCE = 3,    /* to a root; RHD only */
  HBMC_COLL_BROADCAST = 4  /* from a root; RHD only */
} hbmc_coll_t;

/*
 * Create a communicator of `nranks` logical ranks (1..64) using `algo`.
 * For HBMC_ALGO_PIPELINE and HBMC_ALGO_HIER, servers * ranks_per_server must
 * equal nranks; for the pipeline loop_bytes is the per-loop slice ([PIPE]
 * "源码中的流水执行印证": the executor slices the data into loops bounded by
 * its buffer limits), 0 selecting 32 MiB.  For HBMC_ALGO_TREE,
 * ranks_per_server is the arity K (2..64; 0 selects 2).  Other algorithms
 * ignore servers, ranks_per_server and loop_bytes.  Touches no device state.
 * *out receives the handle.
 */
hbmc_status_t hbmc_comm_create(int nranks, hbmc_algo_t algo, int servers, int ranks_per_server,
                               size_t loop_bytes, hbmc_comm_t* out);

/* Free the communicator and its device tables.  The caller must have
 * synchronised every stream that still runs one of its collectives. */
hbmc_status_t hbmc_comm_destroy(hbmc_comm_t comm);

/*
 * Launch forms.  Every form runs the same items with the same element ops in
 * the same order (bit-identical results); they differ in how the steps are
 * launched, which decides the fixed per-step cost ([RHD] "耗时计算": every
 * step pays alpha; [RING-RHD] "Ascend950的AIVAICPU通信引擎与图模式": short
 * messages pay mostly control overhead, which fewer launches remove):
 *  - HBMC_EXEC_STEPS: one kernel launch per non-empty step (stream order
 *    separates the steps);
 *  - HBMC_EXEC_FUSED: all steps of the call in one launch of a single
 *    1024-thread workgroup, a workgroup barrier between steps;
 *  - HBMC_EXEC_COLUMNS: all steps in one launch of the column kernel.  Steps
 *    combine operands at equal element offsets, so the elements of all rank
 *    buffers split into independent columns (column_bytes per rank buffer;
 *    0 chooses about four columns per compute unit, at least 1 KiB) and one
 *    wave runs a column's share of every step in schedule order, without
 *    waiting for other waves ([RING-RHD] "Ring AllReduce带宽最优的环形流水线":
 *    the ring pipelines segments so no one waits for a whole step);
 *  - HBMC_EXEC_LDS: all steps in one launch of the LDS-resident column
 *    kernel: one workgroup per column loads the column of every rank buffer
 *    into LDS once, runs every step on the LDS copies and writes back the
 *    rank buffers the steps wrote.  Each lane owns fixed 16-byte positions
 *    of the column for the whole launch, so steps need no barrier.  The
 *    column length is column_bytes when set, else chosen per call shape by
 *    the model below among 16 B, 32 B, ... lengths that fit LDS;
 *  - HBMC_EXEC_REGS: a whole call in one launch that keeps every operand
 *    in registers.  The schedule is replayed on the host over symbols: each
 *    element's final value on each rank is an expression over the P inputs
 *    at that element, in the schedule's grouping.  The form applies where,
 *    in every interval of elements, either every rank ends with the same
 *    expression and it is a left fold over the ranks (the ring's AllReduce:
 *    segment c folds ranks c+1, c+2, ..., c; Flat; small trees) or a
 *    complete pairwise tree whose leaves are single ranks or merged pairs
 *    (RHD's AllReduce, also with P not a power of two); or every rank ends
 *    with one rank's input (all-gathers of ring, RHD and pipeline, RHD's
 *    broadcast); or the ranks hold the prefixes of one left fold over all
 *    ranks (the ring's reduce-scatter, whose other segments keep the
 *    schedule's partial sums); or, for P a power of two, every rank keeps its
 *    input or holds a node of one pairwise tree above its own leaf (RHD's
 *    reduce-scatter and Reduce).  At most 16 folded terms, tree leaves or
 *    copies, and at most 16 (fold, copy, prefix, nodes) or 8 (tree)
 *    intervals of distinct parameters.  One lane per 16-byte position loads every
 *    operand once, evaluates the expression and stores every rank the
 *    schedule writes there ([RHD] "耗时计算": every step pays alpha, which
 *    this form pays once);
 *  - HBMC_EXEC_FLOW: a call, or a hbmc_run_steps range, in one launch of a
 *    persistent kernel
 *    that runs every step's work as the step kernels do (each step reads
 *    and writes its own bytes in the rank buffers) but lets consecutive steps
 *    overlap: items are cut into tiles at multiples of the tile length
 *    (hbmc_comm_set_flow), tiles are handed out step after step by an atomic
 *    ticket, and a tile waits until the tiles of earlier steps over its
 *    elements are done ([RING-RHD] "Ring AllReduce带宽最优的环形流水线": no
 *    rank waits for a whole step).  Only when set explicitly (AUTO does not
 *    pick it).  Launches of one communicator's call of the same collective,
 *    count, dtype and step range share that range's counters: they must not
 *    overlap in time (one stream, or ordered; graphs order such nodes
 *    themselves);
 *  - HBMC_EXEC_AUTO (default, or the environment variable HBMC_EXEC = auto,
 *    steps, fused, columns, lds, regs or flow): per call the eligible form of least
 *    modelled time, with constants measured on MI355X: steps sum over the
 *    steps max(4.2 us, 3 us + bytes / 6.4 TB/s); fused 2 us + 1.6 us per
 *    step + bytes / 33 GB/s; columns 4 us + 0.85 us per chunk of the longest
 *    column + bytes / 6 TB/s (bytes: the algorithmic HBM bytes of the
 *    steps); lds 4 us + R * H * N * 0.56 us + 2 P count e / 5 TB/s, with R
 *    the columns each workgroup runs one after another, H the serial chunk
 *    passes of the busiest column (a run of n same-range chunks of one step
 *    counting 1 + 0.75 (n - 1)) and N the 16-byte positions per lane.  REGS,
 *    where eligible, is taken before any other form: on MI355X it measured
 *    fastest, or within 11% of the fastest, in every case timed (rings, RHD
 *    and Flat of 3-16 ranks, 1 KiB-4 MiB per rank).
 * A forced form falls back to STEPS where it is not eligible.  Eligibility:
 * both one-launch forms need rank buffers of one 16-byte phase; FUSED needs
 * at most 256 items per step and at most `max_bytes` algorithmic bytes in
 * the call's steps (hbmc_comm_set_fused_limit; default 64 MiB, or the
 * environment variable HBMC_FUSED_LIMIT); COLUMNS needs two or more non-empty
 * steps and P * count * e (the rank buffers' total size) of at most
 * `max_total_bytes` (hbmc_comm_set_columns; default 64 MiB, or
 * HBMC_COLUMNS_LIMIT): working sets the caches hold, so that larger calls
 * keep the per-step HBM traffic the schedule defines; LDS needs what COLUMNS
 * needs, and a column of every rank buffer plus 160 bytes per chunk of the
 * longest column within one workgroup's LDS; REGS needs what COLUMNS needs,
 * all of the call's steps, and the expression forms above; FLOW needs rank
 * buffers of one 16-byte phase, two or more busy steps in the range and at
 * most 32 ranks per item.  The
 * element ops commute bit for bit, so every form gives the same bits.  The
 * forms apply to
 * every call, hbmc_run_steps ranges and graph nodes.  Host only.
 */
typedef enum {
  HBMC_EXEC_AUTO = 0, HBMC_EXEC_STEPS = 1, HBMC_EXEC_FUSED = 2, HBMC_EXEC_COLUMNS = 3, HBMC_EXEC_LDS = 4,
  HBMC_EXEC_REGS = 5, HBMC_EXEC_FLOW = 6
} hbmc_exec_t;
hbmc_status_t hbmc_comm_set_exec_mode(hbmc_comm_t comm, hbmc_exec_t mode);
hbmc_status_t hbmc_comm_set_fused_limit(hbmc_comm_t comm, uint64_t max_bytes);
/* The flow form's settings: tile_bytes per rank buffer (16 .. 2^31, rounded
 * down to a multiple of 16; default 16 KiB), workgroups per compute unit
 * (1 .. 64; default 8), tiles a workgroup takes per ticket (1 .. 4096,
 * consecutive in ticket order and run in order; default 1), and the bound on
 * each wait for an earlier tile in microseconds of the GPU's wall clock
 * (default 1 s).  A wait past the bound
 * gives up: the launch skips the rest of its tiles, ends normally, and the
 * communicator's timeout counter grows (hbmc_comm_flow_timeouts); the
 * buffers then hold a partial result.  flags: 0, or HBMC_FLOW_UNREACHABLE,
 * which makes every wait target a count its column never reaches, so that
 * every tile with an earlier tile gives up after the bound (a test of the
 * give-up path, forced from the host).  Host only. */
#define HBMC_FLOW_UNREACHABLE 1u
hbmc_status_t hbmc_comm_set_flow(hbmc_comm_t comm, uint64_t tile_bytes, uint32_t wgs_per_cu,
                                 uint32_t tiles_per_ticket, uint32_t wait_us, uint32_t flags);
/* The number of flow-form waits that gave up since the last call, over all
 * of the communicator's plans (each counts in its own device allocation),
 * then reset to 0 (waits for the device: call it after the launches in
 * question have completed). */
hbmc_status_t hbmc_comm_flow_timeouts(hbmc_comm_t comm, uint32_t* count);
/* column_bytes: 0, or 16 .. 2^31 (rounded down to a multiple of 16). */
hbmc_status_t hbmc_comm_set_columns(hbmc_comm_t comm, uint64_t max_total_bytes, uint64_t column_bytes);
/* The launch form steps [first_step, last_step) of a call would take (0, 0:
 * all steps), for rank buffers of one 16-byte phase (host only; builds the
 * plan and, for AUTO, its host column table). */
hbmc_status_t hbmc_exec_choice(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                               int first_step, int last_step, hbmc_exec_t* mode);
/* Bytes that steps [first_step, last_step) of a call (0, 0: all steps) move
 * between the compute units and memory in launch form `mode` (AUTO: the form
 * hbmc_exec_choice reports), host only:
 *  - STEPS, FLOW: the steps' algorithmic HBM bytes (every distinct block a
 *    step reads counted once, every block it writes once, step after step);
 *  - FUSED, COLUMNS: each rank's elements that some step reads, once, plus
 *    those some step writes, once -- what crosses to memory when the caches
 *    hold the call's working set, as they do within these forms' limits;
 *  - LDS: exactly what the kernel loads and stores: every column of every
 *    rank it loads, and every column range it stores (composed store
 *    records in a launch of all steps), for the column length the
 *    communicator would use;
 *  - REGS: every operand loaded once and every written rank stored once:
 *    2 P count e for an AllReduce, P count e for a copy (one load, P - 1
 *    stores), (2 P - 1) count e for the ring's reduce-scatter, (P + P/2)
 *    count e for RHD's reduce-scatter (P/2 ranks receive a node per
 *    element), counted region by region for RHD's Reduce.
 * HBMC_ERR_INVALID_ARG for a bad step range, for LDS when no column length
 * fits one workgroup's LDS, and for REGS when the call has no register form
 * or the range is not all of its steps.  Otherwise the figure does not
 * depend on whether the form is eligible for the call. */
hbmc_status_t hbmc_exec_bytes(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                              int first_step, int last_step, hbmc_exec_t mode, uint64_t* bytes);

/*
 * AUTO selection ([RHD] "RHD 在 HCCL 中的定位与启用方式": the algorithm is
 * chosen adaptively from product, data size and rank count; [RHD] "耗时计算"
 * and [TOPO] "AllReduce算法实现": alpha-beta cost models).  An AUTO
 * communicator's candidates are ring, RHD, Flat and a binary tree, plus the
 * pipeline and the hierarchical AllReduce when created with a server shape
 * (servers * ranks_per_server == nranks; 0, 0 for none).  For each
 * (collective, root, count, dtype) it builds every candidate's schedule and
 * keeps the one minimising launches * alpha + algorithmic HBM bytes / beta
 * (ties: fewer launches), caching the choice.  Defaults are this library's
 * measurements on MI355X: alpha = 4.4 us per step launch, beta = 6400 GB/s.
 * hbmc_comm_set_cost_model replaces alpha (us, >= 0) and beta (GB/s, > 0)
 * and forgets earlier choices (an AUTO_RULES communicator accepts it and
 * keeps its rules); hbmc_auto_choice reports the algorithm a call would use
 * (for any communicator: its own algorithm; for AUTO_RULES: the rules'
 * pick).  Host only.
 */
hbmc_status_t hbmc_comm_set_cost_model(hbmc_comm_t comm, double alpha_us, double beta_gbps);
hbmc_status_t hbmc_auto_choice(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                               hbmc_dtype_t dtype, hbmc_algo_t* algo);

/*
 * AllReduce, Y[j] = op over ranks i of X_i[j] ([RING-RHD] "AllReduce的数学抽象与问题定义").
 * On completion every bufs[r][0..count) holds Y, computed in the order the
 * communicator's schedule implies (bit-identical for every rank).
 */
hbmc_status_t hbmc_allreduce(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                             hbmc_op_t op, void* stream);

/*
 * AllReduce for callers that cannot allocate device memory (code that must
 * not call hipMalloc: under stream capture, in tight serving loops, in
 * harnesses that forbid it).  Same arguments, schedule, element ops and
 * results (bit for bit) as hbmc_allreduce, one step kernel per non-empty
 * step whatever the communicator's launch form; the step kernels read their
 * work items from a fixed device array of 2 MiB that the library holds on
 * every GPU it runs on until the process ends, not from memory it
 * allocates.  Each call copies its schedule's item table (160 bytes per
 * item) into that array with one host-to-device copy ordered on `stream`,
 * then enqueues its kernels; it calls no hipMalloc or hipFree and no
 * allocating library routine.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams, or
 * from several host threads) race and must be serialised by the caller;
 * calls on one stream follow each other safely.  The schedule's table must
 * fit the array (at most 13107 items: e.g. ring or RHD with up to 64 ranks,
 * the 4 x 8 pipeline with 32 MiB loops up to 1 GiB per rank), otherwise
 * HBMC_ERR_SCRATCH is returned before anything is enqueued.  The host
 * schedule is built and cached on the first call of a shape, as for
 * hbmc_allreduce.
 */
hbmc_status_t hbmc_allreduce_noalloc(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                                     hbmc_op_t op, void* stream);

/*
 * ReduceScatter.  The vector is split into P segments by the ceiling split
 * (segment k = [min(k q, count), min((k+1) q, count)), q = ceil(count / P),
 * [TOPO] "AllReduce算法实现"); for the pipeline each loop is split that way.
 * On completion bufs[r] holds Y on segment r (each loop's block r for the
 * pipeline); its other segments are unspecified.  RHD with P not a power of
 * two runs the three-part schedule of [RHD] Table 1 (Reduce, non-uniform
 * reduce-scatter over 2^floor(log2 P) virtual ranks, Scatter).
 */
hbmc_status_t hbmc_reduce_scatter(hbmc_comm_t comm, void* const bufs[], size_t count,
                                  hbmc_dtype_t dtype, hbmc_op_t op, void* stream);

/*
 * AllGather.  On entry bufs[r] holds rank r's contribution on segment r (as
 * reduce_scatter leaves it); on completion every buffer holds all segments.
 * `op` is validated but unused, so all three collectives share one signature.
 */
hbmc_status_t hbmc_all_gather(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                              hbmc_op_t op, void* stream);

/*
 * Reduce to `root` (0 <= root < P), RHD communicators only ([RHD] Table 1:
 * Reduce = ReduceScatter + Gather; for P not a power of two the pairs of
 * part1 first merge into the rank with the root's parity).  On completion
 * bufs[root] holds Y; the other buffers are unspecified.
 * HBMC_ERR_UNSUPPORTED for ring and pipeline communicators.
 */
hbmc_status_t hbmc_reduce(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                          hbmc_op_t op, int root, void* stream);

/*
 * Broadcast from `root`, RHD communicators only ([RHD] Table 1: the root's
 * parity picks the part1 ranks that join the 2^k block, distance halving
 * inside the block, then one more send to the remaining ranks).  On
 * completion every buffer holds bufs[root]'s contents.
 * HBMC_ERR_UNSUPPORTED for ring and pipeline communicators.
 */
hbmc_status_t hbmc_broadcast(hbmc_comm_t comm, void* const bufs[], size_t count, hbmc_dtype_t dtype,
                             int root, void* stream);

/*
 * Out-of-place form of every collective ([PIPE] "Rank0 视角的传输任务编排":
 * LocalCopy moves data from input to output memory only when the two differ
 * and is skipped in place).  send[r] holds rank r's input (count elements,
 * read only); on completion recv[r] holds what the in-place call would leave
 * in bufs[r].  Ranks with send[r] != recv[r] are first copied by one
 * LocalCopy launch per 32 such ranks, then the collective runs in place on
 * recv.  send[r] must equal recv[r] or overlap no recv buffer (else
 * HBMC_ERR_INVALID_ARG); send buffers are left unchanged.  `root` is used by
 * Reduce and Broadcast.  Asynchronous and stream-ordered like the others.
 */
hbmc_status_t hbmc_collective_oop(hbmc_comm_t comm, hbmc_coll_t coll, int root, const void* const send[],
                                  void* const recv[], size_t count, hbmc_dtype_t dtype, hbmc_op_t op,
                                  void* stream);

/*
 * Run only schedule steps [first_step, last_step) of a collective (every
 * loop's steps with those indices for the pipeline).  Running [0, k) and then
 * [k, nsteps) equals the whole collective.  For step-by-step checking and
 * per-step timing.  `root` is used by Reduce and Broadcast and ignored
 * otherwise (also in the plan and graph calls below).  Returns
 * HBMC_ERR_INVALID_ARG for an empty or out-of-range step interval.
 */
hbmc_status_t hbmc_run_steps(hbmc_comm_t comm, hbmc_coll_t coll, int root, void* const bufs[],
                             size_t count, hbmc_dtype_t dtype, hbmc_op_t op, int first_step,
                             int last_step, void* stream);

/*
 * Schedule facts, computed on the host without touching the device:
 * number of steps (launches), algorithmic HBM bytes of the whole collective
 * (every distinct block a step reads counted once, every block it writes
 * once), and the largest number of bytes any rank receives from other ranks.
 * Any out-pointer may be NULL.
 */
hbmc_status_t hbmc_plan_info(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                             hbmc_dtype_t dtype, int* nsteps, uint64_t* hbm_bytes,
                             uint64_t* max_recv_bytes);

/* The same for one step: its work items and algorithmic HBM bytes. */
hbmc_status_t hbmc_plan_step_info(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                                  hbmc_dtype_t dtype, int step, int* nitems, uint64_t* hbm_bytes);

/* One work item of a step: every destination rank's range
 * [begin, begin+count) receives, for mode COPY the source, for mode FOLD the
 * left fold of op over the sources in order, and for mode RECV_FOLD
 * op(source 0, left fold over sources 1..).  rank[0..nsrc) are the sources,
 * rank[nsrc..nsrc+ndst) the destinations. */
enum { HBMC_MODE_COPY = 0, HBMC_MODE_FOLD = 1, HBMC_MODE_RECV_FOLD = 2 };
typedef struct {
  int32_t step, mode, nsrc, ndst;
  uint64_t begin, count;
  uint8_t rank[128];
} hbmc_item_t;

/* Copy out every work item of a collective's schedule (host only).  Writes
 * at most `cap` items and sets *n_items to the total. */
hbmc_status_t hbmc_plan_items(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                              hbmc_dtype_t dtype, hbmc_item_t* out, size_t cap, size_t* n_items);

/* One chunk of the column kernel: elements [begin, begin+count) of work item
 * `item` (index in hbmc_plan_items order) of step `step`; it must follow the
 * chunks deps[dep_lo..dep_hi) (all of earlier steps, all in its column). */
typedef struct {
  uint64_t begin;
  uint32_t count, item, step, dep_lo, dep_hi, pad;
} hbmc_chunk_t;

/* The column kernel's chunk table for columns of chunk_bytes (rounded as
 * hbmc_comm_set_columns does; at least 16), host only: writes at most `cap`
 * chunks and `dcap` dependency indices, and sets *n_chunks / *n_deps to the
 * totals. */
hbmc_status_t hbmc_plan_chunks(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count,
                               hbmc_dtype_t dtype, uint64_t chunk_bytes, hbmc_chunk_t* chunks, size_t cap,
                               size_t* n_chunks, uint32_t* deps, size_t dcap, size_t* n_deps);

/* One tile of the flow kernel: the seq-th tile of column `col` (elements
 * [col * tile, (col + 1) * tile) of every rank buffer), the work of step
 * `step` there, chunks [c_lo, c_hi) of the chunk table; and one chunk:
 * elements [begin, begin+count) of work item `item` (hbmc_plan_items order). */
typedef struct {
  uint32_t col, seq, step, c_lo, c_hi, pad;
} hbmc_flow_tile_t;
typedef struct {
  uint64_t begin;
  uint32_t count, item;
} hbmc_flow_chunk_t;

/* The flow kernel's tables for steps [first_step, last_step) (last_step -1:
 * through the last step) and tiles of tile_bytes per rank buffer (rounded as
 * hbmc_comm_set_flow does), host only: tiles in the order the kernel hands
 * them out (step after step, columns ascending; seq counts within the
 * range), at most `cap` tiles and `ccap` chunks written, totals in *n_tiles /
 * *n_chunks.  HBMC_ERR_INVALID_ARG for a range outside the schedule;
 * HBMC_ERR_UNSUPPORTED when an item has more than 32 ranks. */
hbmc_status_t hbmc_plan_flow(hbmc_comm_t comm, hbmc_coll_t coll, int root, size_t count, hbmc_dtype_t dtype,
                             int first_step, int last_step, uint64_t tile_bytes, hbmc_flow_tile_t* tiles,
                             size_t cap, size_t* n_tiles, hbmc_flow_chunk_t* chunks, size_t ccap,
                             size_t* n_chunks);

/*
 * Graph mode ([RING-RHD] section "Ascend950的AIVAICPU通信引擎与图模式": a
 * sequence of collectives is composed into a graph whose data dependencies
 * are analysed at build time, then scheduled and launched as one unit).
 *
 * hbmc_graph_add appends a collective with its buffers fixed (same argument
 * rules as the direct calls; the schedule is built and checked here).  At
 * hbmc_graph_build every collective becomes a chain of kernel nodes, one per
 * schedule step; a collective starts after every earlier one whose rank
 * buffers overlap its own, and collectives on disjoint buffers may run
 * concurrently.  Build uploads the schedules' device tables and instantiates
 * the graph (it must not be called while the calling thread captures a
 * stream); no node can be added after it.
 * hbmc_graph_launch enqueues the whole graph on `stream` (asynchronous,
 * stream-ordered).  The communicators and buffers must outlive the graph.
 * Errors: HBMC_ERR_INVALID_ARG for adding after build, launching before
 * build, or a bad argument; the direct calls' codes otherwise.
 */
typedef struct hbmc_graph* hbmc_graph_t;
hbmc_status_t hbmc_graph_create(hbmc_graph_t* out);
hbmc_status_t hbmc_graph_add(hbmc_graph_t graph, hbmc_comm_t comm, hbmc_coll_t coll, int root,
                             void* const bufs[], size_t count, hbmc_dtype_t dtype, hbmc_op_t op);
hbmc_status_t hbmc_graph_build(hbmc_graph_t graph);
hbmc_status_t hbmc_graph_launch(hbmc_graph_t graph, void* stream);
hbmc_status_t hbmc_graph_destroy(hbmc_graph_t graph);

/* Static text for a status code. */
const char* hbmc_status_string(hbmc_status_t status);

#ifdef __cplusplus
}
#endif
#endif
