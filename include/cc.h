/*
 * cc.h -- C ABI of the collective-reduction engine (libcc.so).
 *
 * N logical ranks live in one GPU's HBM as rank-strided buffers: rank r's
 * buffer starts at  base + r * rank_stride_bytes.  One call carries all N
 * ranks' buffers and performs the whole collective on the caller's HIP stream.
 *
 * The calls follow the primitive table of the slide deck "集合通信与分片矩阵乘法"
 * (slide "I · 原语 · 小结": Broadcast, AllReduce, AllGather, ReduceScatter,
 * AllToAll) and the schedules of the "AllReduce" algorithm notes (算法一 Ring,
 * 算法二 Recursive Halving-Doubling, 算法四 Butterfly).
 *
 * Common rules for every collective call:
 *  - Asynchronous: the call validates, enqueues kernels on `stream` (a
 *    hipStream_t; NULL is the null stream) and returns.  Completion is stream
 *    order, as for the pages' asynchronous collective kernels (slide "NCCL：
 *    GPU 上用的那个库").
 *  - No call allocates device memory.  A schedule that needs staging (see
 *    cc_workspace_size) reads it from cfg->workspace, owned by the caller.
 *  - The caller owns every buffer; the library keeps no pointer after return.
 *  - Element types: CC_INT32 (SUM and PROD wrap modulo 2^32), CC_FLOAT32 and
 *    CC_BFLOAT16.  bf16 is read, widened to fp32, every partial result stays
 *    fp32 through all steps, and the final value is rounded once to bf16
 *    (nearest, ties to even).
 *  - Float MAX is IEEE-754-2019 maximum (NaN if either operand is NaN; +0 is
 *    larger than -0), so it is order-free.  fp32/bf16 SUM and PROD follow the
 *    chosen schedule's association exactly (the textbook ch. 6 "集合通信",
 *    section "六种核心原语": reduction order changes the low bits).
 *  - Chunks: a rank's vector of M elements is cut into N contiguous chunks,
 *    chunk c = [floor(c*M/N), floor((c+1)*M/N)).
 *  - Alignment: bases and strides that are not 16-byte multiples are legal;
 *    they run a slower element-wise path.
 *  - Errors are returned, never raised: CC_ERR_INVALID_ARG for bad arguments
 *    (nranks outside [1, CC_MAX_RANKS], NULL base with a non-zero count,
 *    rank buffers that overlap each other, send and recv buffers that overlap
 *    where the call needs them disjoint, root outside [0, N), a workspace
 *    smaller than cc_workspace_size reports, negative fuse_depth or
 *    blocks_per_cu),
 *    CC_ERR_UNSUPPORTED for a schedule the collective does not have,
 *    CC_ERR_NO_DEVICE when no GPU is visible, CC_ERR_HIP for a launch error.
 *    Every enum below spans the whole int range (its *_MAX_ENUM member), so
 *    any int a C caller passes is a value of the type and is validated.
 *    cc_last_error() returns a message for the last failing call on the
 *    calling thread.
 */
#ifndef CC_H_
#define CC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CC_MAX_RANKS 64

typedef enum {
  CC_OK = 0,
  CC_ERR_INVALID_ARG = 1,
  CC_ERR_UNSUPPORTED = 2,
  CC_ERR_NO_DEVICE = 3,
  CC_ERR_HIP = 4,
  CC_STATUS_MAX_ENUM = 0x7fffffff
} cc_status_t;

typedef enum { CC_INT32 = 0, CC_FLOAT32 = 1, CC_BFLOAT16 = 2, CC_DTYPE_MAX_ENUM = 0x7fffffff } cc_dtype_t;

/* Elementwise operators named by the course lesson "第 3 课：分布式通信原语"
 * (核心概念, item 1: SUM, MAX, PROD). */
typedef enum { CC_SUM = 0, CC_MAX = 1, CC_PROD = 2, CC_OP_MAX_ENUM = 0x7fffffff } cc_op_t;

/* Schedules.  Only CC_ALGO_RING and CC_ALGO_HALVING_DOUBLING (N = 2^k) serve
 * ReduceScatter and AllGather; broadcast takes ring (chain) and
 * halving-doubling (binomial doubling); AllToAll the ring (pairwise) only.
 * Every schedule serves AllReduce, for any N:
 *   HALVING_DOUBLING, BUTTERFLY with N not a power of two fold ranks
 *     (2i, 2i+1), i < r = N - 2^floor(log2 N), into 2i first and copy the
 *     result back last (AllReduce notes, 算法二 "非 2^k 处理", 算法四; blog
 *     "分布式大模型集合通信", RHD "非 2 的整数次幂场景");
 *   TREE: binomial reduce to rank 0 (rank i with i mod 2d = d sends to i-d at
 *     distance d = 1, 2, 4 ...), broadcast back (textbook ch. 6, "Tree
 *     AllReduce");
 *   DOUBLE_TREE: elements [0, M/2) on tree T1, the rest on T2 -- T1 the
 *     in-order binary tree over ranks 1..N-1 under rank 0, T2 the same with
 *     ranks renamed x+1 mod N, complementary leaves for N = 2^k (AllReduce
 *     notes, 算法三; textbook ch. 6, "双二叉树"); a node folds
 *     op(op(own, left child), right child);
 *   RING_2PORT: chunk c folded toward rank c by a clockwise chain over the
 *     N/2 ranks before it and a counter-clockwise chain over the (N-1)/2 ranks
 *     after it, op(op(x_c, cw), ccw) (AllReduce notes, "2-port Ring 优化"). */
typedef enum {
  CC_ALGO_RING = 0,             /* AllReduce notes, 算法一 */
  CC_ALGO_HALVING_DOUBLING = 1, /* AllReduce notes, 算法二 */
  CC_ALGO_BUTTERFLY = 2,        /* AllReduce notes, 算法四; AllReduce only */
  CC_ALGO_TREE = 3,             /* AllReduce only */
  CC_ALGO_DOUBLE_TREE = 4,      /* AllReduce only */
  CC_ALGO_RING_2PORT = 5,       /* AllReduce only */
  CC_ALGO_MAX_ENUM = 0x7fffffff
} cc_algo_t;

typedef enum {
  CC_COLL_ALL_REDUCE = 0,
  CC_COLL_REDUCE_SCATTER = 1,
  CC_COLL_ALL_GATHER = 2,
  CC_COLL_BROADCAST = 3,
  CC_COLL_ALL_TO_ALL = 4,
  CC_COLL_MAX_ENUM = 0x7fffffff
} cc_coll_t;

/* How a schedule is executed.
 *  fuse_depth = 0: fully fused -- one kernel folds every rank's contribution
 *                  in registers in the schedule's order and writes the result
 *                  to every destination (read N*M, write N*M for AllReduce).
 *                  The ring AllReduce from 32 ranks of 16 MiB runs its two
 *                  phases as two such kernels instead: each chunk's whole
 *                  fold stored to its owner, then the owners' chunks copied
 *                  to the other ranks (the same bits, M more elements read;
 *                  faster there).
 *  fuse_depth = 1: stepwise -- one kernel per schedule step, each doing the
 *                  step's reads, combines and writes in HBM.
 *  fuse_depth = k: ring only -- k consecutive ring steps per kernel (other
 *                  schedules treat k > 1 as 1).  The fused DOUBLE_TREE
 *                  kernel holds every rank's vector in registers and serves
 *                  N <= 16; beyond that its stepwise schedule runs (same
 *                  bits, and the stepwise workspace).
 *  workspace / workspace_bytes: caller-owned device memory, at least what
 *  cc_workspace_size returns for the same arguments (may be NULL/0 when that
 *  is 0).
 *  blocks_per_cu: cap on resident workgroups per compute unit (occupancy) for
 *  the call's kernels; 0 lets the library choose (it keeps a few tens of KiB
 *  of loads in flight per CU, which streams HBM best).  Negative is invalid.
 *  grid_sync (0 or 1): ring AllReduce with fuse_depth >= 1 only (any other
 *  collective or schedule returns CC_ERR_UNSUPPORTED).  The passes of
 *  fuse_depth ring steps run in ONE kernel launch instead of one launch per
 *  pass: workgroups take tiles from an ordered queue, and no tile of a pass
 *  starts before every tile of the previous pass is complete -- the
 *  step-by-step synchronisation of the ring (textbook ch. 6, Ring AllReduce;
 *  AllReduce notes, 算法一) as a grid-wide barrier.  It needs no co-resident
 *  grid.  Results are bit-identical to grid_sync = 0.  The workspace then
 *  starts with 512 bytes of queue words (included in cc_workspace_size; must
 *  be 16-byte aligned), which the call clears with a kernel before the
 *  launch.  A wait gives up after 2 s: the uint32 at byte offset 4 of the
 *  workspace is then 1 (the results are undefined) and the kernel still
 *  ends; it reads 0 after a good call.
 *  A NULL cfg means {CC_ALGO_RING, 0, NULL, 0, 0, 0}. */
typedef struct {
  cc_algo_t algo;
  int fuse_depth;
  void* workspace;
  size_t workspace_bytes;
  int blocks_per_cu;
  int grid_sync;
} cc_config_t;

/* N rank buffers: rank r at (char*)base + r * rank_stride_bytes (device memory).
 * Any stride at least the payload works (unaligned ones take the element-wise
 * path).  On MI355X the stride also sets how the ranks' equal offsets spread
 * over the HBM channels.  Rows a multiple of 2 MiB or of 512 MiB apart can
 * land on the same channels and lose up to a quarter of the bandwidth, and
 * so can pads that make N x pad a multiple of 16 MiB (64 ranks of 32 MiB
 * padded by 256 KiB lose a third).  A stride of P + max(32 KiB, P / 1024), P
 * the payload rounded up to a power of two, measured best or within 1-2% of
 * the best pad tried for 8 ranks of 256 MiB (256 MiB + 256 KiB), 16 of
 * 128 MiB, 32 of 64 MiB and 8 bf16 ranks of 527 MiB (1 GiB + 1 MiB: 6.35
 * TB/s against 5.82 with no padding).  For P of 4 to 32 MiB that pad (32
 * KiB) is poor, and P + 1 MiB measured best or within 6% of the best pad
 * tried (32 KiB to 2.25 MiB) at 4 to 64 ranks (fp32 AllReduce: 8 ranks of
 * 16 MiB 5.80 TB/s against 3.57 with 32 KiB, 64 of 32 MiB 6.18 against
 * 6.06); pads of 1/128 of the row were slow at every row size tried.  The
 * library takes the stride as given. */
typedef struct {
  void* base;
  size_t rank_stride_bytes;
} cc_rankbuf_t;

/* hipStream_t, passed as an opaque pointer. */
typedef void* cc_stream_t;

/* AllReduce: every rank's recv = (+) over ranks of send, `count` elements per
 * rank (slides "Reduce 与 AllReduce"; AllReduce notes, 语义与分解).  In place
 * iff send.base == recv.base with equal strides; otherwise the send and recv
 * rank buffers must not overlap.  Schedules: ring, halving-doubling, butterfly. */
cc_status_t cc_all_reduce(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                          cc_op_t op, int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* cc_all_reduce for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same collective, schedules, bits and errors as cc_all_reduce, but the
 * staging a schedule needs (cc_workspace_size: the queue words of grid_sync,
 * the fp32 partials of bf16 stepwise schedules) comes from a fixed array of
 * CC_NOALLOC_SCRATCH_BYTES inside the library instead of cfg->workspace.
 * Each GPU the library runs on holds its own copy of that array until the
 * process ends; the call itself allocates nothing.  cfg->workspace must be
 * NULL and cfg->workspace_bytes 0 (CC_ERR_INVALID_ARG otherwise); a schedule
 * needing more than CC_NOALLOC_SCRATCH_BYTES returns CC_ERR_INVALID_ARG
 * (cc_all_reduce with a workspace serves it).  Every call on one GPU shares
 * that GPU's array and the array keeps the last call's contents (the kernels
 * clear what must start at zero): calls that overlap in time on one GPU --
 * on different streams, or from different threads -- race and give undefined
 * results.  Schedules that need no staging (every fused schedule) never touch
 * the array. */
#define CC_NOALLOC_SCRATCH_BYTES (16u << 20)
cc_status_t cc_all_reduce_noalloc(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                                  cc_op_t op, int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* ReduceScatter: send holds nranks*recvcount elements per rank; rank r's recv
 * (recvcount elements) gets the reduction of chunk r over all ranks (slides
 * "Scatter 与 ReduceScatter").  send and recv must not overlap.  Schedules:
 * ring (each chunk's fold starts at the rank after its owner and ends at the
 * owner), halving-doubling. */
cc_status_t cc_reduce_scatter(cc_rankbuf_t send, cc_rankbuf_t recv, size_t recvcount,
                              cc_dtype_t dtype, cc_op_t op, int nranks, const cc_config_t* cfg,
                              cc_stream_t stream);

/* AllGather: rank r's send (sendcount elements) lands in slot r of every
 * rank's recv (nranks*sendcount elements) (slides "Gather 与 AllGather").
 * No arithmetic.  send and recv must not overlap.  Schedules: ring,
 * halving-doubling. */
cc_status_t cc_all_gather(cc_rankbuf_t send, cc_rankbuf_t recv, size_t sendcount,
                          cc_dtype_t dtype, int nranks, const cc_config_t* cfg,
                          cc_stream_t stream);

/* Broadcast: every rank's recv = the root's send, `count` elements (slides
 * "Broadcast：一份数据发给所有人").  Only the root's send buffer is read.
 * In place iff send.base == recv.base with equal strides.  Schedules: ring
 * (chain root, root+1, ...), halving-doubling (binomial doubling from the
 * root, any N; blog "分布式大模型集合通信", RHD section's rank-0 example). */
cc_status_t cc_broadcast(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                         int root, int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* AllToAll(v): a blocked transpose (slides "AllToAll：分布式的转置").
 * counts: host array [nranks*nranks], counts[i*nranks + j] = rows rank i sends
 * to rank j; a row is elem_per_row elements.  Rank i's send buffer holds its
 * blocks for j = 0..N-1 back to back; rank j's recv buffer receives the blocks
 * from i = 0..N-1 back to back (displacements are the exclusive prefix sums).
 * Every recv buffer must fit within the recv stride and must not overlap any
 * send buffer.  Schedules: ring = the pairwise schedule (blog, "Pairwise（成对）
 * 算法": at step k rank i sends to i+k) when fuse_depth >= 1; fused direct copy
 * when fuse_depth = 0. */
cc_status_t cc_all_to_all(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts,
                          size_t elem_per_row, cc_dtype_t dtype, int nranks,
                          const cc_config_t* cfg, cc_stream_t stream);

/* Bucketed AllReduce (textbook ch. 6, "Bucket fusion": gradients grouped into
 * buckets, one AllReduce per bucket).  Bucket b is the element range
 * [offsets[b], offsets[b] + counts[b]) of every rank's buffer; each bucket is
 * all-reduced on its own, with its own N chunks, exactly as cc_all_reduce on
 * that range would do (same bits).  Buckets must not overlap; empty buckets
 * are skipped.  The fused schedules (fuse_depth 0) with nranks <= 16 run up
 * to 16 buckets per kernel launch; otherwise each bucket runs as its own
 * cc_all_reduce.  A stepwise schedule's workspace is sized by
 * cc_workspace_size(CC_COLL_ALL_REDUCE, ..., largest bucket count, ...).
 * offsets and counts are host arrays of nbuckets entries.  Errors as for
 * cc_all_reduce, plus CC_ERR_INVALID_ARG for overlapping buckets or a bucket
 * beyond the rank stride. */
cc_status_t cc_all_reduce_buckets(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* offsets,
                                  const size_t* counts, int nbuckets, cc_dtype_t dtype, cc_op_t op,
                                  int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* Host-side bucket plan for cc_all_reduce_buckets (textbook ch. 6, "Bucket
 * fusion": parameters in reverse forward order, buckets of about 25 MB).
 * Tensors t = ntensors-1 .. 0 are packed greedily: a bucket is closed when
 * the next tensor would push it past cap_bytes, a tensor larger than the cap
 * gets a bucket of its own; tensors sit back to back inside a bucket, and
 * each bucket starts at a multiple of align_elems elements.  Outputs (host
 * arrays the caller owns, each with room for ntensors entries):
 * bucket_of[t], tensor_offset[t] (element offset in the per-rank flat
 * buffer), bucket_offset[b], bucket_count[b], and *nbuckets.  No device work. */
cc_status_t cc_bucket_plan(const size_t* sizes, int ntensors, size_t elem_bytes, size_t cap_bytes,
                           size_t align_elems, int* bucket_of, size_t* tensor_offset,
                           size_t* bucket_offset, size_t* bucket_count, int* nbuckets);

/* Bytes of caller-owned device workspace the given collective needs.  count is
 * the per-rank element count of the collective's own count argument. */
cc_status_t cc_workspace_size(cc_coll_t coll, const cc_config_t* cfg, int nranks, size_t count,
                              cc_dtype_t dtype, size_t* bytes);

/* Simulated-network accounting of a schedule: the largest number of bytes any
 * rank sends, and the number of communication steps.  Ring AllReduce sends
 * 2(N-1)M/N elements per rank when N divides M (textbook ch. 6, Ring
 * AllReduce; lesson 3 simulator's per-rank counter).  count is the per-rank
 * count of the collective (all_reduce, broadcast: the vector; reduce_scatter:
 * recvcount; all_gather: sendcount; all_to_all: elements per source-destination
 * block of a uniform exchange, sent over the pairwise schedule). */
cc_status_t cc_get_traffic(cc_coll_t coll, cc_algo_t algo, int nranks, size_t count,
                           cc_dtype_t dtype, uint64_t* max_bytes_sent_per_rank, int* steps);

/* The chunk boundaries used by every schedule: bounds[c] = floor(c*count/nranks),
 * c = 0..nranks (bounds must hold nranks+1 entries). */
cc_status_t cc_chunk_bounds(size_t count, int nranks, size_t* bounds);

/* Introspection of the stepwise AllReduce schedules that run as descriptor
 * steps -- TREE, DOUBLE_TREE, RING_2PORT, and HALVING_DOUBLING / BUTTERFLY
 * with N not a power of two: the exact operations the kernels perform, step
 * by step, so that a host program can replay them (tests do, against an
 * independent simulator).  One record per operation on elements
 * [lo, lo+len) of the named ranks:
 *   CC_PLAN_COPY:  out[dst] = out[in1]                 (finished values)
 *   otherwise:     v = local; if IN1: v = op(v, in1); if IN2: v = op(v, in2)
 *                  local = send[dst] if LOCAL_SEND else partial[dst];
 *                  in1 / in2 = send of the rank if *_SEND else its partial;
 *                  v -> out[dst] rounded if FINAL, else -> partial[dst];
 *                  BOTH: the same value also for rank in1.
 * Operations of one step read nothing another operation of that step
 * writes.  out is cc_all_reduce's recv; partials are fp32/int32 values per
 * rank and element.  With records == NULL only *nrecords is set; otherwise
 * cap must hold all of them (CC_ERR_INVALID_ARG if not).  CC_ERR_UNSUPPORTED
 * for the schedules with kernels of their own (ring; halving-doubling and
 * butterfly with N = 2^k) and for nranks < 2. */
#define CC_PLAN_LOCAL_SEND 1u
#define CC_PLAN_IN1 2u
#define CC_PLAN_IN1_SEND 4u
#define CC_PLAN_IN2 8u
#define CC_PLAN_IN2_SEND 16u
#define CC_PLAN_FINAL 32u
#define CC_PLAN_BOTH 64u
#define CC_PLAN_COPY 128u
typedef struct {
  uint32_t step;
  uint32_t flags;
  int32_t dst;
  int32_t in1;
  int32_t in2;
  uint64_t lo;
  uint64_t len;
} cc_plan_op_t;
cc_status_t cc_all_reduce_plan(cc_algo_t algo, int nranks, size_t count, cc_plan_op_t* records, size_t cap,
                               size_t* nrecords);

/* Hierarchical (multi-dimensional) AllReduce (AllReduce notes, 算法五
 * "多维分层 AllReduce" and its BlueConnect example; textbook ch. 6,
 * "分层全归约": ReduceScatter inside the node, AllReduce across nodes among
 * the ranks holding the same shard, AllGather inside the node).
 * The N = dims[0] * ... * dims[ndims-1] ranks form a grid, rank
 * r = r_0 + dims[0] (r_1 + dims[1] (r_2 + ...)), level 0 the innermost (the
 * fastest network tier).  A group of level i is the dims[i] ranks that
 * differ only in coordinate i.  Levels 0 .. ndims-2 run standalone ring
 * ReduceScatters inside their groups: the member with coordinate c keeps
 * chunk c of the group's current range (the range split at floor bounds),
 * its fold starting one member after it.  The outermost level runs a ring
 * AllReduce (as cc_all_reduce, schedule ring) on the shard each rank then
 * holds, and ring AllGathers run back out, level ndims-2 first.  Each
 * receiving member folds op(own, incoming): along a group the chain is
 * op(next, partial).  Levels of size 1 do nothing; when
 * dims[ndims-1] == 1 no AllReduce runs and the AllGathers follow the
 * ReduceScatters.  bf16 partials stay fp32 and are rounded once.
 * ndims in 1..8, every dims[i] >= 1, the product in 1..CC_MAX_RANKS, at
 * most 4 levels of size > 1 (CC_ERR_UNSUPPORTED beyond).  cfg: algo must be
 * CC_ALGO_RING and grid_sync 0 (CC_ERR_UNSUPPORTED otherwise).
 *  fuse_depth = 0: one kernel folds every element's nested chains in
 *                  registers and writes every rank's result (from 32 ranks
 *                  of 4 MiB: writes it to the owner of the element's flat
 *                  ring chunk, and a second kernel copies it from there to
 *                  the other ranks; the same bits);
 *  fuse_depth >= 1: one kernel per ring step of the schedule, the groups of
 *                  a level side by side; partials live in recv (int32,
 *                  fp32) or in the workspace (bf16, fp32 per rank and
 *                  element: cc_hierarchical_workspace_size).
 * When the outermost level is the only one of size > 1, the call runs
 * cc_all_reduce's ring kernels (the same values; fuse_depth as there).
 * In place iff send.base == recv.base with equal strides; otherwise send and
 * recv must not overlap.  Errors as for cc_all_reduce. */
cc_status_t cc_all_reduce_hierarchical(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                                       cc_op_t op, int ndims, const int* dims, const cc_config_t* cfg,
                                       cc_stream_t stream);

/* Bytes of caller-owned device workspace cc_all_reduce_hierarchical needs
 * for these arguments. */
cc_status_t cc_hierarchical_workspace_size(int ndims, const int* dims, const cc_config_t* cfg, size_t count,
                                           cc_dtype_t dtype, size_t* bytes);

/* Simulated-network accounting of the hierarchical AllReduce, per level i
 * (host arrays of ndims entries): level_bytes[i] = the largest number of
 * bytes any rank sends inside its level-i group, level_steps[i] = the ring
 * steps of that level (2 (dims[i] - 1): ReduceScatter and AllGather, or the
 * AllReduce at the outermost level).  With N a multiple of every group's
 * chunking, rank traffic at level i is 2 (p_i - 1) / p_i of the data the
 * level works on: count / (dims[0] ... dims[i-1]) elements (the BlueConnect
 * per-level cost). */
cc_status_t cc_hierarchical_traffic(int ndims, const int* dims, size_t count, cc_dtype_t dtype,
                                    uint64_t* level_bytes, int* level_steps);

/* The stepwise hierarchical AllReduce as operation records, exactly as
 * cc_all_reduce_plan describes them (the records the fuse_depth >= 1 kernels
 * execute; also for a lone outermost level, whose ring kernels reach the
 * same values).  CC_ERR_UNSUPPORTED when the product of dims is 1. */
cc_status_t cc_hierarchical_plan(int ndims, const int* dims, size_t count, cc_plan_op_t* records, size_t cap,
                                 size_t* nrecords);

/* ---- AllToAll variants around MoE routing (textbook ch. 6, "MoE AllToAll 中的
 * 动态路由与专家负载失衡"; blog, "Pairwise（成对）算法").  Every variant is a
 * pure copy: results are bit-identical whatever the schedule.  cfg: algo must
 * be CC_ALGO_RING (CC_ERR_UNSUPPORTED otherwise); fuse_depth 0 runs every
 * transfer at once (direct), fuse_depth >= 1 the pairwise schedule (at step k
 * rank r sends to r + k) where stated. */

/* Expert capacity ceil(nranks * tokens * topk / nexperts * C) with the
 * capacity factor C = factor_num / factor_den, in exact integer arithmetic
 * (textbook ch. 6, "容量因子与有界分配").  With nranks = 1 it is the rows one
 * source may send to one expert, the block size of cc_moe_dispatch_padded. */
cc_status_t cc_moe_capacity(int nranks, size_t tokens, int topk, int nexperts, int factor_num, int factor_den,
                            size_t* capacity);

/* Capacity-padded MoE dispatch (textbook ch. 6, "容量因子与有界分配": fixed
 * expert buffers, rows beyond the capacity dropped, free slots padded so the
 * exchange is uniform).  counts: host array [nranks * nexperts], counts[i*E+e]
 * = rows source rank i routes to expert e; nexperts is a multiple of nranks and
 * expert e lives on rank e / (E/nranks) as local expert e % (E/nranks).
 * send (token side): rank i's rows sorted by expert, back to back.
 * recv (expert side): rank j holds, for source i = 0..N-1 and then local
 * expert l, a block of `capacity` rows: the first min(count, capacity) rows of
 * i's block for expert j*E/N + l, in order, then zero rows (E*capacity rows
 * per rank).  A row is elem_per_row elements.  send and recv must not overlap.
 * fuse_depth 0: direct, every (source, expert) block as one copy of its kept
 * rows and one zero fill of its free slots, 64 blocks per launch.
 * fuse_depth >= 1: pairwise, step k carries the blocks of the pairs (i, i+k). */
cc_status_t cc_moe_dispatch_padded(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts,
                                   size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                   const cc_config_t* cfg, cc_stream_t stream);

/* The combine exchange, the transpose of cc_moe_dispatch_padded: send is the
 * expert side (its layout), recv the token side (its layout); rank i gets back
 * the rows its dispatched rows occupied, and zero rows where a row was dropped.
 * fuse_depth >= 1: pairwise, step k carries expert rank j's blocks for rank
 * j + k. */
cc_status_t cc_moe_combine_padded(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts,
                                  size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                  const cc_config_t* cfg, cc_stream_t stream);

/* Hierarchical AllToAll(v) (textbook ch. 6, "分层 MoE 交换": aggregate inside
 * the node, exchange between nodes, distribute inside the node).  The nranks
 * ranks form nranks/local_size nodes of local_size ranks (rank r on node
 * r / local_size).  Same arguments and result as cc_all_to_all.  Phases:
 * (1) blocks between ranks of one node go to their destination, and rank
 * (n, l) moves its blocks for node n2 != n into the payload of the aggregator
 * (n, n2 mod local_size), ordered by source then destination local index;
 * (2) one transfer per ordered node pair, aggregator -> receiver
 * (n2, n mod local_size); (3) the receiver copies each block to its
 * destination.  Inter-node transfers fall from one per rank pair to one per
 * node pair.  The payloads are staged in the caller's workspace
 * (cc_all_to_all_hierarchical_workspace_size; 2 areas of the inter-node
 * bytes, each rounded up to 256); it must not overlap send or recv.
 * fuse_depth has no effect. */
cc_status_t cc_all_to_all_hierarchical(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts,
                                       size_t elem_per_row, cc_dtype_t dtype, int nranks, int local_size,
                                       const cc_config_t* cfg, cc_stream_t stream);
cc_status_t cc_all_to_all_hierarchical_workspace_size(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype,
                                                      int nranks, int local_size, size_t* bytes);

/* Accounting of an AllToAll(v) exchange (counts as cc_all_to_all), entry 0
 * the flat exchange, entries 1..3 the hierarchical phases (aggregate,
 * exchange, distribute) for the given local_size: transfers between
 * different ranks (a source's aggregated payload for one node counts once,
 * every other non-empty block once), their total bytes, and the most bytes
 * one rank sends.  Host arrays of 4 entries. */
cc_status_t cc_all_to_all_traffic(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                  int local_size, int* flows, uint64_t* total_bytes, uint64_t* max_rank_bytes);

/* The pairwise schedule's per-step bytes (blog, "Pairwise（成对）算法",
 * performance model T = (N-1) a + b * sum_k max_i n_(i,(i+k) mod N)): for
 * k = 0..N-1, step_max[k] = max over i of the bytes of block (i, i+k), and
 * step_total[k] their sum (step 0 is the local block).  Host arrays of
 * nranks entries. */
cc_status_t cc_all_to_all_step_bytes(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                     uint64_t* step_max, uint64_t* step_total);

/* The copies the AllToAll variants above perform, as plain records (tests
 * replay them on the host): for the given arguments -- validated exactly as
 * the call would -- every copy in launch order, step (or phase) by step.
 * src and dst are the byte addresses the kernels would touch (derived from
 * the rank buffers and workspace given; they are never dereferenced here);
 * src = 0 means "fill dst with zero bytes".  kind selects the call:
 * CC_A2A_MOE_DISPATCH / CC_A2A_MOE_COMBINE take counts [nranks*nexperts],
 * nexperts and capacity (local_size is ignored); CC_A2A_HIERARCHICAL takes
 * counts [nranks*nranks] and local_size (nexperts, capacity ignored).
 * With records == NULL only *nrecords is set; otherwise cap must hold all of
 * them (CC_ERR_INVALID_ARG if not). */
typedef enum {
  CC_A2A_MOE_DISPATCH = 1,
  CC_A2A_MOE_COMBINE = 2,
  CC_A2A_HIERARCHICAL = 3,
  CC_A2A_MAX_ENUM = 0x7fffffff
} cc_a2a_kind_t;
typedef struct {
  uint32_t step;
  uint32_t reserved;
  uint64_t src;
  uint64_t dst;
  uint64_t bytes;
} cc_copy_op_t;
cc_status_t cc_all_to_all_plan(cc_a2a_kind_t kind, cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts,
                               int nexperts, size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                               int local_size, const cc_config_t* cfg, cc_copy_op_t* records, size_t cap,
                               size_t* nrecords);

/* ---- Block-wise INT8 compression with error feedback (textbook ch. 6,
 * "量化：降低精度", "梯度通信的分块量化", "错误反馈与残差累积").
 * Per rank and per block of CC_QUANT_BLOCK consecutive elements of the rank's
 * vector (blocks from element 0, the last one possibly short), in float32,
 * one IEEE operation at a time:
 *   u = g + e;  s = max|u| / 127;  q = round-half-even(u / s) clamped to
 *   [-127, 127] (q = 0 when s = 0);  v = q * s;  e <- u - v.
 * g is the gradient (float32, or bf16 widened exactly), e a float32 error
 * accumulator the caller keeps from step to step (start it at zero).  The
 * message a rank would send is q (1 byte per element) plus the scales (one
 * float32 per block): count + 4 ceil(count / 128) bytes, 3.88x smaller than
 * float32.  The AllReduce of the compressed contributions sums the v of all
 * ranks in float32 in the ring AllReduce's order (chunk c's fold starts at
 * rank c) and gives every rank the sum (bf16: rounded once).  dtype is
 * CC_FLOAT32 or CC_BFLOAT16 (CC_ERR_UNSUPPORTED otherwise); cfg.algo must be
 * CC_ALGO_RING.  All buffers are rank-strided device memory. */
#define CC_QUANT_BLOCK 128

/* The compression step: reads grad, updates err, writes q (int8, count per
 * rank) and scales (float32, ceil(count/128) per rank).  No two of the four
 * may overlap. */
cc_status_t cc_quantize_ef(cc_rankbuf_t grad, cc_rankbuf_t err, cc_rankbuf_t q, cc_rankbuf_t scales, size_t count,
                           cc_dtype_t dtype, int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* The reduction side: recv (dtype) of every rank = the ring-order float32 sum
 * of the dequantized messages of all ranks.  recv must not overlap q or
 * scales. */
cc_status_t cc_all_reduce_dequant(cc_rankbuf_t q, cc_rankbuf_t scales, cc_rankbuf_t recv, size_t count,
                                  cc_dtype_t dtype, int nranks, const cc_config_t* cfg, cc_stream_t stream);

/* Compression with error feedback and the AllReduce of the compressed
 * contributions in one call: recv = the sum of every rank's v, err updated.
 * fuse_depth 0: one kernel, no message in memory; fuse_depth >= 1: the two
 * calls above, the message in the caller's workspace
 * (cc_int8_ef_workspace_size).  Same bits either way.  In place iff
 * grad.base == recv.base with equal strides; err overlaps neither. */
cc_status_t cc_all_reduce_int8_ef(cc_rankbuf_t grad, cc_rankbuf_t err, cc_rankbuf_t recv, size_t count,
                                  cc_dtype_t dtype, int nranks, const cc_config_t* cfg, cc_stream_t stream);
cc_status_t cc_int8_ef_workspace_size(const cc_config_t* cfg, int nranks, size_t count, cc_dtype_t dtype,
                                      size_t* bytes);
/* count + 4 ceil(count / CC_QUANT_BLOCK): the bytes of one rank's message. */
cc_status_t cc_int8_message_bytes(size_t count, size_t* bytes);

const char* cc_status_string(cc_status_t status);
const char* cc_last_error(void);
const char* cc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CC_H_ */
