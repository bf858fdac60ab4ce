// Internal interface between the C ABI (cc_api.cpp and the other host
// sources) and the kernels (cc_*.hip).  Host-side only; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cc {

enum Dt { DT_I32 = 0, DT_F32 = 1, DT_BF16 = 2 };
enum Op { OP_SUM = 0, OP_MAX = 1, OP_PROD = 2 };
enum Tree { TREE_HD = 0, TREE_BFLY = 1 };

inline int elem_size(int dt) { return dt == DT_BF16 ? 2 : 4; }
// elements per 16-byte vector
inline int vec_elems(int dt) { return 16 / elem_size(dt); }

constexpr int kBlock = 128;    // threads per workgroup of the reduction kernels (2 wavefronts)
constexpr int kUnroll = 1;     // 16-byte vectors per thread per tile
constexpr int kMaxDesc = 64;   // copy descriptors per launch
constexpr int kMaxRanks = 64;

// Occupancy: the kernels stream HBM with no reuse, and the DRAM serves a
// mixed read/write stream best when each CU keeps only a few tens of KiB of
// loads in flight.  A launch caps the workgroups per CU by reserving dynamic
// LDS (the kernels do not use it); blocks_per_cu = 0 picks the default.
// dynamic LDS bytes that limit a launch to `blocks` workgroups per CU
unsigned lds_for_blocks_per_cu(int blocks);
// default cap for a kernel moving `traffic` bytes per workgroup, aiming at
// `target` bytes in flight per CU, at least `min_blocks`
int default_blocks_per_cu(uint64_t traffic, uint64_t target, int min_blocks);

// The launch guard's refusal (cc_device.h): the launch returns
// hipErrorInvalidConfiguration and the API call reports CC_ERR_UNSUPPORTED
// with this text.
void refuse_launch(const char* why);

// Rank-strided view: rank r at base + r * stride (bytes).
struct Side {
  char* base;
  uint64_t stride;
};

// One reduction launch over the full per-rank vector of M elements, split in
// N chunks [floor(c*M/N), floor((c+1)*M/N)).
struct Red {
  Side send;
  Side recv;
  Side ws;        // staging (accumulator type, 4 bytes per element), or {nullptr,0}
  uint64_t M;
  const uint64_t* bnd;  // host array of N+1 chunk boundaries floor(c*M/N)
  int blocks_per_cu;    // occupancy cap (0 = default)
  int N;
  int dt;
  int op;
  int rs_mode;    // 0: AllReduce output on every rank; 1: ReduceScatter output (chunk c on rank c)
  int vec_ok;     // all addresses of the 16-byte path are 16-byte aligned
  hipStream_t st;
};

// Tiles of kBlock*kUnroll vectors.
inline uint64_t num_tiles(uint64_t M, int dt) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * vec_elems(dt);
  return (M + tile - 1) / tile;
}

// ---- reductions
hipError_t launch_ring_fused(const Red& r);
hipError_t launch_tree_fused(const Red& r, int tree);
// ring ReduceScatter steps [s0, s0+k); partial_in_recv: partials stay in the
// receiving rank's recv buffer (AllReduce, int32/fp32), else in r.ws.
hipError_t launch_ring_rs_pass(const Red& r, int s0, int k, int partial_in_recv);
// the ring AllReduce as passes of k steps in one launch, every tile of a pass
// waiting for all tiles of the previous one; bar: kQueueWords device words
// (cleared by a kernel first).
constexpr int kQueueWords = 2 + 2 * (kMaxRanks - 1);
hipError_t launch_ring_queue(const Red& r, int k, unsigned* bar);
// halving step with distance d; acc_in_recv as above (else r.ws is rank-strided).
hipError_t launch_hd_rs_step(const Red& r, int d, int first, int last, int acc_in_recv);
// butterfly step with distance d.
hipError_t launch_bfly_step(const Red& r, int d, int first, int last, int acc_in_recv);

// ---- tree-shaped fused AllReduces for schedules beyond the power-of-two ones
// binomial tree (TREE_BFLY order over `leaves` = N of NR = 2^ceil(log2 N)
// slots), and halving-doubling / butterfly for N not a power of two (NR = m =
// 2^floor(log2 N) leaves, the first `pairs` = N - m of them pair folds)
hipError_t launch_tree_shaped(const Red& r, int tree, int nr, int leaves, int pairs);
// double binary tree (N <= 16) and 2-port ring (any N)
hipError_t launch_dbt_fused(const Red& r);
hipError_t launch_ring2_fused(const Red& r);

// ---- hierarchical AllReduce, fused: nd (<= kMaxHierLevels) non-trivial
// levels of sizes p[] and rank strides stride[], level `top` running the
// AllReduce (nd: none); segbnd[0..N] bounds the N segments of the vector,
// seg[s] their chunk index per level (8 bits each)
constexpr int kMaxHierLevels = 4;
hipError_t launch_hier_fused(const Red& r, const int* p, const int* stride, int nd, int top, const uint64_t* segbnd,
                             const uint32_t* seg);

// ---- INT8 compression with error feedback: blocks of kQBlock elements of a
// rank's vector, one float32 scale each.  g: gradients (dt), e: float32 error
// accumulators, q: int8 values, s: float32 scales, r: results (dt).  The
// reductions fold each element in the ring order of its chunk
// [floor(c M / N), floor((c+1) M / N)).
constexpr int kQBlock = 128;
struct QLaunch {
  const char* g;
  uint64_t gs;
  char* e;
  uint64_t es;
  char* q;
  uint64_t qs;
  char* s;
  uint64_t ss;
  char* r;
  uint64_t rs;
  uint64_t M;
  int N;
  int dt;  // DT_F32 or DT_BF16
  int vec_ok;
  int blocks_per_cu;
  hipStream_t st;
};
hipError_t launch_quant_ef(const QLaunch& L);        // g, e -> e, q, s
hipError_t launch_dequant_reduce(const QLaunch& L);  // q, s -> r
hipError_t launch_quant_ef_fused(const QLaunch& L);  // g, e -> e, r

// ---- descriptor steps (GDesc flags)
enum : unsigned {
  GD_LOCAL_SEND = 1u,   // local operand from send[dst] (else partial[dst])
  GD_IN1 = 2u,          // combine with in1
  GD_IN1_SEND = 4u,     // in1 from send (else partial)
  GD_IN2 = 8u,          // combine with in2 after in1
  GD_IN2_SEND = 16u,
  GD_FINAL = 32u,       // write the rounded result to recv[dst] (else partial[dst])
  GD_BOTH = 64u,        // also store the result for rank in1
  GD_COPY = 128u,       // recv[dst] = recv[in1], no arithmetic
};
struct GDesc {
  uint64_t lo;
  uint64_t len;
  int dst;
  int in1;
  int in2;
  unsigned flags;
};
constexpr int kMaxGDesc = 64;
// one step: descriptors whose destination ranges do not overlap; partials in
// r.ws (fp32, rank-strided) when it is set, else in recv
hipError_t launch_gsteps(const Red& r, const GDesc* d, int n);

// ---- bucketed AllReduce: up to kMaxSeg independent fused AllReduces over
// element ranges [off, off+len) of the same rank buffers, in one launch.
constexpr int kMaxSeg = 16;
constexpr int kMaxSegRanks = 16;
struct SegLaunch {
  Side send;
  Side recv;
  int N;
  int dt;
  int op;
  int alg;          // 0 ring, 1 halving-doubling, 2 butterfly
  int blocks_per_cu;
  int nseg;
  uint64_t off[kMaxSeg];
  uint64_t len[kMaxSeg];   // each < 2^31
  hipStream_t st;
};
hipError_t launch_fused_seg(const SegLaunch& s);

// ---- gathers (no arithmetic).  ag_mode 0: AllGather phase of an AllReduce,
// everything in recv; 1: standalone AllGather, rank c's shard in send.
struct Gat {
  Side send;
  Side recv;
  uint64_t M;     // full per-rank vector (recv) length
  const uint64_t* bnd;  // host array of N+1 chunk boundaries
  int blocks_per_cu;
  int N;
  int esize;      // bytes per element
  int ag_mode;
  int vec_ok;
  hipStream_t st;
};
hipError_t launch_ag_fused(const Gat& g);
hipError_t launch_ring_ag_pass(const Gat& g, int s0, int k);
hipError_t launch_hd_ag_step(const Gat& g, int d, int first);

// ---- broadcast: one source to N rank buffers (skip < 0: write all)
hipError_t launch_bcast(const char* src, Side dst, int N, int skip, uint64_t nbytes, int vec_ok,
                        int blocks_per_cu, hipStream_t st);

// ---- descriptor copy: up to kMaxDesc (src, dst, bytes) copies in one launch;
// a NULL src fills dst with zero bytes
struct CopyDesc {
  const char* src;
  char* dst;
  uint64_t bytes;
};
hipError_t launch_copies(const CopyDesc* d, int n, int esize, int blocks_per_cu, hipStream_t st);

}  // namespace cc
