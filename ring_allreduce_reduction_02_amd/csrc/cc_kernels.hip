// Fused AllReduce / ReduceScatter kernels (gfx950 / CDNA4) of the
// collective-reduction engine: the ring and the power-of-two trees, whose
// whole schedule runs in one launch.  Other kernels live in cc_trees.hip,
// cc_steps.hip, cc_hier.hip, cc_copy.hip and cc_quant.hip; cc_device.h holds
// what they share.
//
// N logical ranks are rank-strided buffers in one GPU's HBM.  Every kernel
// gives one thread ownership of an element index e across all N ranks: it
// does every read, combine and write that the schedule step performs on e.
// So no step kernel can race with itself, in place or not, and steps are
// ordered by the stream.
//
// The work is streaming and elementwise (one combine per element and rank,
// a few per byte), so the bound is HBM bandwidth, not the ALUs or matrix
// cores: the kernels move 16-byte vectors per lane with nontemporal loads and
// stores, keep partial results in registers, and derive the chunk of a tile
// once per workgroup so that the rank addresses stay in scalar registers.
//
// Schedules (the "AllReduce" algorithm notes, 算法一/二/四; textbook ch. 6
// "集合通信", Ring AllReduce / Algorithm 1):
//  * ring: chunk c's ReduceScatter fold starts at rank c (c+1 for a standalone
//    ReduceScatter) and each step folds in the next rank as
//    acc = op(x_next, acc); the owner then forwards the result around the
//    ring (AllGather).
//  * halving-doubling: distance N/2 first; for every element the fold tree
//    pairs ranks that differ in the top bit, then the next bit, ...
//  * butterfly: distance 1 first; the tree pairs neighbours 2j, 2j+1 first.
// SUM, PROD and the IEEE maximum are commutative bit for bit, so only the
// association tree matters; it is reproduced exactly.

#include "cc_device.h"

namespace cc {
namespace {

// ------------------------------------------------------------------ fused kernels


// The ring fold of one 16-byte vector per rank for a runtime rank count, in
// batches of 8 ranks in the chain's order (the first rank in the first
// batch), each batch's loads issued before the previous batch is folded,
// two register sets in turn.  Taken for bf16, whose lanes unpack and add
// eight values per load: measured on the MI355X (graph replays over
// rotating buffer sets, rows by the rank-stride rule, N = 6, 12, 20, 24,
// 28, 40) 16 MiB per rank 5.07-5.40 TB/s against 4.55-4.97, 64 MiB 5.32-6.09
// against 5.36-5.85, 4 MiB level (3.30-4.16 against 3.31-4.32); fp32 in this
// form took four times the registers and ran at 2.1-5.6 TB/s against
// 5.0-6.2, so it keeps the one-set loop of fold_vec.
template <int DT, int OP>
__device__ __forceinline__ void fold_ring_pipelined(const char* s0, uint64_t ss, int N, int start, uint32_t lane,
                                                    typename Ty<DT>::A* acc) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  const char* p = s0 + (uint64_t)start * ss;
  int r = start;
  auto load8 = [&](u32x4(&buf)[8], int j) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j + q < N) {
        if (j + q > 0) {
          r = r + 1 == N ? 0 : r + 1;
          p = r == 0 ? s0 : p + ss;
        }
        buf[q] = ldg(p + lane);
      }
  };
  auto fold8 = [&](const u32x4(&buf)[8], int j) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j + q < N) {
        A x[V];
        unpack<DT>(buf[q], x);
        if (j + q == 0) {
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] = x[i];
        } else {
          opv<DT, OP>(x, acc);
        }
      }
  };
  u32x4 ba[8], bb[8];
  load8(ba, 0);
  for (int j = 0; j < N; j += 16) {
    load8(bb, j + 8);
    fold8(ba, j);
    load8(ba, j + 16);
    fold8(bb, j + 8);
  }
}

// AllReduce (rs_mode 0): every chunk's N-1 ReduceScatter steps folded in
// registers in the schedule's order, then the AllGather as N stores.
// ReduceScatter (rs_mode 1, ring and halving-doubling): only the owner is
// written; the ring's fold then starts one rank later.
// The ReduceScatter half of a split ring AllReduce (rs_mode 2): the
// AllReduce's fold, stored only to the rank that owns the chunk after the
// ReduceScatter (rank c-1 for chunk c), at the chunk's place in its vector.
// U: 16-byte vectors per thread and rank (a tile of U kBlock vectors).
template <int DT, int OP, int NR, int ALG, int U = 1>
__device__ __forceinline__ void fused_body(const FusedArgs& a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int VT = V * U;  // elements per thread and tile
  constexpr int SZ = Ty<DT>::SZ;
  static_assert(kUnroll == 1, "the tile size is kBlock U vectors");
  // ring: N ranks (NR when fixed at compile time); trees: the runtime rank
  // count, NR being the tree's leaf slots
  const int N = (ALG == ALG_RING && NR > 0) ? NR : a.N;
  // a tree AllReduce folds every element the same way whatever its chunk,
  // so only a ReduceScatter needs the chunk of a tile
  const int tiling = (ALG != ALG_RING && !a.rs_mode) ? 1 : N;
  const TreeShape ts{a.tree_leaves, a.tree_pairs};
  const Tile<VT> t = a.tpc_log2 >= 0 ? tile_pow2<VT>(blockIdx.x, a.tpc_log2)
                                      : tile_floor<VT>(blockIdx.x, a.M, tiling, a.vec_ok);
  if (t.fast) {
    // Every rank's tile starts at a workgroup-uniform address; a lane adds
    // its own 16-byte offset (scalar base + 32-bit vector offset), vector u
    // of the thread another kBlock vectors on.
    const int c = (int)t.c;
    const int start = (ALG == ALG_RING && a.rs_mode == 1) ? wrapN(c + 1, N) : c;
    const uint32_t lane = threadIdx.x * 16u;
    constexpr uint32_t kStep = kBlock * 16u;
    const uint64_t eb = t.e0 * SZ;
    A acc[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ALG == ALG_RING && NR == 0 && DT == DT_BF16)
        fold_ring_pipelined<DT, OP>(a.sb + eb, a.ss, N, start, lane + u * kStep, acc[u]);
      else
        fold_vec<DT, OP, NR, ALG>(a.sb + eb, a.ss, N, start, lane + u * kStep, acc[u], ts);
    }
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = pack<DT>(acc[u]);
    if (a.rs_mode == 1) {
      char* d = a.rb + (uint64_t)c * a.rs + (t.e0 - a.bnd[c]) * SZ + lane;
#pragma unroll
      for (int u = 0; u < U; ++u) stg(d + u * kStep, w[u]);
    } else if (a.rs_mode == 2) {
      char* d = a.rb + (uint64_t)wrapN(c + N - 1, N) * a.rs + eb + lane;
#pragma unroll
      for (int u = 0; u < U; ++u) stg(d + u * kStep, w[u]);
    } else {
      char* d = a.rb + eb + lane;
      if constexpr (NR > 0) {
        if (N == NR) {  // the ring with NR > 0, a tree with every leaf slot used
#pragma unroll
          for (int r = 0; r < NR; ++r, d += a.rs)
#pragma unroll
            for (int u = 0; u < U; ++u) stg(d + u * kStep, w[u]);
        } else {
          for (int r = 0; r < N; ++r, d += a.rs)
#pragma unroll
            for (int u = 0; u < U; ++u) stg(d + u * kStep, w[u]);
        }
      } else {
        for (int r = 0; r < N; ++r, d += a.rs)
#pragma unroll
          for (int u = 0; u < U; ++u) stg(d + u * kStep, w[u]);
      }
    }
  } else {
    // Element-wise (a tile across chunk bounds, a ragged tail, unaligned
    // buffers): the thread's V elements, kBlock apart, are folded in
    // batches of G whose loads are in flight at once; an idle slot repeats
    // the tile's first element and stores nothing.  A tree folds one element
    // at a time (its fold already has NR loads in flight).
    constexpr int G = ALG == ALG_RING ? elem_batch<V, NR>() : 1;
    static_assert(VT % G == 0, "whole batches");
    for (int g0 = 0; g0 < VT; g0 += G) {
      uint64_t ev[G], off[G];
      uint32_t cv[G];
      int st[G];
      bool ok[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const uint64_t e = t.e0 + threadIdx.x + (uint64_t)(g0 + u) * kBlock;
        ok[u] = e < t.e1;
        ev[u] = ok[u] ? e : t.e0;
        off[u] = ev[u] * SZ;
        cv[u] = tiling == 1 ? 0u : chunk_of(a.M, tiling, ev[u]);
        st[u] = (ALG == ALG_RING && a.rs_mode == 1) ? wrapN((int)cv[u] + 1, N) : (int)cv[u];
      }
      A acc[G];
      if constexpr (ALG == ALG_RING) {
        ring_fold_elems<DT, OP, NR, G>(a.sb, a.ss, N, st, off, acc);
      } else {
#pragma unroll
        for (int u = 0; u < G; ++u) acc[u] = fold_elem<DT, OP, NR, ALG>(a.sb, a.ss, N, st[u], off[u], ts);
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (!ok[u]) continue;
        if (a.rs_mode == 1) {
          st1<DT>(a.rb + (uint64_t)cv[u] * a.rs + (ev[u] - bound_of(a.M, tiling, cv[u])) * SZ, acc[u]);
        } else if (a.rs_mode == 2) {
          st1<DT>(a.rb + (uint64_t)wrapN((int)cv[u] + N - 1, N) * a.rs + off[u], acc[u]);
        } else {
          for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + off[u], acc[u]);
        }
      }
    }
  }
}

template <int DT, int OP, int NR, int U>
__global__ __launch_bounds__(kBlock) void k_ring_fused(FusedArgs a) {
  fused_body<DT, OP, NR, ALG_RING, U>(a);
}

// Halving-doubling (TREE_HD) and butterfly / binomial tree (TREE_BFLY) over
// NR leaf slots; the binomial tree leaves slots N.. empty, N not a power of
// two folds the first 2r ranks in pairs into the leading leaves.
template <int DT, int OP, int NR, int TREE>
__global__ __launch_bounds__(kBlock) void k_tree_fused(FusedArgs a) {
  fused_body<DT, OP, NR, TREE == TREE_HD ? ALG_HD : ALG_BFLY>(a);
}

// Binomial tree over exactly N ranks, N not a power of two.
template <int DT, int OP, int N>
__global__ __launch_bounds__(kBlock) void k_btree_fused(FusedArgs a) {
  fused_body<DT, OP, N, ALG_BTREE>(a);
}

}  // namespace


unsigned lds_for_blocks_per_cu(int blocks) {
  if (blocks <= 0) return 0;
  const DevInfo i = dev_info();
  if (i.lds_per_cu <= 0 || i.lds_per_block <= 0) return 0;
  // Rounded down to the allocation granule, so that rounding up cannot push
  // `blocks` reservations past the CU's LDS.  gfx950 hands out LDS in
  // 1280-byte granules (160 KiB = 128 of them): measured with workgroups that
  // record their CU and lifetime, 32 KiB reservations let only 4 share a CU
  // (5 x 26 granules > 128) and 16 KiB only 9, while 30 KiB let 5 and 20 KiB
  // let 8; every reservation tried from 14 to 80 KiB matched that count.
  constexpr unsigned kLdsGranule = 1280;
  unsigned lds = (unsigned)(i.lds_per_cu / blocks) / kLdsGranule * kLdsGranule;
  if (lds > (unsigned)i.lds_per_block) lds = (unsigned)i.lds_per_block;
  return lds;
}

// Workgroups per CU for a kernel moving `traffic` bytes (loads + stores) per
// workgroup, aiming at `target` bytes in flight per CU.  Measured on the
// MI355X: a balanced read/write stream (fused AllReduce) streams best near
// 64 KiB per CU, a read- or write-dominated one (ReduceScatter, AllGather)
// near 144 KiB, broadcast near 72 KiB; more in flight thrashes the DRAM,
// less leaves it idle.
int default_blocks_per_cu(uint64_t traffic, uint64_t target, int min_blocks) {
  if (traffic == 0) return 0;
  int b = (int)((target + traffic / 2) / traffic);
  if (b < min_blocks) b = min_blocks;
  return b > 16 ? 16 : b;
}


namespace {

// The split form of the fused ring AllReduce: two launches, the ReduceScatter
// (every chunk's fold stored to its owner only) and the AllGather (the
// owner's chunk copied to the other ranks).  It moves (2N+1) M s bytes
// against the one-launch form's 2 N M s, as two streams that are each read-
// or write-heavy instead of one with N loads and N stores per vector, which
// the HBM serves faster from 32 ranks of 16 MiB on.  Measured on the MI355X
// (graph replays over rotating buffer sets of 1 GiB or more, rows by the
// rank-stride rule, two runs of each form; split time over one-launch time,
// mean and range over N = 32, 40, 48, 56, 64): fp32 16 MiB per rank 0.89
// (0.85-0.93), 32 MiB 0.92 (0.88-0.96), 64 MiB 0.95 (0.92-0.96); bf16
// 16 MiB 0.93 (0.86-0.97), 32 MiB 0.95 (0.89-0.98), 64 MiB 0.97 (0.94-1.02).
// At 8 MiB (fp32 1.00, bf16 1.06), 4 MiB and below (1.04-1.24, the second
// launch included) and below 32 ranks (28 ranks: 0.99-1.26) the one-launch
// form is as fast or faster.
bool ring_split(const Red& r) {
  return r.N >= 32 && r.M * (uint64_t)(16 / vec_elems(r.dt)) >= (16ull << 20);
}

// A grid of 8 to 16 one-vector tiles per CU (4 to 8 MiB per rank) takes two
// vectors per thread: half the workgroups, each thread with twice the loads
// in flight, in one round.  Measured on the MI355X (graph replays over
// rotating buffer sets, one vector against two): int32 4 ranks x 1,048,576
// 8.16-8.27 us against 6.64-6.70; fp32 8 ranks of 4 MiB 15.5-15.7 against
// 12.5-12.6, of 8 MiB 28.3-28.8 against 26.8-26.9; fp32 16 ranks of 4 MiB
// 32.8-33.0 against 26.1.  Below (the element-wise path of small chunks, then
// twice the elements per thread) and above (2 MiB per rank level, 16 MiB and
// up 2-25% slower) one vector per thread stays.
// mode: FusedArgs::rs_mode (0 AllReduce, 1 ReduceScatter, 2 the split form's
// first launch).
hipError_t launch_ring_kernel(const Red& r, int mode) {
  FusedArgs a = fused_args(r);
  a.rs_mode = mode;
  const uint64_t tiles1 = num_tiles(r.M, r.dt);
  const int cus = dev_info().cus;
  const bool wide = cus > 0 && tiles1 >= 8ull * (uint64_t)cus && tiles1 <= 16ull * (uint64_t)cus;
  if (wide) a.tpc_log2 = pow2_tiles_per_chunk_v(r.M, r.N, 2 * vec_elems(r.dt), r.vec_ok);
  const uint64_t tile2 = 2ull * kBlock * vec_elems(r.dt);
  const dim3 grid((unsigned)(wide ? (r.M + tile2 - 1) / tile2 : tiles1)), blk(kBlock);
  const bool runtime_n = r.N != 2 && r.N != 3 && r.N != 4 && r.N != 8 && r.N != 16;
  // Two measured exceptions to the byte rule (2 GiB per buffer, rows 256 KiB
  // beyond the payload apart): at N = 3, 8 workgroups per CU (6.44 fp32 and
  // 6.45 bf16 TB/s against 6.12 and 6.01 at 4); at N = 2 in fp32,
  // 6 (6.21-6.31 against 5.92-6.00 at the rule's 8; bf16 keeps 8).
  const int ring_bpc = r.blocks_per_cu > 0 ? r.blocks_per_cu
                       : r.N == 3                     ? 8
                       : (r.N == 2 && r.dt != DT_BF16) ? 6
                                                       : 0;
  const unsigned lds =
      mode ? rs_fused_lds(r)
      : runtime_n ? lds_for_blocks_per_cu(r.blocks_per_cu > 0 ? r.blocks_per_cu
                                                              : one_round_blocks(num_tiles(r.M, r.dt),
                                                                                 batched_ring_blocks_per_cu(r.N, r.dt)))
                  : ar_fused_lds(r, ring_bpc);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    auto go = [&](auto u) {
      constexpr int U = decltype(u)::value;
      switch (r.N) {
        case 2: CC_LAUNCH((k_ring_fused<DT, OP, 2, U>), grid, blk, lds, r.st, a); break;
        case 3: CC_LAUNCH((k_ring_fused<DT, OP, 3, U>), grid, blk, lds, r.st, a); break;
        case 4: CC_LAUNCH((k_ring_fused<DT, OP, 4, U>), grid, blk, lds, r.st, a); break;
        case 8: CC_LAUNCH((k_ring_fused<DT, OP, 8, U>), grid, blk, lds, r.st, a); break;
        case 16: CC_LAUNCH((k_ring_fused<DT, OP, 16, U>), grid, blk, lds, r.st, a); break;
        default: CC_LAUNCH((k_ring_fused<DT, OP, 0, U>), grid, blk, lds, r.st, a); break;
      }
      return hipGetLastError();
    };
    return wide ? go(IC<2>{}) : go(IC<1>{});
  });
}

}  // namespace

hipError_t launch_ring_fused(const Red& r) {
  if (r.rs_mode == 0 && ring_split(r)) {
    const hipError_t e = launch_ring_kernel(r, 2);
    if (e != hipSuccess) return e;
    const Gat g{r.recv, r.recv, r.M, r.bnd, r.blocks_per_cu, r.N, 16 / vec_elems(r.dt), 0, r.vec_ok, r.st};
    return launch_ag_fused(g);
  }
  return launch_ring_kernel(r, r.rs_mode);
}

hipError_t launch_tree_fused(const Red& r, int tree) {
  const FusedArgs a = fused_args(r);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = r.rs_mode ? rs_fused_lds(r) : ar_fused_lds(r, r.blocks_per_cu);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
#define CC_TREE_CASE(NR)                                                                      \
  case NR:                                                                                    \
    if (tree == TREE_HD)                                                                      \
      CC_LAUNCH((k_tree_fused<DT, OP, NR, TREE_HD>), grid, blk, lds, r.st, a);       \
    else                                                                                      \
      CC_LAUNCH((k_tree_fused<DT, OP, NR, TREE_BFLY>), grid, blk, lds, r.st, a);     \
    break;
    switch (r.N) {
      CC_TREE_CASE(2)
      CC_TREE_CASE(4)
      CC_TREE_CASE(8)
      CC_TREE_CASE(16)
      CC_TREE_CASE(32)
      CC_TREE_CASE(64)
      default: return hipErrorInvalidValue;
    }
#undef CC_TREE_CASE
    return hipGetLastError();
  });
}

hipError_t launch_tree_shaped(const Red& r, int tree, int nr, int leaves, int pairs) {
  FusedArgs a = fused_args(r);
  a.tree_leaves = leaves;
  a.tree_pairs = pairs;
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = ar_fused_lds(r, r.blocks_per_cu);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    if (tree == TREE_BFLY && pairs == 0 && leaves < nr && leaves <= 16) {
      // binomial tree with a compile-time rank count
      switch (leaves) {
#define CC_BTREE_CASE(NN) \
  case NN: CC_LAUNCH((k_btree_fused<DT, OP, NN>), grid, blk, lds, r.st, a); break;
        CC_BTREE_CASE(3) CC_BTREE_CASE(5) CC_BTREE_CASE(6) CC_BTREE_CASE(7) CC_BTREE_CASE(9)
        CC_BTREE_CASE(10) CC_BTREE_CASE(11) CC_BTREE_CASE(12) CC_BTREE_CASE(13) CC_BTREE_CASE(14)
        CC_BTREE_CASE(15)
#undef CC_BTREE_CASE
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
#define CC_SHAPED_CASE(NR)                                                                    \
  case NR:                                                                                    \
    if (tree == TREE_HD)                                                                      \
      CC_LAUNCH((k_tree_fused<DT, OP, NR, TREE_HD>), grid, blk, lds, r.st, a);       \
    else                                                                                      \
      CC_LAUNCH((k_tree_fused<DT, OP, NR, TREE_BFLY>), grid, blk, lds, r.st, a);     \
    break;
    switch (nr) {
      CC_SHAPED_CASE(2)
      CC_SHAPED_CASE(4)
      CC_SHAPED_CASE(8)
      CC_SHAPED_CASE(16)
      CC_SHAPED_CASE(32)
      CC_SHAPED_CASE(64)
      default: return hipErrorInvalidValue;
    }
#undef CC_SHAPED_CASE
    return hipGetLastError();
  });
}

}  // namespace cc
