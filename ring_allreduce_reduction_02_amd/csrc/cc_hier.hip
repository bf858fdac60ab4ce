// The fused hierarchical AllReduce kernel of the collective-reduction engine
// (the "AllReduce" algorithm notes, 算法五 多维分层 AllReduce; textbook ch. 6
// "集合通信", 分层全归约).

#include "cc_device.h"

namespace cc {
namespace {

// ------------------------------------------------------------------ hierarchical AllReduce

// Rank r = sum of c_i * stride[i] over the (at most kMaxHierLevels)
// non-trivial levels.  The vector splits into N segments -- the level-0
// chunks, each split into its level-1 chunks, and so on -- each with one
// chunk index per level (seg[s], 8 bits per level); bnd holds their bounds.
// An element's value is the nested ring chains of the pages' decomposition:
// the outermost level (top; nd when the outermost level of the hierarchy
// has size 1 and no AllReduce runs) folds its members from chunk index c
// (AllReduce order), every other level from c + 1 (standalone
// ReduceScatter order), each chain op(next, partial), the members' values
// being the inner levels' chains.
struct HierArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  uint64_t M;
  int N;
  int nd;
  int top;
  int vec_ok;
  int tpc_log2;  // segments of exactly 2^k full tiles: log2 of k, else -1
  int one;       // store each result once, to the owner of its flat ring chunk
  int p[kMaxHierLevels];
  int stride[kMaxHierLevels];
  uint32_t seg[kMaxRanks];       // the segments' chunk indices, 8 bits per level
  uint64_t bnd[kMaxRanks + 1];   // the segments' bounds
};

// The segment of element e: the flat floor chunk floor(((e + 1) N - 1) / M)
// of the ring kernels' closed form, settled by the segment bounds.  The
// nested bounds (each level's floor split of its range) lie within a few
// elements of the flat floor bounds floor(s M / N), so where segments hold
// more than a few elements the estimate is the segment or one beside it and
// the loops take at most one step; they correct any estimate, since the
// bounds rise from 0 to M.
__device__ __forceinline__ uint32_t hier_seg(const HierArgs& a, uint64_t e) {
  uint32_t s = chunk_of(a.M, a.N, e);
  while (s > 0 && e < a.bnd[s]) --s;
  while (s + 1 < (uint32_t)a.N && e >= a.bnd[s + 1]) ++s;
  return s;
}

// First coordinate of each level's chain for segment s: the top level
// starts at its chunk index c (AllReduce order), every other level at c + 1.
__device__ __forceinline__ int hier_first(const HierArgs& a, uint32_t seg, int i) {
  const int c = (int)((seg >> (8 * i)) & 255u);
  if (i == a.top) return c;
  return c + 1 == a.p[i] ? 0 : c + 1;
}

// acc = x (first member of a chain) or op(x, acc)
template <int DT, int OP, int VN>
__device__ __forceinline__ void hier_join(bool first, const typename Ty<DT>::A (&x)[VN],
                                          typename Ty<DT>::A (&acc)[VN]) {
#pragma unroll
  for (int k = 0; k < VN; ++k) acc[k] = first ? x[k] : opf<DT, OP>(x[k], acc[k]);
}

// The levels of one segment, uniform across the workgroup: sizes (1 beyond
// nd), first coordinate of each chain, rank strides.
struct HierLv {
  int p[kMaxHierLevels], f[kMaxHierLevels], sd[kMaxHierLevels];
};

__device__ __forceinline__ HierLv hier_lv(const HierArgs& a, uint32_t seg) {
  HierLv L;
#pragma unroll
  for (int i = 0; i < kMaxHierLevels; ++i) {
    L.p[i] = i < a.nd ? a.p[i] : 1;
    L.f[i] = i < a.nd ? hier_first(a, seg, i) : 0;
    L.sd[i] = i < a.nd ? a.stride[i] : 0;
  }
  return L;
}

// A position in the walk over the N leaves in fold order (level 0 fastest):
// j[i] counts the members of level i's chain already passed, c[i] is the
// coordinate of the current one.  Every index is a compile-time constant, so
// the state lives in scalar registers.
struct HierPos {
  int c[kMaxHierLevels], j[kMaxHierLevels];
};

__device__ __forceinline__ HierPos hier_begin(const HierLv& L) {
  HierPos w;
#pragma unroll
  for (int i = 0; i < kMaxHierLevels; ++i) {
    w.c[i] = L.f[i];
    w.j[i] = 0;
  }
  return w;
}

__device__ __forceinline__ int hier_rank(const HierLv& L, const HierPos& w) {
  int r = 0;
#pragma unroll
  for (int i = 0; i < kMaxHierLevels; ++i) r += w.c[i] * L.sd[i];
  return r;
}

// next leaf; after the last one the walk starts over at the first
__device__ __forceinline__ void hier_step(const HierLv& L, HierPos& w) {
  bool carry = true;
#pragma unroll
  for (int i = 0; i < kMaxHierLevels; ++i) {
    if (carry) {
      if (w.j[i] + 1 < L.p[i]) {
        ++w.j[i];
        w.c[i] = w.c[i] + 1 == L.p[i] ? 0 : w.c[i] + 1;
        carry = false;
      } else {
        w.j[i] = 0;
        w.c[i] = L.f[i];
      }
    }
  }
}

// Folds the leaf at walk position w into the chain accumulators: the level-0
// chain takes it, and every level whose chain it completes passes its value
// on to the level above.
template <int DT, int OP, int VN>
__device__ __forceinline__ void hier_take(const HierLv& L, const HierPos& w, const typename Ty<DT>::A (&x)[VN],
                                          typename Ty<DT>::A (&a0)[VN], typename Ty<DT>::A (&a1)[VN],
                                          typename Ty<DT>::A (&a2)[VN], typename Ty<DT>::A (&a3)[VN]) {
  hier_join<DT, OP, VN>(w.j[0] == 0, x, a0);
  if (w.j[0] + 1 == L.p[0]) {
    hier_join<DT, OP, VN>(w.j[1] == 0, a0, a1);
    if (w.j[1] + 1 == L.p[1]) {
      hier_join<DT, OP, VN>(w.j[2] == 0, a1, a2);
      if (w.j[2] + 1 == L.p[2]) hier_join<DT, OP, VN>(w.j[3] == 0, a2, a3);
    }
  }
}

constexpr int kHierBatch = 8;  // leaves loaded ahead of their folds

// The rank that owns element e after a flat ring ReduceScatter: c - 1 for
// its chunk c = floor(((e + 1) N - 1) / M).
__device__ __forceinline__ int hier_owner(const HierArgs& a, uint64_t e) {
  const int c = (int)chunk_of(a.M, a.N, e);
  return c == 0 ? a.N - 1 : c - 1;
}

// The workgroup's tile: its segment, and whether it takes the vector path.
template <int V>
__device__ __forceinline__ Tile<V> hier_tile(const HierArgs& a) {
  if (a.tpc_log2 >= 0) return tile_pow2<V>(blockIdx.x, a.tpc_log2);
  const uint64_t tile = (uint64_t)kBlock * V;
  Tile<V> t;
  t.e0 = (uint64_t)blockIdx.x * tile;
  t.e1 = t.e0 + tile < a.M ? t.e0 + tile : a.M;
  t.c = hier_seg(a, t.e0);
  t.fast = a.vec_ok && t.e1 - t.e0 == tile && t.e1 <= a.bnd[t.c + 1];
  return t;
}

// A vector-path tile's results: to every rank, or once, to the owners.
template <int DT>
__device__ __forceinline__ void hier_store(const HierArgs& a, const Tile<Ty<DT>::V>& t,
                                           const typename Ty<DT>::A (&res)[Ty<DT>::V]) {
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const uint32_t lane = threadIdx.x * 16u;
  if (a.one) {
    const int o0 = hier_owner(a, t.e0);
    if (o0 == hier_owner(a, t.e1 - 1)) {
      stg(a.rb + (uint64_t)o0 * a.rs + t.e0 * SZ + lane, pack<DT>(res));
    } else {  // the tile holds a flat chunk bound
      const uint64_t e = t.e0 + (uint64_t)threadIdx.x * V;
#pragma unroll
      for (int k = 0; k < V; ++k) st1<DT>(a.rb + (uint64_t)hier_owner(a, e + k) * a.rs + (e + k) * SZ, res[k]);
    }
  } else {
    const u32x4 o = pack<DT>(res);
    char* d = a.rb + t.e0 * SZ;
    for (int r = 0; r < a.N; ++r, d += a.rs) stg(d + lane, o);
  }
}

// The element-wise path (a tile across segment bounds, a ragged tail,
// unaligned buffers).
template <int DT, int OP>
__device__ __forceinline__ void hier_elems(const HierArgs& a, const Tile<Ty<DT>::V>& t) {
  typedef typename Ty<DT>::A A;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = a.N;
  // a thread's elements are kBlock apart: the segment is looked up again
  // only when an element leaves the previous one's
  uint64_t slo = 1, shi = 0;
  uint32_t scode = 0;
  for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
    if (e < slo || e >= shi) {
      const uint32_t sg = hier_seg(a, e);
      slo = a.bnd[sg];
      shi = a.bnd[sg + 1];
      scode = a.seg[sg];
    }
    const HierLv L = hier_lv(a, scode);
    HierPos ld = hier_begin(L), fw = ld;
    A a0[1], a1[1], a2[1], a3[1];
    // batches of leaf loads in flight before their folds, as on the
    // vector path (one load at a time left every element waiting N times)
    for (int l0 = 0; l0 < N; l0 += kHierBatch) {
      A raw[kHierBatch];
#pragma unroll
      for (int q = 0; q < kHierBatch; ++q) {
        raw[q] = ld1<DT>(a.sb + (uint64_t)hier_rank(L, ld) * a.ss + e * SZ);
        hier_step(L, ld);
      }
#pragma unroll
      for (int q = 0; q < kHierBatch; ++q)
        if (l0 + q < N) {
          const A x[1] = {raw[q]};
          hier_take<DT, OP, 1>(L, fw, x, a0, a1, a2, a3);
          hier_step(L, fw);
        }
    }
    if (a.one)
      st1<DT>(a.rb + (uint64_t)hier_owner(a, e) * a.rs + e * SZ, a3[0]);
    else
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, a3[0]);
  }
}

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_hier_fused(HierArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  static_assert(kMaxHierLevels == 4, "four levels");
  const int N = a.N;
  const Tile<V> t = hier_tile<V>(a);
  if (!t.fast) {
    hier_elems<DT, OP>(a, t);
    return;
  }
  const uint32_t lane = threadIdx.x * 16u;
  const char* s0 = a.sb + t.e0 * SZ;
  const HierLv L = hier_lv(a, a.seg[t.c]);
  HierPos ld = hier_begin(L), fw = ld;
  A a0[V], a1[V], a2[V], a3[V];
  for (int l0 = 0; l0 < N; l0 += kHierBatch) {
    // every load of the batch is issued before the first fold; past the
    // last leaf the walk has wrapped to valid ranks whose values go unused
    u32x4 raw[kHierBatch];
#pragma unroll
    for (int q = 0; q < kHierBatch; ++q) {
      raw[q] = ldg(s0 + (uint64_t)hier_rank(L, ld) * a.ss + lane);
      hier_step(L, ld);
    }
#pragma unroll
    for (int q = 0; q < kHierBatch; ++q)
      if (l0 + q < N) {
        A x[V];
        unpack<DT>(raw[q], x);
        hier_take<DT, OP, V>(L, fw, x, a0, a1, a2, a3);
        hier_step(L, fw);
      }
  }
  hier_store<DT>(a, t, a3);
}

// The same fold with the grid fixed at compile time (level sizes P0..P3, 1
// beyond the grid's levels): a leaf's position in every chain is a constant
// of its index, so the joins are straight-line code without selects, and
// only the ranks (from the segment's first coordinates) are computed at run
// time, on the scalar unit.  Taken for bf16 on the grids below, where a lane
// folds eight elements per leaf and the runtime walk's selects cost most.
// Measured on the MI355X (best of two runs each, on one machine, rows by the
// hierarchical workload's layout): bf16 8x8 and 4x4x4 of 2 MiB per rank
// 5.48-5.68 TB/s against 4.44-4.71; 8x8 and 4x4x4 of 32 MiB (the split
// form) 5.60-5.98 against 5.48-5.92; 2x2x2, 4x2, 2x4 of 256 MiB 6.33-6.38
// against 6.23-6.30 at the default 3 workgroups per CU.  For fp32 the
// runtime walk was as fast or faster (2x2x2 6.36-6.39 against 6.22-6.29).
template <int P0, int P1, int P2, int P3>
__device__ __forceinline__ int grid_rank(const HierLv& L, int q) {
  const int j[4] = {q % P0, (q / P0) % P1, (q / (P0 * P1)) % P2, q / (P0 * P1 * P2)};
  const int p[4] = {P0, P1, P2, P3};
  int r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = L.f[i] + j[i];
    r += (c >= p[i] ? c - p[i] : c) * L.sd[i];
  }
  return r;
}

template <int DT, int OP, int P0, int P1, int P2, int P3>
__global__ __launch_bounds__(kBlock) void k_hier_grid(HierArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int NL = P0 * P1 * P2 * P3;
  const Tile<V> t = hier_tile<V>(a);
  if (!t.fast) {
    hier_elems<DT, OP>(a, t);
    return;
  }
  const uint32_t lane = threadIdx.x * 16u;
  const char* s0 = a.sb + t.e0 * SZ;
  const HierLv L = hier_lv(a, a.seg[t.c]);
  A a0[V], a1[V], a2[V], a3[V];
#pragma unroll
  for (int q0 = 0; q0 < NL; q0 += kHierBatch) {
    u32x4 raw[kHierBatch];
#pragma unroll
    for (int k = 0; k < kHierBatch; ++k)
      if (q0 + k < NL) raw[k] = ldg(s0 + (uint64_t)grid_rank<P0, P1, P2, P3>(L, q0 + k) * a.ss + lane);
#pragma unroll
    for (int k = 0; k < kHierBatch; ++k) {
      const int q = q0 + k;
      if (q >= NL) break;
      const int j0 = q % P0, j1 = (q / P0) % P1, j2 = (q / (P0 * P1)) % P2, j3 = q / (P0 * P1 * P2);
      A x[V];
      unpack<DT>(raw[k], x);
      hier_join<DT, OP, V>(j0 == 0, x, a0);
      if (j0 + 1 == P0) {
        hier_join<DT, OP, V>(j1 == 0, a0, a1);
        if (j1 + 1 == P1) {
          hier_join<DT, OP, V>(j2 == 0, a1, a2);
          if (j2 + 1 == P2) hier_join<DT, OP, V>(j3 == 0, a2, a3);
        }
      }
    }
  }
  hier_store<DT>(a, t, a3);
}

// The split form, as the flat ring's: the fold stored once, to the rank that
// owns the element's flat ring chunk after a ReduceScatter, then the ring
// AllGather's copy from those owners to every other rank.  Taken from 32
// ranks of 4 MiB on.  Measured on the MI355X (graph replays over rotating
// buffer sets of 1 GiB or more, rows by the rank-stride rule, fp32 and bf16;
// split time over one-launch time): 64 ranks (8x8, 4x4x4, 2x32) 0.83-0.92
// from 4 to 32 MiB per rank, 0.87-0.99 at 64 MiB, 0.96-1.00 at 2 MiB; 32
// ranks (4x8, 2x16, 2x2x2x4) 0.89-1.00 from 4 to 32 MiB, 0.95-1.01 at 64
// MiB, 1.03-1.08 at 2 MiB.  The first launch, N loads and one store per
// vector, streams best at 4 workgroups per CU (at 64 MiB per rank 2x32
// 0.89-0.96 against 1.07-1.17 at 2, 0.92-1.00 at 3).
bool hier_split(const Red& r) {
  return r.N >= 32 && r.M * (uint64_t)(16 / vec_elems(r.dt)) >= (4ull << 20);
}
constexpr int kHierOneBlocks = 4;

}  // namespace

hipError_t launch_hier_fused(const Red& r, const int* p, const int* stride, int nd, int top, const uint64_t* segbnd,
                             const uint32_t* seg) {
  if (nd < 1 || nd > kMaxHierLevels || top < 0 || top > nd || r.N < 2 || r.N > kMaxRanks) return hipErrorInvalidValue;
  HierArgs a;
  a.sb = r.send.base; a.ss = r.send.stride;
  a.rb = r.recv.base; a.rs = r.recv.stride;
  a.M = r.M; a.N = r.N; a.nd = nd; a.top = top; a.vec_ok = r.vec_ok;
  // the N segments are equal when every level splits exactly
  a.tpc_log2 = pow2_tiles_per_chunk(r.M, r.N, r.dt, r.vec_ok);
  for (int i = 0; i < kMaxHierLevels; ++i) {
    a.p[i] = i < nd ? p[i] : 1;
    a.stride[i] = i < nd ? stride[i] : 0;
  }
  for (int s = 0; s < r.N; ++s) a.seg[s] = seg[s];
  for (int s = 0; s <= r.N; ++s) a.bnd[s] = segbnd[s];
  a.one = hier_split(r) ? 1 : 0;
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const int bpc = a.one ? kHierOneBlocks : hier_blocks_per_cu(r.N);
  const unsigned lds = lds_for_blocks_per_cu(r.blocks_per_cu > 0 ? r.blocks_per_cu
                                                                 : one_round_blocks(num_tiles(r.M, r.dt), bpc));
  // the level sizes (each at most kMaxRanks) as one number
  const int g4 = ((a.p[0] * 65 + a.p[1]) * 65 + a.p[2]) * 65 + a.p[3];
  hipError_t e = by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    if constexpr (DT == DT_BF16) {
#define CC_GRID(P0, P1, P2, P3)                                                  \
  case ((P0 * 65 + P1) * 65 + P2) * 65 + P3:                                   \
    CC_LAUNCH((k_hier_grid<DT, OP, P0, P1, P2, P3>), grid, blk, lds, r.st, a); \
    return hipGetLastError();
      switch (g4) {
        CC_GRID(2, 2, 2, 1)
        CC_GRID(4, 2, 1, 1)
        CC_GRID(2, 4, 1, 1)
        CC_GRID(8, 8, 1, 1)
        CC_GRID(4, 4, 4, 1)
        default: break;
      }
#undef CC_GRID
    }
    CC_LAUNCH((k_hier_fused<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
  if (e != hipSuccess || !a.one) return e;
  // the AllGather from the owners of the flat ring chunks
  uint64_t fb[kMaxRanks + 1];
  for (int c = 0; c <= r.N; ++c) fb[c] = (uint64_t)(((unsigned __int128)c * r.M) / (unsigned)r.N);
  const Gat g{r.recv, r.recv, r.M, fb, r.blocks_per_cu, r.N, 16 / vec_elems(r.dt), 0, r.vec_ok, r.st};
  return launch_ag_fused(g);
}

}  // namespace cc
