// Fused AllReduce kernels of the schedules beyond the ring and the power-of-two
// trees: the double binary tree (the "AllReduce" algorithm notes, 算法三;
// textbook ch. 6 "集合通信", 双二叉树), the 2-port ring (the notes, 2-port Ring
// 优化), and the bucketed AllReduce, several buckets per launch (textbook
// ch. 6, Bucket fusion).

#include "cc_device.h"

namespace cc {
namespace {

// ------------------------------------------------------------------ double binary tree

// Fold of the in-order binary tree over the leaf slots x[0..n) (n <= NR):
// slot y with lowest set bit 2^j (j >= 1) has the left child y - 2^(j-1) and
// the right child y + c, c the largest of 2^(j-1), 2^(j-2), ... with
// y + c < n (none if there is none); a node is op(op(own, left), right).
// Slot 0 sits on top of the root, the largest power of two below n.
// Subtrees are folded level by level, every slot index fixed at compile
// time; the clipping of right children near n only selects among them.
template <int DT, int OP, int NR>
__device__ __forceinline__ void dbt_fold(typename Ty<DT>::A (*x)[Ty<DT>::V], int n, int V,
                                         typename Ty<DT>::A* out) {
  constexpr int L = ilog2<NR>();
#pragma unroll
  for (int j = 1; j < L; ++j) {
    const int b = 1 << j;
#pragma unroll
    for (int y = b; y < NR; y += 2 * b) {
      if (y < n) {
#pragma unroll
        for (int i = 0; i < Ty<DT>::V; ++i)
          if (i < V) x[y][i] = opf<DT, OP>(x[y][i], x[y - b / 2][i]);
        bool done = false;
#pragma unroll
        for (int c = b / 2; c >= 1; c /= 2)
          if (!done && y + c < NR && y + c < n) {
#pragma unroll
            for (int i = 0; i < Ty<DT>::V; ++i)
              if (i < V) x[y][i] = opf<DT, OP>(x[y][i], x[y + c][i]);
            done = true;
          }
      }
    }
  }
  bool done = false;
#pragma unroll
  for (int p2 = NR / 2; p2 >= 1; p2 /= 2)
    if (!done && p2 <= n - 1) {
#pragma unroll
      for (int i = 0; i < Ty<DT>::V; ++i)
        if (i < V) out[i] = opf<DT, OP>(x[0][i], x[p2][i]);
      done = true;
    }
  if (!done) {
#pragma unroll
    for (int i = 0; i < Ty<DT>::V; ++i)
      if (i < V) out[i] = x[0][i];
  }
}

// Double binary tree AllReduce: elements [0, M/2) use the tree above over
// ranks in order, [M/2, M) the same tree with rank p in slot p-1 (slot s
// holds rank s+1 mod N).  The host passes bnd = {0, M/2, M} so a tile lies in
// one half on the vector path.  EXACT: N == NR, every slot holds a rank and
// the fold's shape is fixed at compile time (the slot loads then cannot be
// split by rank-count branches, which would let the compiler wait on each
// load before issuing the next).
template <int DT, int OP, int NR, bool EXACT>
__global__ __launch_bounds__(kBlock) void k_dbt_fused(FusedArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = EXACT ? NR : a.N;
  const Tile<V> t = tile_floor<V>(blockIdx.x, a.M, 2, a.vec_ok);
  if (t.fast) {
    const int half = (int)t.c;
    const uint32_t lane = threadIdx.x * 16u;
    const uint64_t eb = t.e0 * SZ;
    // slot s holds rank s (first half) or s+1 mod N (second half): a scalar
    // pointer walk; all loads are issued before any is used.  With a runtime
    // N the slots past N load rank 0's vector again (a cache hit, never
    // used): a load under a rank-count branch would make its register a
    // join of two values, whose copy waits for the load before the next one
    // is issued.
    const char* const b0 = a.sb + eb;
    const char* p = half ? b0 + a.ss : b0;
    u32x4 raw[NR];
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      raw[s] = ldg((s < N ? p : b0) + lane);
      p = s >= N ? p : ((half && s + 2 == N) ? b0 : p + a.ss);
    }
    A x[NR][V];
#pragma unroll
    for (int s = 0; s < NR; ++s)
      if (s < N) unpack<DT>(raw[s], x[s]);
    A acc[V];
    dbt_fold<DT, OP, NR>(x, N, V, acc);
    const u32x4 w = pack<DT>(acc);
    char* d = a.rb + eb;
    for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, w);
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const int half = e >= a.bnd[1] ? 1 : 0;
      A x[NR][V];
#pragma unroll
      for (int s = 0; s < NR; ++s)
        if (s < N) {
          const int r = half == 0 ? s : (s + 1 == N ? 0 : s + 1);
          x[s][0] = ld1<DT>(a.sb + (uint64_t)r * a.ss + e * SZ);
        }
      A acc[V];
      dbt_fold<DT, OP, NR>(x, N, 1, acc);
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, acc[0]);
    }
  }
}

// ------------------------------------------------------------------ 2-port ring

// Fold of a chain of `len` ranks starting at `first` and stepping by `dir`
// (+1 or -1 mod N): acc = x_first, then acc = op(x_next, acc) -- the order a
// partial picks up contributions as it travels rank to rank.  Loads are
// issued eight at a time.
template <int DT, int OP>
__device__ __forceinline__ void chain_vec(const char* s0, uint64_t ss, int N, int first, int dir, int len,
                                          uint32_t lane, typename Ty<DT>::A* acc) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  int r = first;
  unpack<DT>(ldg(s0 + (uint64_t)r * ss + lane), acc);
  for (int j = 1; j < len; j += 8) {
    u32x4 raw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j + q < len) {
        r += dir;
        r = r == N ? 0 : (r < 0 ? N - 1 : r);
        raw[q] = ldg(s0 + (uint64_t)r * ss + lane);
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j + q < len) {
        A y[V];
        unpack<DT>(raw[q], y);
        opv<DT, OP>(y, acc);
      }
  }
}

template <int DT, int OP>
__device__ __forceinline__ typename Ty<DT>::A chain_elem(const char* sb, uint64_t ss, int N, int first, int dir,
                                                         int len, uint64_t off) {
  typedef typename Ty<DT>::A A;
  int r = first;
  A acc = ld1<DT>(sb + (uint64_t)r * ss + off);
  for (int j = 1; j < len; ++j) {
    r += dir;
    r = r == N ? 0 : (r < 0 ? N - 1 : r);
    acc = opf<DT, OP>(ld1<DT>(sb + (uint64_t)r * ss + off), acc);
  }
  return acc;
}

// 2-port ring AllReduce: chunk c (owned by rank c) is folded by a clockwise
// chain over ranks c-a .. c (the owner last) and a counter-clockwise chain
// over ranks c+b .. c+1, a = N/2, b = (N-1)/2; the result op(cw, ccw) goes
// to every rank.
// NR > 0: N <= NR (N == NR when EXACT, a compile-time rank count); every
// rank's vector is loaded first, in ring order from rank c-a, then both
// chains fold from registers.  NR = 0: any N, the chains load as they go.
template <int DT, int OP, int NR, bool EXACT>
__global__ __launch_bounds__(kBlock) void k_ring2_fused(FusedArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = EXACT ? NR : a.N;
  const int ca = N / 2, cb = (N - 1) / 2;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const int c = (int)t.c;
    const uint32_t lane = threadIdx.x * 16u;
    const uint64_t eb = t.e0 * SZ;
    A acc[V];
    if constexpr (NR > 0) {
      // raw[j] = rank c - a + j: the clockwise chain is raw[0..a], the
      // counter-clockwise chain raw[N-1] down to raw[a+1]
      u32x4 raw[NR];
      int r = c - ca < 0 ? c - ca + N : c - ca;
#pragma unroll
      for (int j = 0; j < NR; ++j)
        if (j < N) {
          raw[j] = ldg(a.sb + eb + (uint64_t)r * a.ss + lane);
          r = r + 1 == N ? 0 : r + 1;
        }
      unpack<DT>(raw[0], acc);
#pragma unroll
      for (int j = 1; j < NR; ++j)
        if (j <= ca) {
          A y[V];
          unpack<DT>(raw[j], y);
          opv<DT, OP>(y, acc);
        }
      if (cb > 0) {
        A acc2[V];
#pragma unroll
        for (int j = NR - 1; j >= 1; --j)
          if (j == N - 1) unpack<DT>(raw[j], acc2);
#pragma unroll
        for (int j = NR - 2; j >= 1; --j)
          if (j < N - 1 && j > ca) {
            A y[V];
            unpack<DT>(raw[j], y);
            opv<DT, OP>(y, acc2);
          }
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = opf<DT, OP>(acc[i], acc2[i]);
      }
    } else {
      chain_vec<DT, OP>(a.sb + eb, a.ss, N, c - ca < 0 ? c - ca + N : c - ca, 1, ca + 1, lane, acc);
      if (cb > 0) {
        A acc2[V];
        chain_vec<DT, OP>(a.sb + eb, a.ss, N, c + cb >= N ? c + cb - N : c + cb, -1, cb, lane, acc2);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = opf<DT, OP>(acc[i], acc2[i]);
      }
    }
    const u32x4 w = pack<DT>(acc);
    char* d = a.rb + eb;
    for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, w);
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const int c = (int)chunk_of(a.M, N, e);
      A acc = chain_elem<DT, OP>(a.sb, a.ss, N, c - ca < 0 ? c - ca + N : c - ca, 1, ca + 1, e * SZ);
      if (cb > 0)
        acc = opf<DT, OP>(acc, chain_elem<DT, OP>(a.sb, a.ss, N, c + cb >= N ? c + cb - N : c + cb, -1, cb, e * SZ));
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, acc);
    }
  }
}

// ------------------------------------------------------------------ bucketed AllReduce

// Up to kMaxSeg independent AllReduces over element ranges (buckets) of the
// same rank buffers; bucket k has its own N chunks (boundaries relative to
// the bucket start).  Workgroup b works on tile (b - tile0[k]) of bucket k.
struct SegArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  int N;
  int nseg;
  uint32_t vecmask;                           // bit k: bucket k's start is 16-byte aligned
  uint32_t tile0[kMaxSeg + 1];                // prefix sums of tiles per bucket
  uint64_t off[kMaxSeg];                      // element offset of bucket k in every rank buffer
  uint32_t bnd[kMaxSeg][kMaxSegRanks + 1];    // chunk boundaries of bucket k, relative to it
};

template <int DT, int OP, int NR, int ALG>
__global__ __launch_bounds__(kBlock) void k_fused_seg(SegArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = NR > 0 ? NR : a.N;
  const uint32_t b = blockIdx.x;
  // bucket of this workgroup: an unrolled scan, so the prefix loads are
  // independent (one scalar-memory round trip instead of a search chain)
  // (unused prefix entries hold 0x7fffffff, above any workgroup index)
  // b >= t  <=>  the sign bit of t - 1 - b (all values < 2^31): integer
  // arithmetic on the scalar unit, no per-compare vector round trip
  uint32_t k = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i) k += (a.tile0[i] - 1u - b) >> 31;
  const uint32_t* bk = a.bnd[k];
  const uint64_t len = bk[N];
  const uint64_t tile = (uint64_t)kBlock * V;
  const uint64_t e0 = (uint64_t)(b - a.tile0[k]) * tile;
  const uint64_t e1 = e0 + tile < len ? e0 + tile : len;
  // chunk count: f >= bnd  <=>  f - bnd >= 0 (bucket lengths are < 2^31)
  const int32_t f0 = (int32_t)e0, f1 = (int32_t)(e1 - 1);
  int32_t c0 = 0, c1 = 0;
  if constexpr (NR > 0) {
#pragma unroll
    for (int i = 1; i < NR; ++i) {
      c0 += 1 + ((f0 - (int32_t)bk[i]) >> 31);
      c1 += 1 + ((f1 - (int32_t)bk[i]) >> 31);
    }
  } else {
    for (int i = 1; i < N; ++i) {
      c0 += 1 + ((f0 - (int32_t)bk[i]) >> 31);
      c1 += 1 + ((f1 - (int32_t)bk[i]) >> 31);
    }
  }
  const uint64_t base = a.off[k];
  if (((a.vecmask >> k) & 1) && e1 - e0 == tile && c0 == c1) {
    const uint32_t lane = threadIdx.x * 16u;
    const uint64_t eb = (base + e0) * SZ;
    A acc[V];
    fold_vec<DT, OP, NR, ALG>(a.sb + eb, a.ss, N, (int)c0, lane, acc);
    const u32x4 w = pack<DT>(acc);
    char* d = a.rb + eb;
    if constexpr (NR > 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r, d += a.rs) stg(d + lane, w);
    } else {
      for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, w);
    }
  } else {
    for (uint64_t e = e0 + threadIdx.x; e < e1; e += kBlock) {
      uint32_t c = 0;
      for (int i = 1; i < N; ++i) c += bk[i] <= e ? 1u : 0u;
      const uint64_t off = (base + e) * SZ;
      const A acc = fold_elem<DT, OP, NR, ALG, true>(a.sb, a.ss, N, (int)c, off);  // bucket trees: every leaf one rank
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + off, acc);
    }
  }
}

}  // namespace

hipError_t launch_dbt_fused(const Red& r) {
  FusedArgs a = fused_args(r);
  a.bnd[0] = 0;
  a.bnd[1] = r.M / 2;
  a.bnd[2] = r.M;
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = ar_fused_lds(r, r.blocks_per_cu);
  int nr = 2;
  while (nr < r.N) nr *= 2;
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
#define CC_DBT_CASE(NR)                                                                       \
  case NR:                                                                                     \
    if (r.N == NR)                                                                             \
      CC_LAUNCH((k_dbt_fused<DT, OP, NR, true>), grid, blk, lds, r.st, a);            \
    else                                                                                       \
      CC_LAUNCH((k_dbt_fused<DT, OP, NR, false>), grid, blk, lds, r.st, a);           \
    break;
    switch (nr) {
      CC_DBT_CASE(2)
      CC_DBT_CASE(4)
      CC_DBT_CASE(8)
      CC_DBT_CASE(16)
      default: return hipErrorInvalidValue;
    }
#undef CC_DBT_CASE
    return hipGetLastError();
  });
}

hipError_t launch_ring2_fused(const Red& r) {
  const FusedArgs a = fused_args(r);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = ar_fused_lds(r, r.blocks_per_cu);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    switch (r.N) {
      case 4: CC_LAUNCH((k_ring2_fused<DT, OP, 4, true>), grid, blk, lds, r.st, a); break;
      case 8: CC_LAUNCH((k_ring2_fused<DT, OP, 8, true>), grid, blk, lds, r.st, a); break;
      case 16: CC_LAUNCH((k_ring2_fused<DT, OP, 16, true>), grid, blk, lds, r.st, a); break;
      default:
        if (r.N <= 16) CC_LAUNCH((k_ring2_fused<DT, OP, 16, false>), grid, blk, lds, r.st, a);
        else CC_LAUNCH((k_ring2_fused<DT, OP, 0, false>), grid, blk, lds, r.st, a);
    }
    return hipGetLastError();
  });
}

hipError_t launch_fused_seg(const SegLaunch& L) {
  SegArgs a;
  a.sb = L.send.base; a.ss = L.send.stride;
  a.rb = L.recv.base; a.rs = L.recv.stride;
  a.N = L.N; a.nseg = L.nseg; a.vecmask = 0;
  const int es = elem_size(L.dt);
  const uint64_t tile = (uint64_t)kBlock * vec_elems(L.dt);
  const bool sides_al = ((((uintptr_t)L.send.base | (uintptr_t)L.recv.base | L.send.stride | L.recv.stride) & 15u) == 0);
  for (int k = 0; k <= kMaxSeg; ++k) a.tile0[k] = 0x7fffffffu;
  a.tile0[0] = 0;
  for (int k = 0; k < L.nseg; ++k) {
    a.off[k] = L.off[k];
    for (int c = 0; c <= L.N; ++c) a.bnd[k][c] = (uint32_t)(((unsigned __int128)c * L.len[k]) / (unsigned)L.N);
    a.tile0[k + 1] = a.tile0[k] + (uint32_t)((L.len[k] + tile - 1) / tile);
    if (sides_al && ((L.off[k] * es) & 15u) == 0) a.vecmask |= 1u << k;
  }
  if (a.tile0[L.nseg] == 0) return hipSuccess;
  const dim3 grid(a.tile0[L.nseg]), blk(kBlock);
  const unsigned lds = occupancy_lds(L.blocks_per_cu, kVecBytes * 2 * L.N, kBalancedTarget, 2);
  return by_dt_op(L.dt, L.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    if (L.alg == ALG_RING) {
      switch (L.N) {
        case 4: CC_LAUNCH((k_fused_seg<DT, OP, 4, ALG_RING>), grid, blk, lds, L.st, a); break;
        case 8: CC_LAUNCH((k_fused_seg<DT, OP, 8, ALG_RING>), grid, blk, lds, L.st, a); break;
        case 16: CC_LAUNCH((k_fused_seg<DT, OP, 16, ALG_RING>), grid, blk, lds, L.st, a); break;
        default: CC_LAUNCH((k_fused_seg<DT, OP, 0, ALG_RING>), grid, blk, lds, L.st, a); break;
      }
    } else {
#define CC_SEG_CASE(NR)                                                                        \
  case NR:                                                                                     \
    if (L.alg == ALG_HD)                                                                       \
      CC_LAUNCH((k_fused_seg<DT, OP, NR, ALG_HD>), grid, blk, lds, L.st, a);          \
    else                                                                                       \
      CC_LAUNCH((k_fused_seg<DT, OP, NR, ALG_BFLY>), grid, blk, lds, L.st, a);        \
    break;
      switch (L.N) {
        CC_SEG_CASE(2)
        CC_SEG_CASE(4)
        CC_SEG_CASE(8)
        CC_SEG_CASE(16)
        default: return hipErrorInvalidValue;
      }
#undef CC_SEG_CASE
    }
    return hipGetLastError();
  });
}

}  // namespace cc
