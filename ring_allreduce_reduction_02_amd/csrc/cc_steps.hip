// Stepwise kernels of the collective-reduction engine: ring ReduceScatter
// passes of k steps, halving-doubling and butterfly steps, AllGather passes,
// descriptor steps of the other schedules, and the one-launch stepwise ring
// whose passes are separated by grid-wide waits (the "AllReduce" algorithm
// notes, 算法一/二/四; textbook ch. 6 "集合通信", Ring AllReduce).

#include "cc_device.h"

namespace cc {
namespace {

// ------------------------------------------------------------------ ring steps

struct PassArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  char* wb;  // staging: one accumulator per element (the chunk's in-flight partial)
  uint64_t M;
  int N;
  int rs_mode;
  int vec_ok;
  int s0;
  int k;
  int pin_recv;  // partials live in the receiving rank's recv buffer
  int tpc_log2;  // chunks of exactly 2^k full tiles: log2 of k, else -1
  uint64_t bnd[kMaxRanks + 1];
};

// Ring ReduceScatter steps s0 .. s0+k-1 for every chunk: the partial that the
// step-(s0-1) receiver holds is read, the next k ranks' contributions are
// folded in, and the result is left where the step-(s0+k-1) receiver holds it.
template <int DT, int OP>
__device__ __forceinline__ void ring_pass_tile(const PassArgs& a, uint64_t tile, int s0, int k) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = a.N;
  const bool fin = s0 + k == N - 1;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(tile, a.tpc_log2) : tile_floor<V>(tile, a.M, N, a.vec_ok);
  if (t.fast) {
    const int c = (int)t.c;
    const int start = a.rs_mode ? wrapN(c + 1, N) : c;
    const uint64_t b0 = a.bnd[c];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t e = vec_elem(t.e0, u, V);
      A acc[V];
      if (s0 == 0)
        unpack<DT>(ldg(a.sb + (uint64_t)start * a.ss + e * SZ), acc);
      else if (a.pin_recv)
        unpack<DT>(ldg(a.rb + (uint64_t)wrapN(start + s0, N) * a.rs + e * SZ), acc);
      else
        ldw_vec<DT>(a.wb + e * 4, acc);
      for (int j = s0 + 1; j <= s0 + k; ++j) {
        A x[V];
        unpack<DT>(ldg(a.sb + (uint64_t)wrapN(start + j, N) * a.ss + e * SZ), x);
        opv<DT, OP>(x, acc);
      }
      if (fin) {
        if (a.rs_mode)
          stg(a.rb + (uint64_t)c * a.rs + (e - b0) * SZ, pack<DT>(acc));
        else
          stg(a.rb + (uint64_t)wrapN(start + N - 1, N) * a.rs + e * SZ, pack<DT>(acc));
      } else if (a.pin_recv) {
        stg(a.rb + (uint64_t)wrapN(start + s0 + k, N) * a.rs + e * SZ, pack<DT>(acc));
      } else {
        stw_vec<DT>(a.wb + e * 4, acc);
      }
    }
  } else {
    // Element-wise (a tile across chunk boundaries, a ragged tail, unaligned
    // buffers): a thread's V elements, kBlock apart, go in batches of G
    // whose loads are all issued before any is used, so their latencies
    // overlap; an idle slot loads the tile's first element and stores
    // nothing.
    // Two slots per batch: the passes run at up to 16 workgroups per CU
    // (eight waves per SIMD, 64 registers a lane), which four slots would
    // exceed.  Tile-relative element offsets keep the per-slot state to two
    // 32-bit words (offset, chain start); the chunk follows from the start.
    constexpr int G = 2;
    const char* const sb0 = a.sb + t.e0 * SZ;
    char* const rb0 = a.rb + t.e0 * SZ;
    char* const wb0 = a.wb + t.e0 * 4;
    for (int g0 = 0; g0 < V; g0 += G) {
      uint32_t lo[G];
      int sv[G];
      bool ok[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const uint32_t l = threadIdx.x + (uint32_t)(g0 + u) * kBlock;
        ok[u] = t.e0 + l < t.e1;
        lo[u] = ok[u] ? l : 0u;
        const int c = (int)chunk_of(a.M, N, t.e0 + lo[u]);
        sv[u] = a.rs_mode ? wrapN(c + 1, N) : c;
      }
      // The running partial's source is the same for the whole pass, so
      // each source gets the whole body as straight-line code: a per-slot
      // choice of load would make each loaded register a join of values,
      // and the copy into it would wait for the load before the next one
      // issues.
      auto body = [&](auto first) {
        A acc[G], x1[G];
#pragma unroll
        for (int u = 0; u < G; ++u) acc[u] = first(u);
        // the pass's first step (k >= 1) in the same straight-line block, so
        // its loads are issued beside the partial's
#pragma unroll
        for (int u = 0; u < G; ++u) x1[u] = ld1<DT>(sb0 + (uint64_t)wrapN(sv[u] + s0 + 1, N) * a.ss + lo[u] * SZ);
#pragma unroll
        for (int u = 0; u < G; ++u) acc[u] = opf<DT, OP>(x1[u], acc[u]);
        for (int j = s0 + 2; j <= s0 + k; ++j) {
          A x[G];
#pragma unroll
          for (int u = 0; u < G; ++u) x[u] = ld1<DT>(sb0 + (uint64_t)wrapN(sv[u] + j, N) * a.ss + lo[u] * SZ);
#pragma unroll
          for (int u = 0; u < G; ++u) acc[u] = opf<DT, OP>(x[u], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
          if (!ok[u]) continue;
          if (fin) {
            if (a.rs_mode) {
              const uint32_t c = (uint32_t)(sv[u] == 0 ? N - 1 : sv[u] - 1);
              st1<DT>(a.rb + (uint64_t)c * a.rs + (t.e0 + lo[u] - bound_of(a.M, N, c)) * SZ, acc[u]);
            } else {
              st1<DT>(rb0 + (uint64_t)wrapN(sv[u] + N - 1, N) * a.rs + lo[u] * SZ, acc[u]);
            }
          } else if (a.pin_recv) {
            st1<DT>(rb0 + (uint64_t)wrapN(sv[u] + s0 + k, N) * a.rs + lo[u] * SZ, acc[u]);
          } else {
            stw1<DT>(wb0 + lo[u] * 4, acc[u]);
          }
        }
      };
      if (s0 == 0)
        body([&](int u) { return ld1<DT>(sb0 + (uint64_t)sv[u] * a.ss + lo[u] * SZ); });
      else if (a.pin_recv)
        body([&](int u) { return ld1<DT>(rb0 + (uint64_t)wrapN(sv[u] + s0, N) * a.rs + lo[u] * SZ); });
      else
        body([&](int u) { return ldw1<DT>(wb0 + lo[u] * 4); });
    }
  }
}

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_ring_pass(PassArgs a) {
  ring_pass_tile<DT, OP>(a, blockIdx.x, a.s0, a.k);
}

// ------------------------------------------------------------------ halving-doubling steps

struct StepArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  char* wb;      // rank-strided accumulators (staging)
  uint64_t ws;
  uint64_t M;
  int N;
  int rs_mode;
  int vec_ok;
  int d;         // partner distance of this step
  int first;     // operands come from the send buffers
  int last;      // results are final (buffer type)
  int acc_recv;  // intermediate accumulators live in recv (else in wb)
  int tpc_log2;  // chunks of exactly 2^k full tiles: log2 of k, else -1
  uint64_t bnd[kMaxRanks + 1];
};

template <int DT>
__device__ __forceinline__ void step_load_vec(const StepArgs& a, int r, uint64_t e, typename Ty<DT>::A* x) {
  constexpr int SZ = Ty<DT>::SZ;
  if (a.first) unpack<DT>(ldg(a.sb + (uint64_t)r * a.ss + e * SZ), x);
  else if (a.acc_recv) unpack<DT>(ldg(a.rb + (uint64_t)r * a.rs + e * SZ), x);
  else ldw_vec<DT>(a.wb + (uint64_t)r * a.ws + e * 4, x);
}
template <int DT>
__device__ __forceinline__ typename Ty<DT>::A step_load1(const StepArgs& a, int r, uint64_t e) {
  constexpr int SZ = Ty<DT>::SZ;
  if (a.first) return ld1<DT>(a.sb + (uint64_t)r * a.ss + e * SZ);
  if (a.acc_recv) return ld1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ);
  return ldw1<DT>(a.wb + (uint64_t)r * a.ws + e * 4);
}
// intermediate (not last) store of rank r's accumulator
template <int DT>
__device__ __forceinline__ void step_store_vec(const StepArgs& a, int r, uint64_t e, const typename Ty<DT>::A* x) {
  constexpr int SZ = Ty<DT>::SZ;
  if (a.acc_recv) stg(a.rb + (uint64_t)r * a.rs + e * SZ, pack<DT>(x));
  else stw_vec<DT>(a.wb + (uint64_t)r * a.ws + e * 4, x);
}
template <int DT>
__device__ __forceinline__ void step_store1(const StepArgs& a, int r, uint64_t e, typename Ty<DT>::A x) {
  constexpr int SZ = Ty<DT>::SZ;
  if (a.acc_recv) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, x);
  else stw1<DT>(a.wb + (uint64_t)r * a.ws + e * 4, x);
}

// Recursive-halving step with distance d: before it, rank i holds the block
// range of the ranks that share its bits at and above d; the ranks agreeing
// with chunk c on those bits keep c and combine the partner's copy of it.
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_hd_rs_step(StepArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = a.N, d = a.d;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const int c = (int)t.c;
    const int base = c & ~(d - 1);
    const uint64_t b0 = a.bnd[c];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t e = vec_elem(t.e0, u, V);
      for (int m = 0; m < d; ++m) {
        const int i = base | m, p = i ^ d;
        A x[V], y[V];
        step_load_vec<DT>(a, i, e, x);
        step_load_vec<DT>(a, p, e, y);
        opv<DT, OP>(y, x);  // x = op(y, x): commutative, the tree is what counts
        if (a.last) {
          if (a.rs_mode) stg(a.rb + (uint64_t)c * a.rs + (e - b0) * SZ, pack<DT>(x));
          else stg(a.rb + (uint64_t)c * a.rs + e * SZ, pack<DT>(x));
        } else {
          step_store_vec<DT>(a, i, e, x);
        }
      }
    }
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const uint32_t c = chunk_of(a.M, N, e);
      const int base = (int)c & ~(d - 1);
      for (int m = 0; m < d; ++m) {
        const int i = base | m, p = i ^ d;
        A v = opf<DT, OP>(step_load1<DT>(a, p, e), step_load1<DT>(a, i, e));
        if (a.last) {
          if (a.rs_mode) st1<DT>(a.rb + (uint64_t)c * a.rs + (e - bound_of(a.M, N, c)) * SZ, v);
          else st1<DT>(a.rb + (uint64_t)c * a.rs + e * SZ, v);
        } else {
          step_store1<DT>(a, i, e, v);
        }
      }
    }
  }
}

// Butterfly step with distance d: every pair (i, i+d), i without bit d,
// exchanges the full vector and both keep op of the two.
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_bfly_step(StepArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const int N = a.N, d = a.d;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t e = vec_elem(t.e0, u, V);
      for (int i = 0; i < N; ++i) {
        if (i & d) continue;
        const int p = i | d;
        A x[V], y[V];
        step_load_vec<DT>(a, i, e, x);
        step_load_vec<DT>(a, p, e, y);
        opv<DT, OP>(y, x);
        if (a.last) {
          const u32x4 w = pack<DT>(x);
          stg(a.rb + (uint64_t)i * a.rs + e * SZ, w);
          stg(a.rb + (uint64_t)p * a.rs + e * SZ, w);
        } else {
          step_store_vec<DT>(a, i, e, x);
          step_store_vec<DT>(a, p, e, x);
        }
      }
    }
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      for (int i = 0; i < N; ++i) {
        if (i & d) continue;
        const int p = i | d;
        A v = opf<DT, OP>(step_load1<DT>(a, p, e), step_load1<DT>(a, i, e));
        if (a.last) {
          st1<DT>(a.rb + (uint64_t)i * a.rs + e * SZ, v);
          st1<DT>(a.rb + (uint64_t)p * a.rs + e * SZ, v);
        } else {
          step_store1<DT>(a, i, e, v);
          step_store1<DT>(a, p, e, v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ gathers

struct GatArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  uint64_t M;
  int N;
  int mode;  // 0: AllGather phase of AllReduce (all in recv); 1: standalone
  int vec_ok;
  int s0;
  int k;
  int tpc_log2;  // chunks of exactly 2^k full tiles: log2 of k, else -1
  uint64_t bnd[kMaxRanks + 1];
};

// Ring AllGather steps s0 .. s0+k-1: chunk c is copied from the rank that
// holds it before step s0 to the next k ranks along the ring.  In the
// AllReduce the owner of chunk c is rank c-1; in the standalone AllGather
// rank c starts with chunk c (its send buffer) and also keeps a copy.
template <int SZ>
__device__ __forceinline__ void ring_ag_tile(const GatArgs& a, uint64_t tile, int s0, int k) {
  constexpr int V = 16 / SZ;
  const int N = a.N;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(tile, a.tpc_log2) : tile_floor<V>(tile, a.M, N, a.vec_ok);
  if (t.fast) {
    const int c = (int)t.c;
    const uint64_t b0 = a.bnd[c];
    const bool from_send = a.mode == 1 && s0 == 0;
    const int holder = a.mode == 0 ? modN(c - 1 + s0, N) : wrapN(c + s0, N);
    const int first_dst = a.mode == 0 ? wrapN(holder + 1, N) : wrapN(holder + 1, N);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t e = vec_elem(t.e0, u, V);
      const u32x4 w = from_send ? ldg(a.sb + (uint64_t)c * a.ss + (e - b0) * SZ)
                                : ldg(a.rb + (uint64_t)holder * a.rs + e * SZ);
      if (from_send) stg(a.rb + (uint64_t)c * a.rs + e * SZ, w);
      for (int q = 0; q < k; ++q) stg(a.rb + (uint64_t)modN(first_dst + q, N) * a.rs + e * SZ, w);
    }
  } else {
    // element-wise: a thread's V elements are loaded before any is stored
    // (an idle slot loads the tile's first element and stores nothing)
    // (the chunk's start comes from its closed form: a per-lane read of the
    // bound table would be a load whose wait precedes the element's load)
    typedef typename std::conditional<SZ == 2, uint16_t, uint32_t>::type W;
    const bool from_send = a.mode == 1 && s0 == 0;
    W v[V];
    uint64_t ev[V];
    int cv[V], hv[V];
    bool ok[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const uint64_t e = t.e0 + threadIdx.x + (uint64_t)u * kBlock;
      ok[u] = e < t.e1;
      ev[u] = ok[u] ? e : t.e0;
      cv[u] = (int)chunk_of(a.M, N, ev[u]);
      const int h = cv[u] - 1 + s0;  // in [-1, 2N - 2]
      hv[u] = a.mode == 0 ? (h < 0 ? h + N : wrapN(h, N)) : wrapN(cv[u] + s0, N);
      const char* src = from_send ? a.sb + (uint64_t)cv[u] * a.ss + (ev[u] - bound_of(a.M, N, (uint32_t)cv[u])) * SZ
                                  : a.rb + (uint64_t)hv[u] * a.rs + ev[u] * SZ;
      v[u] = *(const W*)src;
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
      if (!ok[u]) continue;
      const uint64_t e = ev[u];
      if (from_send) *(W*)(a.rb + (uint64_t)cv[u] * a.rs + e * SZ) = v[u];
      for (int q = 0; q < k; ++q) *(W*)(a.rb + (uint64_t)wrapN(hv[u] + 1 + q, N) * a.rs + e * SZ) = v[u];
    }
  }
}

template <int SZ>
__global__ __launch_bounds__(kBlock) void k_ring_ag_pass(GatArgs a) {
  ring_ag_tile<SZ>(a, blockIdx.x, a.s0, a.k);
}

// The AllGather in one pass, with the N stores of a tile's vectors shared
// between G groups of kBlock threads: every group loads the tile's vectors of
// chunk c (the standalone AllGather's shard of rank c, or the AllReduce's
// chunk on its owner; the first load brings the lines into the XCD's L2, the
// other group finds them there) and stores them to ranks g, g + G, g + 2G,
// ...  Element-wise tiles run the pass's own path in the first group.
template <int SZ, int G>
__global__ __launch_bounds__(kBlock * G) void k_ag_groups(GatArgs a) {
  constexpr int V = 16 / SZ;
  const int N = a.N;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  const uint32_t g = threadIdx.x / kBlock, lane = threadIdx.x % kBlock;
  if (t.fast) {
    const int c = (int)t.c;
    const uint64_t e = t.e0 + (uint64_t)lane * V;
    if (a.mode == 1) {
      const u32x4 w = ldg(a.sb + (uint64_t)c * a.ss + (e - a.bnd[c]) * SZ);
      for (int r = (int)g; r < N; r += G) stg(a.rb + (uint64_t)r * a.rs + e * SZ, w);
    } else {  // AllReduce: from the owner, rank c-1, to every other rank
      const int own = c == 0 ? N - 1 : c - 1;
      const u32x4 w = ldg(a.rb + (uint64_t)own * a.rs + e * SZ);
      for (int r = (int)g; r < N; r += G)
        if (r != own) stg(a.rb + (uint64_t)r * a.rs + e * SZ, w);
    }
  } else if (g == 0) {
    ring_ag_tile<SZ>(a, blockIdx.x, 0, N - 1);
  }
}

// ------------------------------------------------------------------ descriptor steps

// One step of a schedule given as descriptors (tree, double tree, 2-port
// ring, halving-doubling and butterfly for N not a power of two).  Each
// descriptor covers elements [lo, lo+len) of the ranks it names:
//   copy:     recv[dst] = recv[in1]                       (finished values)
//   combine:  v = op(op(local, in1), in2)  (in1, in2 optional)
//             local = send[dst] or partial[dst]; in1/in2 = send or partial
//             of their rank; v goes to partial[dst] or, final, rounded to
//             recv[dst]; `both` stores it for rank in1 too (the butterfly's
//             pairwise exchange, done by one thread for both ranks).
// partial[r] is recv[r] when the accumulator type is the element type
// (int32, fp32), else an fp32 rank-strided staging buffer.
struct GArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  char* wb;       // fp32 partials (bf16), or nullptr: partials in recv
  uint64_t ws;
  int n;
  uint64_t vecmask;
  uint32_t tpre[kMaxGDesc + 1];
  GDesc d[kMaxGDesc];
};

template <int DT>
__device__ __forceinline__ char* part_ptr(const GArgs& a, int r, uint64_t e) {
  return a.wb ? a.wb + (uint64_t)r * a.ws + e * 4 : a.rb + (uint64_t)r * a.rs + e * Ty<DT>::SZ;
}

template <int DT>
__device__ __forceinline__ void part_load_vec(const GArgs& a, int r, uint64_t e, typename Ty<DT>::A* v) {
  if (a.wb)
    ldw_vec<DT>(a.wb + (uint64_t)r * a.ws + e * 4, v);
  else
    unpack<DT>(ldg(a.rb + (uint64_t)r * a.rs + e * Ty<DT>::SZ), v);
}

template <int DT>
__device__ __forceinline__ void part_store_vec(const GArgs& a, int r, uint64_t e, const typename Ty<DT>::A* v) {
  if (a.wb)
    stw_vec<DT>(a.wb + (uint64_t)r * a.ws + e * 4, v);
  else
    stg(a.rb + (uint64_t)r * a.rs + e * Ty<DT>::SZ, pack<DT>(v));
}

template <int DT>
__device__ __forceinline__ typename Ty<DT>::A part_load1(const GArgs& a, int r, uint64_t e) {
  return a.wb ? ldw1<DT>(a.wb + (uint64_t)r * a.ws + e * 4) : ld1<DT>(a.rb + (uint64_t)r * a.rs + e * Ty<DT>::SZ);
}

template <int DT>
__device__ __forceinline__ void part_store1(const GArgs& a, int r, uint64_t e, typename Ty<DT>::A v) {
  if (a.wb)
    stw1<DT>(a.wb + (uint64_t)r * a.ws + e * 4, v);
  else
    st1<DT>(a.rb + (uint64_t)r * a.rs + e * Ty<DT>::SZ, v);
}

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_gsteps(GArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  const uint32_t b = blockIdx.x;
  int k = 0;
  for (int step = kMaxGDesc / 2; step >= 1; step /= 2)
    if (k + step < a.n && a.tpre[k + step] <= b) k += step;
  const GDesc& g = a.d[k];
  const uint64_t tile = (uint64_t)kBlock * V;
  const uint64_t e0 = g.lo + (uint64_t)(b - a.tpre[k]) * tile;
  const uint64_t e1 = e0 + tile < g.lo + g.len ? e0 + tile : g.lo + g.len;
  const unsigned f = g.flags;
  if (((a.vecmask >> k) & 1) && e1 - e0 == tile) {
    const uint64_t e = e0 + (uint64_t)threadIdx.x * V;
    if (f & GD_COPY) {
      stg(a.rb + (uint64_t)g.dst * a.rs + e * SZ, ldg(a.rb + (uint64_t)g.in1 * a.rs + e * SZ));
      return;
    }
    A acc[V], y[V];
    if (f & GD_LOCAL_SEND) unpack<DT>(ldg(a.sb + (uint64_t)g.dst * a.ss + e * SZ), acc);
    else part_load_vec<DT>(a, g.dst, e, acc);
    if (f & GD_IN1) {
      if (f & GD_IN1_SEND) unpack<DT>(ldg(a.sb + (uint64_t)g.in1 * a.ss + e * SZ), y);
      else part_load_vec<DT>(a, g.in1, e, y);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = opf<DT, OP>(acc[i], y[i]);
    }
    if (f & GD_IN2) {
      if (f & GD_IN2_SEND) unpack<DT>(ldg(a.sb + (uint64_t)g.in2 * a.ss + e * SZ), y);
      else part_load_vec<DT>(a, g.in2, e, y);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = opf<DT, OP>(acc[i], y[i]);
    }
    if (f & GD_FINAL) {
      const u32x4 w = pack<DT>(acc);
      stg(a.rb + (uint64_t)g.dst * a.rs + e * SZ, w);
      if (f & GD_BOTH) stg(a.rb + (uint64_t)g.in1 * a.rs + e * SZ, w);
    } else {
      part_store_vec<DT>(a, g.dst, e, acc);
      if (f & GD_BOTH) part_store_vec<DT>(a, g.in1, e, acc);
    }
  } else {
    for (uint64_t e = e0 + threadIdx.x; e < e1; e += kBlock) {
      if (f & GD_COPY) {
        if constexpr (SZ == 2)
          *(uint16_t*)(a.rb + (uint64_t)g.dst * a.rs + e * 2) = *(const uint16_t*)(a.rb + (uint64_t)g.in1 * a.rs + e * 2);
        else
          *(uint32_t*)(a.rb + (uint64_t)g.dst * a.rs + e * 4) = *(const uint32_t*)(a.rb + (uint64_t)g.in1 * a.rs + e * 4);
        continue;
      }
      A acc = (f & GD_LOCAL_SEND) ? ld1<DT>(a.sb + (uint64_t)g.dst * a.ss + e * SZ) : part_load1<DT>(a, g.dst, e);
      if (f & GD_IN1)
        acc = opf<DT, OP>(acc, (f & GD_IN1_SEND) ? ld1<DT>(a.sb + (uint64_t)g.in1 * a.ss + e * SZ)
                                                  : part_load1<DT>(a, g.in1, e));
      if (f & GD_IN2)
        acc = opf<DT, OP>(acc, (f & GD_IN2_SEND) ? ld1<DT>(a.sb + (uint64_t)g.in2 * a.ss + e * SZ)
                                                  : part_load1<DT>(a, g.in2, e));
      if (f & GD_FINAL) {
        st1<DT>(a.rb + (uint64_t)g.dst * a.rs + e * SZ, acc);
        if (f & GD_BOTH) st1<DT>(a.rb + (uint64_t)g.in1 * a.rs + e * SZ, acc);
      } else {
        part_store1<DT>(a, g.dst, e, acc);
        if (f & GD_BOTH) part_store1<DT>(a, g.in1, e, acc);
      }
    }
  }
}

// ------------------------------------------------------------------ one-launch stepwise ring

// The stepwise ring AllReduce in one launch.  The passes (k ring steps each;
// ReduceScatter passes, then AllGather passes) are cut into claims of
// `claim` tiles; workgroups take claims from a queue in global order, and a
// claim of pass p starts only after every claim of pass p-1 has completed --
// a grid-wide barrier between steps.  Because claims are handed out in order,
// every claim a waiting workgroup depends on is held by a running workgroup,
// so the schedule cannot deadlock whatever number of workgroups is resident.
//
// bar[0]: next claim; bar[1]: timed-out flag; bar[2 + p]: completed claims
// of pass p.  All are cleared by k_clear_words before the launch.  A wait
// gives up after spin_ticks of the constant-rate wall clock and sets bar[1];
// once it is set no later wait of the launch waits, so every wave always
// exits (the results are then undefined and bar[1] tells the caller).
struct QueueArgs {
  PassArgs p;   // ReduceScatter passes (s0, k unused)
  GatArgs g;    // AllGather passes (s0, k unused)
  unsigned* bar;
  uint64_t spin_ticks;
  uint64_t ntiles;    // tiles per pass
  uint32_t claim;     // tiles per claim
  uint32_t nclaims;   // claims per pass
  int k;              // ring steps per pass
  int npass;          // ReduceScatter passes (as many AllGather passes follow)
};

// thread 0 only: wait until *w reaches target (or the launch has timed out)
__device__ __forceinline__ void wait_count(unsigned* w, unsigned target, unsigned* flag, uint64_t spin_ticks) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
    if (wall_clock64() - t0 > spin_ticks) {
      __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The claim index is shared through the first word of the launch's dynamic
// LDS (the occupancy reservation, at least 16 bytes): a static __shared__
// word would come on top of a reservation that may already be the whole LDS.
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_ring_queue(QueueArgs a) {
  extern __shared__ unsigned lds_words[];
  unsigned& s_q = lds_words[0];
  const int N = a.p.N, k = a.k, P = a.npass;
  const unsigned total = 2u * (unsigned)P * a.nclaims;
  int ready = 0;  // claims of passes <= ready may start
  for (;;) {
    if (threadIdx.x == 0) s_q = __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned q = s_q;
    if (q >= total) break;
    const int pass = (int)(q / a.nclaims);
    const uint64_t t0 = (uint64_t)(q - (unsigned)pass * a.nclaims) * a.claim;
    const uint64_t t1 = t0 + a.claim < a.ntiles ? t0 + a.claim : a.ntiles;
    if (pass > ready) {
      if (threadIdx.x == 0) {
        wait_count(a.bar + 2 + (pass - 1), a.nclaims, a.bar + 1, a.spin_ticks);
        // drop lines this CU and its L2 cached before pass-1 completed (one
        // invalidation serves the whole workgroup: its waves share the CU)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      ready = pass;
    }
    if (pass < P) {
      const int s0 = pass * k, kk = k < N - 1 - s0 ? k : N - 1 - s0;
      for (uint64_t t = t0; t < t1; ++t) ring_pass_tile<DT, OP>(a.p, t, s0, kk);
    } else {
      const int s0 = (pass - P) * k, kk = k < N - 1 - s0 ? k : N - 1 - s0;
      for (uint64_t t = t0; t < t1; ++t) ring_ag_tile<Ty<DT>::SZ>(a.g, t, s0, kk);
    }
    // publish the claim: every wave waits for its stores to reach the L2,
    // then one write-back of the L2 makes them visible to the other XCDs'
    // caches before the claim is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __builtin_amdgcn_s_waitcnt(0);  // the write-back has completed
      __hip_atomic_fetch_add(a.bar + 2 + pass, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Clears the queue words before the launch (a kernel, not a memset, so the
// pair can be captured in a graph).
__global__ void k_clear_words(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Recursive-doubling AllGather step with distance d: the ranks whose partner
// (rank XOR d) holds chunk c receive it.
template <int SZ>
__global__ __launch_bounds__(kBlock) void k_hd_ag_step(GatArgs a) {
  constexpr int V = 16 / SZ;
  const int N = a.N, d = a.s0, first = a.k;  // s0 carries d, k carries "first"
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const int c = (int)t.c;
    const uint64_t b0 = a.bnd[c];
    const int base = (c ^ d) & ~(d - 1);
    const bool from_send = a.mode == 1 && first;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t e = vec_elem(t.e0, u, V);
      if (from_send) {
        const u32x4 w = ldg(a.sb + (uint64_t)c * a.ss + (e - b0) * SZ);
        stg(a.rb + (uint64_t)c * a.rs + e * SZ, w);
        stg(a.rb + (uint64_t)(c ^ 1) * a.rs + e * SZ, w);
      } else {
        for (int m = 0; m < d; ++m) {
          const int i = base | m, p = i ^ d;
          stg(a.rb + (uint64_t)i * a.rs + e * SZ, ldg(a.rb + (uint64_t)p * a.rs + e * SZ));
        }
      }
    }
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const int c = (int)chunk_of(a.M, N, e);
      const int base = (c ^ d) & ~(d - 1);
      if (a.mode == 1 && first) {
        const char* src = a.sb + (uint64_t)c * a.ss + (e - bound_of(a.M, N, (uint32_t)c)) * SZ;
        for (int q = 0; q < 2; ++q) {
          char* dst = a.rb + (uint64_t)(q ? (c ^ 1) : c) * a.rs + e * SZ;
          if constexpr (SZ == 2) *(uint16_t*)dst = *(const uint16_t*)src;
          else *(uint32_t*)dst = *(const uint32_t*)src;
        }
      } else {
        for (int m = 0; m < d; ++m) {
          const int i = base | m, p = i ^ d;
          const char* src = a.rb + (uint64_t)p * a.rs + e * SZ;
          char* dst = a.rb + (uint64_t)i * a.rs + e * SZ;
          if constexpr (SZ == 2) *(uint16_t*)dst = *(const uint16_t*)src;
          else *(uint32_t*)dst = *(const uint32_t*)src;
        }
      }
    }
  }
}


}  // namespace

hipError_t launch_gsteps(const Red& r, const GDesc* d, int n) {
  GArgs a;
  a.sb = r.send.base; a.ss = r.send.stride;
  a.rb = r.recv.base; a.rs = r.recv.stride;
  a.wb = r.ws.base; a.ws = r.ws.stride;
  a.n = 0; a.vecmask = 0; a.tpre[0] = 0;
  const int es = elem_size(r.dt);
  const uint64_t tile = (uint64_t)kBlock * vec_elems(r.dt);
  for (int i = 0; i < n && a.n < kMaxGDesc; ++i) {
    if (d[i].len == 0) continue;
    const int j = a.n++;
    a.d[j] = d[i];
    a.tpre[j + 1] = a.tpre[j] + (uint32_t)((d[i].len + tile - 1) / tile);
    // vector path: the element offset keeps 16-byte alignment for the
    // elements and for the fp32 partials
    const bool al = r.vec_ok && ((d[i].lo * es) & 15u) == 0 && (!a.wb || ((d[i].lo * 4) & 15u) == 0);
    if (al) a.vecmask |= 1ull << j;
  }
  for (int j = a.n; j < kMaxGDesc; ++j) a.tpre[j + 1] = a.tpre[a.n];
  if (a.n == 0) return hipSuccess;
  const dim3 grid(a.tpre[a.n]), blk(kBlock);
  const unsigned lds = occupancy_lds(r.blocks_per_cu, kVecBytes * 4, kSkewedTarget);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    CC_LAUNCH((k_gsteps<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

hipError_t launch_ring_rs_pass(const Red& r, int s0, int k, int partial_in_recv) {
  if (k < 1 || s0 < 0 || s0 + k > r.N - 1) return hipErrorInvalidValue;  // a pass folds at least one step
  PassArgs a;
  a.sb = r.send.base; a.ss = r.send.stride;
  a.rb = r.recv.base; a.rs = r.recv.stride;
  a.wb = r.ws.base;
  a.M = r.M; a.N = r.N; a.rs_mode = r.rs_mode; a.vec_ok = r.vec_ok;
  a.s0 = s0; a.k = k; a.pin_recv = partial_in_recv;
  a.tpc_log2 = pow2_tiles_per_chunk(r.M, r.N, r.dt, r.vec_ok);
  for (int c = 0; c <= r.N; ++c) a.bnd[c] = r.bnd[c];
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = occupancy_lds(r.blocks_per_cu, kVecBytes * (k + 2), kSkewedTarget);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    CC_LAUNCH((k_ring_pass<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

constexpr int kQueueBlocksPerCu = 4;

hipError_t launch_ring_queue(const Red& r, int k, unsigned* bar) {
  if (k < 1 || r.N < 2) return hipErrorInvalidValue;  // every pass folds at least one step
  QueueArgs a;
  PassArgs& p = a.p;
  p.sb = r.send.base; p.ss = r.send.stride;
  p.rb = r.recv.base; p.rs = r.recv.stride;
  p.wb = r.ws.base;
  p.M = r.M; p.N = r.N; p.rs_mode = 0; p.vec_ok = r.vec_ok;
  p.s0 = 0; p.k = k; p.pin_recv = r.dt != DT_BF16;
  GatArgs& g = a.g;
  g.sb = r.send.base; g.ss = r.send.stride;
  g.rb = r.recv.base; g.rs = r.recv.stride;
  g.M = r.M; g.N = r.N; g.mode = 0; g.vec_ok = r.vec_ok; g.s0 = 0; g.k = k;
  for (int c = 0; c <= r.N; ++c) p.bnd[c] = g.bnd[c] = r.bnd[c];
  p.tpc_log2 = g.tpc_log2 = pow2_tiles_per_chunk(r.M, r.N, r.dt, r.vec_ok);
  a.bar = bar;
  a.k = k;
  a.npass = (r.N - 1 + k - 1) / k;
  a.ntiles = num_tiles(r.M, r.dt);
  int dev = 0, rate_khz = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate_khz <= 0)
    rate_khz = 100000;
  a.spin_ticks = (uint64_t)rate_khz * 2000;  // 2 s
  // about one claim per resident workgroup and pass.  Each claim ends with a
  // write-back of its XCD's L2, which costs about half a microsecond and
  // serialises within the XCD, so the default keeps claims few and large:
  // 4 workgroups per CU.
  const int bpc = r.blocks_per_cu > 0 ? r.blocks_per_cu : kQueueBlocksPerCu;
  const uint64_t slots = (uint64_t)bpc * (uint64_t)(cus > 0 ? cus : 1);
  a.claim = (uint32_t)((a.ntiles + slots - 1) / slots);
  a.nclaims = (uint32_t)((a.ntiles + a.claim - 1) / a.claim);
  unsigned lds = lds_for_blocks_per_cu(bpc);
  if (lds < 16) lds = 16;  // the claim word
  const DevInfo di = dev_info();
  if (di.lds_per_block > 0 && lds > (unsigned)di.lds_per_block) return hipErrorInvalidConfiguration;
  CC_LAUNCH(k_clear_words, dim3(1), dim3(256), 0, r.st, bar, 2 + 2 * a.npass);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid(a.nclaims), blk(kBlock);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    CC_LAUNCH((k_ring_queue<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

static StepArgs step_args(const Red& r, int d, int first, int last, int acc_in_recv) {
  StepArgs a;
  a.sb = r.send.base; a.ss = r.send.stride;
  a.rb = r.recv.base; a.rs = r.recv.stride;
  a.wb = r.ws.base; a.ws = r.ws.stride;
  a.M = r.M; a.N = r.N; a.rs_mode = r.rs_mode; a.vec_ok = r.vec_ok;
  a.d = d; a.first = first; a.last = last; a.acc_recv = acc_in_recv;
  a.tpc_log2 = pow2_tiles_per_chunk(r.M, r.N, r.dt, r.vec_ok);
  for (int c = 0; c <= r.N; ++c) a.bnd[c] = r.bnd[c];
  return a;
}

hipError_t launch_hd_rs_step(const Red& r, int d, int first, int last, int acc_in_recv) {
  const StepArgs a = step_args(r, d, first, last, acc_in_recv);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = occupancy_lds(r.blocks_per_cu, kVecBytes * 3 * d, kSkewedTarget);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    CC_LAUNCH((k_hd_rs_step<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

hipError_t launch_bfly_step(const Red& r, int d, int first, int last, int acc_in_recv) {
  const StepArgs a = step_args(r, d, first, last, acc_in_recv);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = occupancy_lds(r.blocks_per_cu, kVecBytes * 2 * r.N, kSkewedTarget);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    CC_LAUNCH((k_bfly_step<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

static GatArgs gat_args(const Gat& g, int s0, int k) {
  GatArgs a;
  a.sb = g.send.base; a.ss = g.send.stride;
  a.rb = g.recv.base; a.rs = g.recv.stride;
  a.M = g.M; a.N = g.N; a.mode = g.ag_mode; a.vec_ok = g.vec_ok;
  a.s0 = s0; a.k = k;
  a.tpc_log2 = pow2_tiles_per_chunk_v(g.M, g.N, 16 / g.esize, g.vec_ok);
  for (int c = 0; c <= g.N; ++c) a.bnd[c] = g.bnd[c];
  return a;
}

static unsigned gat_tiles(const Gat& g) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * (16 / g.esize);
  return (unsigned)((g.M + tile - 1) / tile);
}

hipError_t launch_ring_ag_pass(const Gat& g, int s0, int k) {
  const GatArgs a = gat_args(g, s0, k);
  const dim3 grid(gat_tiles(g)), blk(kBlock);
  const unsigned lds = occupancy_lds(g.blocks_per_cu, kVecBytes * (k + 2), kSkewedTarget);
  if (g.esize == 2) CC_LAUNCH((k_ring_ag_pass<2>), grid, blk, lds, g.st, a);
  else CC_LAUNCH((k_ring_ag_pass<4>), grid, blk, lds, g.st, a);
  return hipGetLastError();
}

// Store groups and workgroups per CU of the standalone AllGather, from
// sweeps on the MI355X (fp32 and bf16, 2 GiB of output, rows by the
// rank-stride rule; 1, 2, 4, 8 groups at 1-12 workgroups per CU).  Two groups
// at an occupancy that keeps about 64-100 KiB of a tile's traffic in flight
// per CU, against one thread storing to all N ranks at its own default, TB/s
// (fp32, two runs): N = 8 6.35-6.44 (5.52-5.72), 9 6.04 (5.71-5.85), 16
// 6.36-6.40 (5.93-6.11), 17 6.30-6.33 (5.89-6.06), 48 5.91-5.98 (4.10-4.18),
// 64 6.01 (4.67-4.86); four or eight groups came within 2% of two where they
// were not worse.  From 21 to 40 ranks and up to 7 one thread per vector
// streams as well or better (N = 24 5.97-6.15 against 5.87-5.90 with two
// groups, 33 6.13-6.24 against 5.78-5.81, 3-7 5.7-6.4).
// (Broadcast has the same one-to-N shape, but two groups did not beat its
// single-thread kernel: N = 8 5.23-5.31 against 5.86-5.94 TB/s at these
// occupancies, level within noise at 12-64 ranks.)
static int ag_groups(int N) { return (N >= 8 && N <= 20) || N > 40 ? 2 : 1; }
static int ag_blocks_per_cu(int N) { return N <= 12 ? 3 : N <= 20 ? 2 : 1; }

template <int SZ>
static hipError_t launch_ag_groups(const GatArgs& a, unsigned tiles, unsigned lds, hipStream_t st) {
  CC_LAUNCH((k_ag_groups<SZ, 2>), dim3(tiles), dim3(kBlock * 2), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_ag_fused(const Gat& g) {
  // the grouped kernel within 32-bit work-item counts
  const int G = (uint64_t)gat_tiles(g) * kBlock * ag_groups(g.N) <= 0xffffffffull ? ag_groups(g.N) : 1;
  if (G == 1) {
    // one group follows the write-heavy byte rule, capped at 10 workgroups
    // per CU below 6 ranks and at 8 from 6 on: the rule's 11-16 overfill the
    // write queues (fp32, 2 GiB per buffer: N = 4 6.35 TB/s at 10 against
    // 5.46 at the rule's 14; N = 2 6.44 against 5.82 at 16; N = 6 6.28 at 8
    // against 5.91 at 10)
    Gat c = g;
    if (c.blocks_per_cu <= 0) {
      const int b = default_blocks_per_cu(kVecBytes * (uint64_t)(g.N + 1), kSkewedTarget, 1);
      const int cap = g.N < 6 ? 10 : 8;
      c.blocks_per_cu = one_round_blocks(gat_tiles(g), b > cap ? cap : b);
    }
    return launch_ring_ag_pass(c, 0, g.N - 1);
  }
  const GatArgs a = gat_args(g, 0, g.N - 1);
  const unsigned tiles = gat_tiles(g);
  const int bpc = g.blocks_per_cu > 0 ? g.blocks_per_cu : one_round_blocks(tiles, ag_blocks_per_cu(g.N));
  const unsigned lds = lds_for_blocks_per_cu(bpc);
  return g.esize == 2 ? launch_ag_groups<2>(a, tiles, lds, g.st) : launch_ag_groups<4>(a, tiles, lds, g.st);
}

hipError_t launch_hd_ag_step(const Gat& g, int d, int first) {
  const GatArgs a = gat_args(g, d, first);
  const dim3 grid(gat_tiles(g)), blk(kBlock);
  const unsigned lds = occupancy_lds(g.blocks_per_cu, kVecBytes * 2 * d, kSkewedTarget);
  if (g.esize == 2) CC_LAUNCH((k_hd_ag_step<2>), grid, blk, lds, g.st, a);
  else CC_LAUNCH((k_hd_ag_step<4>), grid, blk, lds, g.st, a);
  return hipGetLastError();
}

}  // namespace cc
