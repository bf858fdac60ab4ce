// Device code shared by the kernel source files of the collective-reduction
// engine (cc_kernels.hip, cc_hier.hip, cc_copy.hip, cc_quant.hip): element
// types and their 16-byte packing, nontemporal loads and stores, the
// operators, chunk arithmetic, the schedules' fold orders, and the host-side
// launch helpers (type/operator dispatch, occupancy reservations).  Every
// definition has internal linkage, so each source file gets its own copy.
#pragma once

#include <stdint.h>

#include <cstdio>
#include <mutex>
#include <type_traits>

#include "cc_launch.h"
#include "cc_lds.h"

namespace cc {
namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct IC {
  static constexpr int value = V;
};

// ------------------------------------------------------------------ types

template <int DT>
struct Ty;
template <>
struct Ty<DT_I32> {
  typedef uint32_t A;  // accumulate in uint32: SUM/PROD wrap modulo 2^32
  static constexpr int V = 4;
  static constexpr int SZ = 4;
};
template <>
struct Ty<DT_F32> {
  typedef float A;
  static constexpr int V = 4;
  static constexpr int SZ = 4;
};
template <>
struct Ty<DT_BF16> {
  typedef float A;  // bf16 widened exactly; partials stay fp32
  static constexpr int V = 8;
  static constexpr int SZ = 2;
};

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet, sign kept),
// overflow carries into the exponent and gives +-inf.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;   // a select, not a branch
}

template <int DT>
__device__ __forceinline__ void unpack(u32x4 w, typename Ty<DT>::A* x) {
  if constexpr (DT == DT_I32) {
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  } else if constexpr (DT == DT_F32) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  } else {
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
  }
}

template <int DT>
__device__ __forceinline__ u32x4 pack(const typename Ty<DT>::A* x) {
  u32x4 w;
  if constexpr (DT == DT_I32) {
    w.x = x[0]; w.y = x[1]; w.z = x[2]; w.w = x[3];
  } else if constexpr (DT == DT_F32) {
    w.x = __float_as_uint(x[0]); w.y = __float_as_uint(x[1]);
    w.z = __float_as_uint(x[2]); w.w = __float_as_uint(x[3]);
  } else {
    w.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
    w.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
    w.z = bf16_rne(x[4]) | (bf16_rne(x[5]) << 16);
    w.w = bf16_rne(x[6]) | (bf16_rne(x[7]) << 16);
  }
  return w;
}

// accumulator <-> its 32-bit pattern (staging buffers hold accumulators)
template <int DT>
__device__ __forceinline__ typename Ty<DT>::A from_bits(uint32_t b) {
  if constexpr (DT == DT_I32) return b; else return __uint_as_float(b);
}
template <int DT>
__device__ __forceinline__ uint32_t to_bits(typename Ty<DT>::A a) {
  if constexpr (DT == DT_I32) return a; else return __float_as_uint(a);
}

// one element in the buffer type
template <int DT>
__device__ __forceinline__ typename Ty<DT>::A ld1(const char* p) {
  if constexpr (DT == DT_BF16) return __uint_as_float((uint32_t)(*(const uint16_t*)p) << 16);
  else if constexpr (DT == DT_F32) return *(const float*)p;
  else return *(const uint32_t*)p;
}
template <int DT>
__device__ __forceinline__ void st1(char* p, typename Ty<DT>::A v) {
  if constexpr (DT == DT_BF16) *(uint16_t*)p = (uint16_t)bf16_rne(v);
  else if constexpr (DT == DT_F32) *(float*)p = v;
  else *(uint32_t*)p = v;
}
// one accumulator in a staging buffer
template <int DT>
__device__ __forceinline__ typename Ty<DT>::A ldw1(const char* p) {
  return from_bits<DT>(*(const uint32_t*)p);
}
template <int DT>
__device__ __forceinline__ void stw1(char* p, typename Ty<DT>::A v) {
  *(uint32_t*)p = to_bits<DT>(v);
}

__device__ __forceinline__ u32x4 ldg(const char* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void stg(char* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }

// V accumulators in a staging buffer (4 bytes each, 16-byte aligned)
template <int DT>
__device__ __forceinline__ void ldw_vec(const char* p, typename Ty<DT>::A* x) {
#pragma unroll
  for (int q = 0; q < Ty<DT>::V / 4; ++q) {
    u32x4 w = ldg(p + 16 * q);
    x[4 * q + 0] = from_bits<DT>(w.x); x[4 * q + 1] = from_bits<DT>(w.y);
    x[4 * q + 2] = from_bits<DT>(w.z); x[4 * q + 3] = from_bits<DT>(w.w);
  }
}
template <int DT>
__device__ __forceinline__ void stw_vec(char* p, const typename Ty<DT>::A* x) {
#pragma unroll
  for (int q = 0; q < Ty<DT>::V / 4; ++q) {
    u32x4 w;
    w.x = to_bits<DT>(x[4 * q + 0]); w.y = to_bits<DT>(x[4 * q + 1]);
    w.z = to_bits<DT>(x[4 * q + 2]); w.w = to_bits<DT>(x[4 * q + 3]);
    stg(p + 16 * q, w);
  }
}

// ------------------------------------------------------------------ operators

// NaN if either is NaN, +0 over -0; written as selects so that a fold of
// loaded values stays straight-line code (its loads can all be in flight).
__device__ __forceinline__ float fmax_ieee(float a, float b) {
  const float eq = __uint_as_float(__float_as_uint(a) & __float_as_uint(b));  // a == b: +0 beats -0
  const float m = a > b ? a : (a == b ? eq : b);
  return (a != a || b != b) ? __uint_as_float(0x7fc00000u) : m;
}

template <int DT, int OP>
__device__ __forceinline__ typename Ty<DT>::A opf(typename Ty<DT>::A a, typename Ty<DT>::A b) {
  if constexpr (DT == DT_I32) {
    if constexpr (OP == OP_SUM) return a + b;
    else if constexpr (OP == OP_PROD) return a * b;
    else return (int32_t)a > (int32_t)b ? a : b;
  } else {
    if constexpr (OP == OP_SUM) return a + b;
    else if constexpr (OP == OP_PROD) return a * b;
    else return fmax_ieee(a, b);
  }
}

template <int DT, int OP>
__device__ __forceinline__ void opv(const typename Ty<DT>::A* x, typename Ty<DT>::A* acc) {
#pragma unroll
  for (int i = 0; i < Ty<DT>::V; ++i) acc[i] = opf<DT, OP>(x[i], acc[i]);
}

// ------------------------------------------------------------------ chunks

// Chunk c holds [floor(c*M/N), floor((c+1)*M/N)) for every schedule.  The
// chunk of an element e is the largest c with floor(c*M/N) <= e, which holds
// for c <= ((e+1)*N - 1)/M, so one quotient gives it with no scan over the
// N+1 bounds.  The quotient is below N <= 64: a float
// estimate through the reciprocal is within 2^-14 of num/M (each of the two
// conversions, the reciprocal and the product adds at most about 2^-23
// relative error), so its floor is off by at most one, and one 64-bit
// remainder check makes it exact -- a few instructions instead of the long
// expansion of a 64-bit integer division.
__device__ __forceinline__ float u64_to_f32(uint64_t x) {
  return (float)(uint32_t)(x >> 32) * 4294967296.0f + (float)(uint32_t)x;
}
__device__ __forceinline__ uint32_t chunk_of(uint64_t M, int N, uint64_t e) {
  const uint64_t num = (e + 1) * (uint64_t)N - 1;  // < M N
  uint32_t q = (uint32_t)(u64_to_f32(num) * __builtin_amdgcn_rcpf(u64_to_f32(M)));
  const int64_t rem = (int64_t)(num - (uint64_t)q * M);
  if (rem < 0) --q;
  else if ((uint64_t)rem >= M) ++q;
  return q;
}
// The floor bound floor(c M / N) itself, for a per-element chunk c: c M is
// exact in a double (c <= 64 and M below 2^41), the product with the
// rounded reciprocal of N is within 2^-5 of c M / N, and one integer check
// corrects the floor (no 64-bit division, and no load of the bound table
// with a per-lane index, whose wait would come before the next load).
__device__ __forceinline__ uint64_t bound_of(uint64_t M, int N, uint32_t c) {
  const uint64_t x = (uint64_t)c * M;
  uint64_t q = (uint64_t)((double)x * (1.0 / (double)N));
  if (q * (uint64_t)N > x) --q;
  else if ((q + 1) * (uint64_t)N <= x) ++q;
  return q;
}
__device__ __forceinline__ int wrapN(int r, int N) { return r >= N ? r - N : r; }
// Elements per batch in the element-wise paths: the batch's loads are all in
// flight together, and four slots keep the registers of a bf16 thread (eight
// elements) near those of an fp32 one.
constexpr int kElemBatch = 4;
// Slots per batch for a fold over NR ranks (a runtime-N ring: four ranks at a
// time): about 16 loads in flight, which fit the registers the compiler
// allots; beyond that it issues a slot's loads one after another.
template <int V, int NR>
__device__ constexpr int elem_batch() {
  const int g = 16 / (NR > 0 ? NR : 4);
  return g < 1 ? 1 : (g > V ? V : (g > kElemBatch ? kElemBatch : g));
}
__device__ __forceinline__ int modN(int r, int N) { return ((r % N) + N) % N; }

template <int V>
struct Tile {
  uint64_t e0, e1;
  uint32_t c;
  bool fast;
};

// The workgroup's element range and, when the whole tile is full-width and
// lies in one chunk, that chunk (uniform across the workgroup), from the
// closed-form chunks of the tile's first and last element.
template <int V>
__device__ __forceinline__ Tile<V> tile_floor(uint64_t idx, uint64_t M, int N, int vec_ok) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * V;
  Tile<V> t;
  t.e0 = idx * tile;
  t.e1 = t.e0 + tile < M ? t.e0 + tile : M;
  const uint32_t c0 = chunk_of(M, N, t.e0);
  const uint32_t c1 = chunk_of(M, N, t.e1 - 1);
  t.c = c0;
  t.fast = vec_ok && (t.e1 - t.e0) == tile && c0 == c1;
  return t;
}

__device__ __forceinline__ uint64_t vec_elem(uint64_t e0, int u, int V) {
  return e0 + ((uint64_t)u * kBlock + threadIdx.x) * (uint64_t)V;
}

// ------------------------------------------------------------------ fold orders

template <int L>
__device__ constexpr int bitrev(int t) {
  int r = 0;
  for (int i = 0; i < L; ++i)
    if (t & (1 << i)) r |= 1 << (L - 1 - i);
  return r;
}
template <int NR>
__device__ constexpr int ilog2() {
  int l = 0;
  while ((1 << l) < NR) ++l;
  return l;
}

// Pairwise tree over the leaves in load order t = 0..n-1 (n <= NR), adjacent
// pairs first (a binary counter keeps one partial per level).  For butterfly
// and the binomial tree the order is the leaf index itself (distance 1
// first); for halving-doubling it is the bit-reversed index, which pairs
// leaves at distance NR/2 first.  When n < NR the partials left on the levels
// set in n are merged from the smallest up, lower leaves on the left: the
// binomial tree's result at rank 0 when leaves n.. are absent.
// The code stays straight-line so that every load can be issued before the
// folds that wait for it: with n < NR (FULL false) the stack updates of
// absent leaves are discarded by selects, and with CLAMP their loads read
// leaf n-1 again (a loader that reads registers takes the leaf as is).
template <int DT, int OP, int NR, int TREE, bool FULL, bool CLAMP = !FULL, typename Load>
__device__ __forceinline__ void tree_fold(Load load, typename Ty<DT>::A* out, int V, int n) {
  typedef typename Ty<DT>::A A;
  constexpr int L = ilog2<NR>();
  constexpr int VM = Ty<DT>::V;
  A stk[L + 1][VM];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    const int r = TREE == TREE_HD ? bitrev<L>(t) : t;
    A v[VM];
    if constexpr (CLAMP)
      load(r < n ? r : n - 1, v);
    else
      load(r, v);
    // t's trailing one bits = the completed subtrees to its left
    int ones = 0;
    while ((t >> ones) & 1) ++ones;
#pragma unroll
    for (int l = 0; l < L; ++l) {
      if (l < ones) {
#pragma unroll
        for (int i = 0; i < VM; ++i)
          if (i < V) v[i] = opf<DT, OP>(stk[l][i], v[i]);
      }
    }
    const bool keep = FULL || t < n;
#pragma unroll
    for (int l = 0; l <= L; ++l)
      if (l == ones) {
#pragma unroll
        for (int i = 0; i < VM; ++i)
          if (i < V) stk[l][i] = keep ? v[i] : stk[l][i];
      }
  }
  if (FULL || n == NR) {
#pragma unroll
    for (int i = 0; i < VM; ++i)
      if (i < V) out[i] = stk[L][i];
    return;
  }
  bool have = false;
#pragma unroll
  for (int l = 0; l <= L; ++l)
    if ((n >> l) & 1) {
#pragma unroll
      for (int i = 0; i < VM; ++i)
        if (i < V) out[i] = have ? opf<DT, OP>(stk[l][i], out[i]) : stk[l][i];
      have = true;
    }
}

// ALG_BTREE: the binomial tree over exactly NR ranks (NR not a power of two),
// its leaf count fixed at compile time.
enum Alg { ALG_RING = 0, ALG_HD = 1, ALG_BFLY = 2, ALG_BTREE = 3 };

template <int N>
__device__ constexpr int pow2_ceil() {
  int p = 1;
  while (p < N) p *= 2;
  return p;
}

// Fold of one 16-byte vector of every rank, rank r's vector at
// s0 + r*ss + lane (s0 and ss workgroup-uniform, lane the lane's offset).
// Ring: the chain x_start, x_start+1, ... folded as acc = op(x_next, acc);
// trees: as above.  N is NR when NR > 0.
// Trees (halving-doubling, butterfly, binomial): leaf v of the tree is rank
// v + pairs, except that the first `pairs` leaves are the pair folds
// op(x_2v, x_2v+1) (N not a power of two: the first 2r ranks fold in pairs
// before the power-of-two schedule); `leaves` of them exist.
struct TreeShape {
  int leaves;
  int pairs;
};

template <int DT, int OP, int NR, int ALG>
__device__ __forceinline__ void fold_vec(const char* s0, uint64_t ss, int N, int start, uint32_t lane,
                                         typename Ty<DT>::A* acc, TreeShape ts = TreeShape{NR, 0}) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  if constexpr (ALG == ALG_BTREE) {
    tree_fold<DT, OP, pow2_ceil<NR>(), TREE_BFLY, false, false>(
        [&](int v, A* x) {
          if (v < NR) unpack<DT>(ldg(s0 + (uint64_t)v * ss + lane), x);
        },
        acc, V, NR);
  } else if constexpr (ALG != ALG_RING) {
    constexpr int TR = ALG == ALG_HD ? TREE_HD : TREE_BFLY;
    if (ts.leaves == NR && ts.pairs == 0) {
      tree_fold<DT, OP, NR, TR, true>(
          [&](int v, A* x) { unpack<DT>(ldg(s0 + (uint64_t)v * ss + lane), x); }, acc, V, NR);
    } else {
      // leaf v: op(x_2v, x_2v+1) for v < pairs, else x_(v+pairs); both loads
      // are issued either way (the second repeats the first's address)
      tree_fold<DT, OP, NR, TR, false>(
          [&](int v, A* x) {
            const bool pr = v < ts.pairs;
            const char* p = s0 + (uint64_t)(pr ? 2 * v : v + ts.pairs) * ss + lane;
            const u32x4 ra = ldg(p), rb = ldg(pr ? p + ss : p);
            A y[V];
            unpack<DT>(ra, x);
            unpack<DT>(rb, y);
#pragma unroll
            for (int i = 0; i < V; ++i) x[i] = pr ? opf<DT, OP>(x[i], y[i]) : x[i];
          },
          acc, V, ts.leaves);
    }
  } else if constexpr (NR > 0) {
    u32x4 raw[NR];
    const char* p = s0 + (uint64_t)start * ss;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      raw[j] = ldg(p + lane);
      p = (start + j + 1 == NR) ? s0 : p + ss;
    }
    unpack<DT>(raw[0], acc);
#pragma unroll
    for (int j = 1; j < NR; ++j) {
      A x[V];
      unpack<DT>(raw[j], x);
      opv<DT, OP>(x, acc);
    }
  } else {
    const char* p = s0 + (uint64_t)start * ss;
    unpack<DT>(ldg(p + lane), acc);
    int r = start;
    for (int j = 1; j < N; j += 8) {
      u32x4 raw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j + q < N) {
          r = r + 1 == N ? 0 : r + 1;
          p = r == 0 ? s0 : p + ss;
          raw[q] = ldg(p + lane);
        }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j + q < N) {
          A x[V];
          unpack<DT>(raw[q], x);
          opv<DT, OP>(x, acc);
        }
    }
  }
}

// The same fold for one element at byte offset `off` of every rank.  Trees:
// FULL when every leaf is one rank (ts = {NR, 0}), which loads each once.
template <int DT, int OP, int NR, int ALG, bool FULL = false>
__device__ __forceinline__ typename Ty<DT>::A fold_elem(const char* sb, uint64_t ss, int N, int start,
                                                        uint64_t off, TreeShape ts = TreeShape{NR, 0}) {
  typedef typename Ty<DT>::A A;
  if constexpr (ALG == ALG_BTREE) {
    A acc[Ty<DT>::V];
    tree_fold<DT, OP, pow2_ceil<NR>(), TREE_BFLY, false, false>(
        [&](int v, A* x) {
          if (v < NR) x[0] = ld1<DT>(sb + (uint64_t)v * ss + off);
        },
        acc, 1, NR);
    return acc[0];
  } else if constexpr (ALG != ALG_RING) {
    constexpr int TR = ALG == ALG_HD ? TREE_HD : TREE_BFLY;
    A acc[Ty<DT>::V];
    if constexpr (FULL) {
      tree_fold<DT, OP, NR, TR, true>([&](int v, A* x) { x[0] = ld1<DT>(sb + (uint64_t)v * ss + off); }, acc, 1, NR);
      return acc[0];
    }
    tree_fold<DT, OP, NR, TR, false>(
        [&](int v, A* x) {
          // both loads issued either way (the second repeats the first's
          // address when leaf v is a single rank): straight-line code
          const bool pr = v < ts.pairs;
          const uint64_t r0 = pr ? (uint64_t)(2 * v) : (uint64_t)(v + ts.pairs);
          const A xa = ld1<DT>(sb + r0 * ss + off);
          const A xb = ld1<DT>(sb + (pr ? r0 + 1 : r0) * ss + off);
          x[0] = pr ? opf<DT, OP>(xa, xb) : xa;
        },
        acc, 1, ts.leaves);
    return acc[0];
  } else {
    A acc = ld1<DT>(sb + (uint64_t)start * ss + off);
    for (int j = 1; j < N; ++j) acc = opf<DT, OP>(ld1<DT>(sb + (uint64_t)wrapN(start + j, N) * ss + off), acc);
    return acc;
  }
}

// The ring fold of one element in each of a thread's V slots (slot u: byte
// offset off[u], chain from rank st[u]), in fold_elem's order, with the
// slots' loads in flight together.  With a runtime N the chain goes four
// ranks at a time; past the chain's end a slot reloads its first rank and a
// select drops the value, so the code stays straight-line.
template <int DT, int OP, int NR, int V>
__device__ __forceinline__ void ring_fold_elems(const char* sb, uint64_t ss, int N, const int* st,
                                                const uint64_t* off, typename Ty<DT>::A* acc) {
  typedef typename Ty<DT>::A A;
#pragma unroll
  for (int u = 0; u < V; ++u) acc[u] = ld1<DT>(sb + (uint64_t)st[u] * ss + off[u]);
  if constexpr (NR > 0) {
#pragma unroll
    for (int j = 1; j < NR; ++j) {
      A x[V];
#pragma unroll
      for (int u = 0; u < V; ++u) x[u] = ld1<DT>(sb + (uint64_t)wrapN(st[u] + j, NR) * ss + off[u]);
#pragma unroll
      for (int u = 0; u < V; ++u) acc[u] = opf<DT, OP>(x[u], acc[u]);
    }
  } else {
    for (int j = 1; j < N; j += 4) {
      A x[4][V];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const int r = j + q < N ? wrapN(st[u] + j + q, N) : st[u];
          x[q][u] = ld1<DT>(sb + (uint64_t)r * ss + off[u]);
        }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < V; ++u) acc[u] = j + q < N ? opf<DT, OP>(x[q][u], acc[u]) : acc[u];
    }
  }
}

// The tile of workgroup idx when every chunk holds exactly 2^tpc_log2 full
// tiles: its chunk is a shift of the tile index, and it takes the vector path.
template <int V>
__device__ __forceinline__ Tile<V> tile_pow2(uint64_t idx, int tpc_log2) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * V;
  Tile<V> t;
  t.e0 = idx * tile;
  t.e1 = t.e0 + tile;
  t.c = (uint32_t)(idx >> tpc_log2);
  t.fast = true;
  return t;
}

// ------------------------------------------------------------------ dispatch

template <typename F>
hipError_t by_dt_op(int dt, int op, F f) {
  switch (dt * 3 + op) {
    case 0: return f(IC<DT_I32>{}, IC<OP_SUM>{});
    case 1: return f(IC<DT_I32>{}, IC<OP_MAX>{});
    case 2: return f(IC<DT_I32>{}, IC<OP_PROD>{});
    case 3: return f(IC<DT_F32>{}, IC<OP_SUM>{});
    case 4: return f(IC<DT_F32>{}, IC<OP_MAX>{});
    case 5: return f(IC<DT_F32>{}, IC<OP_PROD>{});
    case 6: return f(IC<DT_BF16>{}, IC<OP_SUM>{});
    case 7: return f(IC<DT_BF16>{}, IC<OP_MAX>{});
    case 8: return f(IC<DT_BF16>{}, IC<OP_PROD>{});
  }
  return hipErrorInvalidValue;
}

// log2 of the tiles per chunk when the M elements split into N chunks of
// exactly 2^k full tiles each (the chunk bounds bnd[c] = floor(c M / N) are
// then c 2^k tiles), else -1
int pow2_tiles_per_chunk_v(uint64_t M, int N, int velems, int vec_ok) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * velems;
  if (!vec_ok || N < 1 || M % ((uint64_t)N * tile)) return -1;
  const uint64_t tpc = M / N / tile;
  if (tpc == 0 || (tpc & (tpc - 1))) return -1;
  int k = 0;
  while ((1ull << k) < tpc) ++k;
  return k;
}
int pow2_tiles_per_chunk(uint64_t M, int N, int dt, int vec_ok) {
  return pow2_tiles_per_chunk_v(M, N, vec_elems(dt), vec_ok);
}
struct DevInfo {
  int lds_per_cu = 0;
  int lds_per_block = 0;
  int cus = 0;
};

// Per-device attributes, queried once per device; the lock makes calls from
// several host threads safe.
DevInfo dev_info() {
  static std::mutex mu;
  static DevInfo cache[64];
  static bool have[64] = {};
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) d = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!have[d]) {
    DevInfo i;
    if (hipDeviceGetAttribute(&i.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, d) != hipSuccess)
      i.lds_per_cu = 0;
    if (hipDeviceGetAttribute(&i.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, d) != hipSuccess)
      i.lds_per_block = 0;
    if (hipDeviceGetAttribute(&i.cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) i.cus = 0;
    cache[d] = i;
    have[d] = true;
  }
  return cache[d];
}

// Static LDS of a kernel (its __shared__ declarations), from the runtime.
unsigned kernel_static_lds(const void* k) {
  hipFuncAttributes at;
  return hipFuncGetAttributes(&at, k) == hipSuccess ? (unsigned)at.sharedSizeBytes : 0u;
}

// A launch whose static plus dynamic LDS would exceed the per-workgroup
// limit is refused before it reaches the GPU (the call reports
// CC_ERR_UNSUPPORTED).
hipError_t refuse_lds(unsigned static_bytes, unsigned dynamic_bytes) {
  char why[160];
  snprintf(why, sizeof why, "a kernel's LDS (%u static + %u reserved bytes) exceeds the %d bytes a workgroup may use",
           static_bytes, dynamic_bytes, dev_info().lds_per_block);
  refuse_launch(why);
  return hipErrorInvalidConfiguration;
}

}  // namespace

// Every kernel launch of the library: the LDS guard, then the launch.  The
// kernel's static LDS is queried once per launch site and instantiation.
#define CC_LAUNCH(K, GRID, BLK, LDS, ST, ...)                                                  \
  do {                                                                                          \
    static const unsigned cc_static_lds_ = ::cc::kernel_static_lds(reinterpret_cast<const void*>(K)); \
    if (!lds_fits(cc_static_lds_, (LDS), ::cc::dev_info().lds_per_block))                      \
      return ::cc::refuse_lds(cc_static_lds_, (LDS));                                           \
    hipLaunchKernelGGL(K, GRID, BLK, LDS, ST, __VA_ARGS__);                                     \
  } while (0)

namespace {
constexpr uint64_t kBalancedTarget = 64 * 1024;
constexpr uint64_t kSkewedTarget = 144 * 1024;
constexpr uint64_t kBcastTarget = 72 * 1024;
constexpr uint64_t kVecBytes = (uint64_t)kBlock * kUnroll * 16;   // one vector access of a workgroup

unsigned occupancy_lds(int requested, uint64_t traffic, uint64_t target, int min_blocks = 1) {
  return lds_for_blocks_per_cu(requested > 0 ? requested : default_blocks_per_cu(traffic, target, min_blocks));
}

// Fused AllReduce kernels with a runtime rank count keep one batch of leaf
// loads in flight per thread (8, plus the first leaf for the ring) whatever N
// is, so the byte rule above undersizes them at small N.  Measured on the
// MI355X (fused SUM, 2 GiB per buffer, 2 to 8 workgroups per CU): the fp32
// ring streams best with 4 up to N = 8, 3 up to 16 and 2 beyond.  A bf16
// lane also unpacks and rounds eight elements per vector and wants more
// workgroups: 6 up to N = 6 (N = 5: 6.32 TB/s against 5.69 at 4), 4 up to 12
// (N = 10: 5.92 against 5.50 at 3), 3 up to 16, 2 beyond.  The hierarchical
// kernel, whose per-leaf walk is longer, takes 3 up to 16 ranks (at 8 ranks
// in rows 256 MiB + 256 KiB apart 6.26-6.30 TB/s against 6.15-6.17 at 4 and
// 5.85 at 2) and 2 beyond (8x8 5.74 against 5.53 at 3, 4x4x4 5.67 against
// 5.47, 4x8 5.87 against 5.70; 2 GiB per buffer, unpadded rows).
int batched_ring_blocks_per_cu(int N, int dt) {
  if (dt == DT_BF16) return N <= 6 ? 6 : N <= 12 ? 4 : N <= 16 ? 3 : 2;
  return N <= 8 ? 4 : N <= 16 ? 3 : 2;
}
int hier_blocks_per_cu(int N) { return N <= 16 ? 3 : 2; }

// A fused AllReduce grid small enough to be resident all at once (at most 16
// workgroups per CU) runs best that way: its loads all issue in the first
// round instead of waiting for a second.  Raises `blocks` to the workgroups
// per CU that hold the whole grid.  Measured on the int32 ring at N = 4,
// 1,048,576 elements (2,048 tiles, graph replays): 6.75 us at 8 per CU
// against 7.35 at the byte rule's 4 with the buffers cache-resident, 8.32
// against 8.43 from HBM.  The fused ReduceScatter, AllGather and
// hierarchical AllReduce take the same rule (16 rotating buffer sets, fp32,
// 4,096 tiles: AllGather at N = 16 27.9 us against 32.6, ReduceScatter at
// N = 16 29.9 against 32.1, hierarchical 4x2 28.3 against 33.3).
int one_round_blocks(uint64_t tiles, int blocks) {
  const int cus = dev_info().cus;
  if (cus <= 0 || tiles > 16ull * (uint64_t)cus) return blocks;
  const int need = (int)((tiles + cus - 1) / cus);
  return need > blocks ? need : blocks;
}
}  // namespace

namespace {

// ------------------------------------------------------------------ fused AllReduce arguments

struct FusedArgs {
  const char* sb;
  uint64_t ss;
  char* rb;
  uint64_t rs;
  uint64_t M;
  int N;
  int rs_mode;
  int vec_ok;
  int tree_leaves;  // trees: leaves of the power-of-two tree (<= NR)
  int tree_pairs;   // trees: leading leaves that are pair folds
  // log2 of the tiles per chunk when every chunk is exactly 2^k full tiles
  // (M = N 2^k tiles) and the buffers are 16-byte aligned, else -1
  int tpc_log2;
  uint64_t bnd[kMaxRanks + 1];
};

FusedArgs fused_args(const Red& r) {
  FusedArgs a;
  a.sb = r.send.base; a.ss = r.send.stride;
  a.rb = r.recv.base; a.rs = r.recv.stride;
  a.M = r.M; a.N = r.N; a.rs_mode = r.rs_mode; a.vec_ok = r.vec_ok;
  a.tree_leaves = r.N; a.tree_pairs = 0;
  a.tpc_log2 = pow2_tiles_per_chunk(r.M, r.N, r.dt, r.vec_ok);
  for (int c = 0; c <= r.N; ++c) a.bnd[c] = r.bnd[c];
  return a;
}

// LDS reservation of a fused AllReduce that folds all N ranks of a tile and
// stores N results (2N vector accesses per workgroup).  A bf16 lane unpacks,
// folds and rounds eight elements per 16-byte vector (fp32: four), so from 8
// ranks on it wants more bytes in flight: at N = 8 in rows 256 KiB beyond
// the payload apart, 3 workgroups per CU against the byte rule's 2 took the
// ring from 6.19-6.21 to 6.43 TB/s and the trees, double tree and 2-port
// ring up 2.5-3.5% (halving-doubling 6.17 against 6.02); at N = 16 the rule
// gives 2 either way.
// (`blocks` > 0 overrides the choice.)
unsigned ar_fused_lds(const Red& r, int blocks) {
  if (blocks <= 0) {
    const uint64_t target = (r.dt == DT_BF16 && r.N >= 8) ? kBalancedTarget * 3 / 2 : kBalancedTarget;
    blocks = one_round_blocks(num_tiles(r.M, r.dt), default_blocks_per_cu(kVecBytes * 2 * r.N, target, 2));
  }
  return lds_for_blocks_per_cu(blocks);
}

// LDS reservation of a fused ReduceScatter (N loads, one store per tile; ring
// and halving-doubling).  The read-heavy byte rule holds up to 5 ranks but
// puts too many workgroups on a CU from 8 on.  Measured (2 GiB per buffer,
// rows 256 KiB beyond the payload apart), fp32 ring: N = 8 6.63 TB/s at 4
// against 6.44 at the rule's 8, N = 12 6.22 at 4 against 6.12 at 6, N = 16
// 6.67 at 3 against 6.54 at 4, N = 32 6.65 at 3 against 6.20 at 2;
// halving-doubling at N = 8: 6.56 (fp32) and 6.79 (bf16) at 4 against 6.25
// and 6.38 at 8.
unsigned rs_fused_lds(const Red& r) {
  if (r.blocks_per_cu > 0) return lds_for_blocks_per_cu(r.blocks_per_cu);
  const int b = r.N < 8 ? default_blocks_per_cu(kVecBytes * (r.N + 1), kSkewedTarget, 1) : r.N <= 12 ? 4 : 3;
  return lds_for_blocks_per_cu(one_round_blocks(num_tiles(r.M, r.dt), b));
}

}  // namespace

}  // namespace cc
