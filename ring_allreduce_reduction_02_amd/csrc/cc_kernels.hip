// HIP kernels (gfx950 / CDNA4) of the collective-reduction engine.
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

#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "cc_launch.h"

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

// Chunk c holds [bnd[c], bnd[c+1]) with bnd[c] = floor(c*M/N) (computed on the
// host).  The chunk of an element e is the number of inner boundaries at or
// below e; with a workgroup-uniform e the loop runs on the scalar unit.
__device__ __forceinline__ uint32_t chunk_in(const uint64_t* bnd, int N, uint64_t e) {
  uint32_t c = 0;
  for (int i = 1; i < N; ++i) c += bnd[i] <= e ? 1u : 0u;
  return c;
}
// The same chunk when the bounds are exactly floor(c*M/N), as they are for
// every schedule's chunks: floor(c*M/N) <= e holds for c <= ((e+1)*N - 1)/M,
// so one quotient replaces the scan.  The quotient is below N <= 64: a float
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
// lies in one chunk, that chunk (uniform across the workgroup).
template <int V>
__device__ __forceinline__ Tile<V> tile_at(uint64_t idx, uint64_t M, const uint64_t* bnd, int N, int vec_ok) {
  const uint64_t tile = (uint64_t)kBlock * kUnroll * V;
  Tile<V> t;
  t.e0 = idx * tile;
  t.e1 = t.e0 + tile < M ? t.e0 + tile : M;
  const uint32_t c0 = chunk_in(bnd, N, t.e0);
  const uint32_t c1 = chunk_in(bnd, N, t.e1 - 1);
  t.c = c0;
  t.fast = vec_ok && (t.e1 - t.e0) == tile && c0 == c1;
  return t;
}
template <int V>
__device__ __forceinline__ Tile<V> tile_of(uint64_t M, const uint64_t* bnd, int N, int vec_ok) {
  return tile_at<V>(blockIdx.x, M, bnd, N, vec_ok);
}
// The same for chunks at the floor bounds floor(c M / N): the chunks of the
// tile's first and last element by the closed form, a fixed cost instead of
// a scan over the N+1 bounds (each step of which waits for a scalar load).
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

// ------------------------------------------------------------------ fused kernels

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

// AllReduce (rs_mode 0): every chunk's N-1 ReduceScatter steps folded in
// registers in the schedule's order, then the AllGather as N stores.
// ReduceScatter (rs_mode 1, ring and halving-doubling): only the owner is
// written; the ring's fold then starts one rank later.
template <int DT, int OP, int NR, int ALG>
__device__ __forceinline__ void fused_body(const FusedArgs& a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  static_assert(kUnroll == 1, "one 16-byte vector per thread");
  // ring: N ranks (NR when fixed at compile time); trees: the runtime rank
  // count, NR being the tree's leaf slots
  const int N = (ALG == ALG_RING && NR > 0) ? NR : a.N;
  // a tree AllReduce folds every element the same way whatever its chunk,
  // so only a ReduceScatter needs the chunk of a tile
  const int tiling = (ALG != ALG_RING && !a.rs_mode) ? 1 : N;
  const TreeShape ts{a.tree_leaves, a.tree_pairs};
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, tiling, a.vec_ok);
  if (t.fast) {
    // Every rank's tile starts at a workgroup-uniform address; a lane adds
    // its own 16-byte offset (scalar base + 32-bit vector offset).
    const int c = (int)t.c;
    const int start = (ALG == ALG_RING && a.rs_mode) ? wrapN(c + 1, N) : c;
    const uint32_t lane = threadIdx.x * 16u;
    const uint64_t eb = t.e0 * SZ;
    A acc[V];
    fold_vec<DT, OP, NR, ALG>(a.sb + eb, a.ss, N, start, lane, acc, ts);
    const u32x4 w = pack<DT>(acc);
    if (a.rs_mode) {
      stg(a.rb + (uint64_t)c * a.rs + (t.e0 - a.bnd[c]) * SZ + lane, w);
    } else {
      char* d = a.rb + eb;
      if constexpr (NR > 0) {
        if (N == NR) {  // the ring with NR > 0, a tree with every leaf slot used
#pragma unroll
          for (int r = 0; r < NR; ++r, d += a.rs) stg(d + lane, w);
        } else {
          for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, w);
        }
      } else {
        for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, w);
      }
    }
  } else {
    // Element-wise (a tile across chunk bounds, a ragged tail, unaligned
    // buffers): the thread's V elements, kBlock apart, are folded in
    // batches of G whose loads are in flight at once; an idle slot repeats
    // the tile's first element and stores nothing.  A tree folds one element
    // at a time (its fold already has NR loads in flight).
    constexpr int G = ALG == ALG_RING ? elem_batch<V, NR>() : 1;
    for (int g0 = 0; g0 < V; g0 += G) {
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
        st[u] = (ALG == ALG_RING && a.rs_mode) ? wrapN((int)cv[u] + 1, N) : (int)cv[u];
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
        if (a.rs_mode) {
          st1<DT>(a.rb + (uint64_t)cv[u] * a.rs + (ev[u] - bound_of(a.M, tiling, cv[u])) * SZ, acc[u]);
        } else {
          for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + off[u], acc[u]);
        }
      }
    }
  }
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kBlock) void k_ring_fused(FusedArgs a) {
  fused_body<DT, OP, NR, ALG_RING>(a);
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
  int p[kMaxHierLevels];
  int stride[kMaxHierLevels];
  uint32_t seg[kMaxRanks];
  uint64_t bnd[kMaxRanks + 1];
};

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

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void k_hier_fused(HierArgs a) {
  typedef typename Ty<DT>::A A;
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  static_assert(kMaxHierLevels == 4, "four levels");
  const int N = a.N;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_of<V>(a.M, a.bnd, N, a.vec_ok);
  if (t.fast) {
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
    const u32x4 o = pack<DT>(a3);
    char* d = a.rb + t.e0 * SZ;
    for (int r = 0; r < N; ++r, d += a.rs) stg(d + lane, o);
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const HierLv L = hier_lv(a, a.seg[chunk_in(a.bnd, N, e)]);
      HierPos fw = hier_begin(L);
      A a0[1], a1[1], a2[1], a3[1];
      for (int l = 0; l < N; ++l) {
        A x[1] = {ld1<DT>(a.sb + (uint64_t)hier_rank(L, fw) * a.ss + e * SZ)};
        hier_take<DT, OP, 1>(L, fw, x, a0, a1, a2, a3);
        hier_step(L, fw);
      }
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, a3[0]);
    }
  }
}

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

// ------------------------------------------------------------------ copies

struct BcArgs {
  const char* src;
  char* db;
  uint64_t ds;
  uint64_t nbytes;
  int N;
  int skip;
  int vec_ok;
};

constexpr int kCopyBlock = 128;
constexpr uint64_t kBcastTile = (uint64_t)kCopyBlock * 16;

// One read of the root's buffer, N (or N-1) writes.
__global__ __launch_bounds__(kCopyBlock) void k_bcast(BcArgs a) {
  const uint64_t b0 = (uint64_t)blockIdx.x * kBcastTile;
  const uint64_t b1 = b0 + kBcastTile < a.nbytes ? b0 + kBcastTile : a.nbytes;
  if (a.vec_ok && b1 - b0 == kBcastTile) {
    const uint64_t off = b0 + (uint64_t)threadIdx.x * 16;
    const u32x4 w = ldg(a.src + off);
    for (int r = 0; r < a.N; ++r)
      if (r != a.skip) stg(a.db + (uint64_t)r * a.ds + off, w);
  } else {
    for (uint64_t b = b0 + threadIdx.x; b < b1; b += kCopyBlock) {
      const uint8_t v = (uint8_t)a.src[b];
      for (int r = 0; r < a.N; ++r)
        if (r != a.skip) a.db[(uint64_t)r * a.ds + b] = (char)v;
    }
  }
}

struct CopyArgs {
  const char* src[kMaxDesc];
  char* dst[kMaxDesc];
  uint64_t bytes[kMaxDesc];
  uint64_t tpre[kMaxDesc + 1];  // prefix sums of tiles per descriptor
  uint64_t vecmask;             // bit i: descriptor i is 16-byte aligned
  int n;
  int esize;
};

constexpr uint64_t kCopyTile = (uint64_t)kCopyBlock * 16;

// Flat tiling over a list of copies: workgroup b copies tile (b - tpre[k]) of
// descriptor k (found by binary search), so skewed block sizes still spread
// over the whole chip.
__global__ __launch_bounds__(kCopyBlock) void k_copies(CopyArgs a) {
  const uint64_t b = blockIdx.x;
  int lo = 0, hi = a.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (b >= a.tpre[mid]) lo = mid; else hi = mid;
  }
  const int k = lo;
  const uint64_t o0 = (b - a.tpre[k]) * kCopyTile;
  const uint64_t nb = a.bytes[k];
  const uint64_t o1 = o0 + kCopyTile < nb ? o0 + kCopyTile : nb;
  const char* src = a.src[k];
  char* dst = a.dst[k];
  if (src == nullptr) {  // a fill descriptor: zeros
    if ((a.vecmask >> k) & 1) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (uint64_t o = o0 + (uint64_t)threadIdx.x * 16; o < o1; o += kCopyTile) stg(dst + o, z);
    } else {
      for (uint64_t o = o0 + threadIdx.x; o < o1; o += kCopyBlock) dst[o] = 0;
    }
  } else if ((a.vecmask >> k) & 1) {
    for (uint64_t o = o0 + (uint64_t)threadIdx.x * 16; o < o1; o += kCopyTile) stg(dst + o, ldg(src + o));
  } else {
    for (uint64_t o = o0 + threadIdx.x; o < o1; o += kCopyBlock) dst[o] = src[o];
  }
}

// ------------------------------------------------------------------ INT8 compression with error feedback

// Block-wise INT8 (one float32 scale per kQBlock elements of a rank's vector,
// blocks from element 0): u = g + e; s = max|u| / 127; q = round-half-even(u / s)
// clamped to [-127, 127] (0 when s = 0); v = q s; e <- u - v.  Every step is one
// IEEE float32 operation, so the values match a scalar evaluation bit for bit.
struct QArgs {
  const char* gb;  // gradients (DT), rank-strided
  uint64_t gs;
  char* eb;  // error accumulators (float32), rank-strided
  uint64_t es;
  char* qb;  // int8 values, rank-strided
  uint64_t qs;
  char* sb;  // float32 scales, rank-strided
  uint64_t ss;
  char* rb;  // results (DT), rank-strided
  uint64_t rs;
  uint64_t M;
  int N;
  int vec_ok;
  int tpc_log2;  // chunks of exactly 2^k full tiles: log2 of k, else -1
  uint64_t bnd[kMaxRanks + 1];
};

__device__ __forceinline__ float q_scale(float m) { return m / 127.0f; }
// q as the integer it is (through int32: rint of a small negative ratio is
// -0.0, an int8 has no signed zero, and v = q s must then be +0)
__device__ __forceinline__ float q_round(float u, float s) {
  if (s == 0.0f) return 0.0f;
  const float r = __builtin_rintf(u / s);
  return (float)(int32_t)(r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r));
}

// max over the LANES lanes (a power of two <= 32) holding one block
template <int LANES>
__device__ __forceinline__ float lane_group_max(float m) {
#pragma unroll
  for (int o = LANES / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// max over the 128 threads of the workgroup (two wavefronts); red holds two
// floats of dynamic LDS.  Every thread of the workgroup must call it.
__device__ __forceinline__ float workgroup_max(float m, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float r = fmaxf(red[0], red[1]);
  __syncthreads();
  return r;
}

// V int8 values <-> a lane's packed bytes
template <int V>
struct QPack;
template <>
struct QPack<4> {
  typedef uint32_t T;
  __device__ static T pack(const float* q) {
    T w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= ((uint32_t)(int32_t)q[i] & 0xffu) << (8 * i);
    return w;
  }
  __device__ static void unpack(T w, float* q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (float)(int8_t)(w >> (8 * i));
  }
};
template <>
struct QPack<8> {
  typedef uint2 T;
  __device__ static T pack(const float* q) {
    return make_uint2(QPack<4>::pack(q), QPack<4>::pack(q + 4));
  }
  __device__ static void unpack(T w, float* q) {
    QPack<4>::unpack(w.x, q);
    QPack<4>::unpack(w.y, q + 4);
  }
};

// The compression of one lane's V elements of one rank (fast path): returns
// v and writes e, and the int8 values and the block scale when Q is set.
template <int DT, bool Q>
__device__ __forceinline__ void quant_lane(const float* x, const float* e, float* v, char* ep, char* qp, char* sp) {
  constexpr int V = Ty<DT>::V;
  float u[V], m = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    u[i] = x[i] + e[i];
    m = fmaxf(m, fabsf(u[i]));
  }
  m = lane_group_max<kQBlock / V>(m);
  const float s = q_scale(m);
  float q[V], en[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    q[i] = q_round(u[i], s);
    v[i] = q[i] * s;
    en[i] = u[i] - v[i];
  }
  stw_vec<DT_F32>(ep, en);
  if constexpr (V == 8) stw_vec<DT_F32>(ep + 16, en + 4);
  if constexpr (Q) {
    *(typename QPack<V>::T*)qp = QPack<V>::pack(q);
    if ((threadIdx.x & (kQBlock / V - 1)) == 0) *(float*)sp = s;
  }
}

template <int DT>
__device__ __forceinline__ void load_ge(const QArgs& a, uint64_t e0, int r, uint32_t lane, float* x, float* e) {
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  unpack<DT>(ldg(a.gb + (uint64_t)r * a.gs + e0 * SZ + lane * 16u), x);
  const char* ep = a.eb + (uint64_t)r * a.es + (e0 + (uint64_t)lane * V) * 4;
  unpack<DT_F32>(ldg(ep), e);
  if constexpr (V == 8) unpack<DT_F32>(ldg(ep + 16), e + 4);
}

// Element-wise compression of the block starting at element b0 of rank r:
// every thread of the workgroup takes element b0 + threadIdx.x (if < e1).
template <int DT>
__device__ __forceinline__ float quant_elem_scale(const QArgs& a, uint64_t b0, uint64_t e1, int r, float* red,
                                                  float* u_out) {
  const uint64_t e = b0 + threadIdx.x;
  float u = 0.0f;
  if (e < e1) u = ld1<DT>(a.gb + (uint64_t)r * a.gs + e * Ty<DT>::SZ) + *(const float*)(a.eb + (uint64_t)r * a.es + e * 4);
  *u_out = u;
  return q_scale(workgroup_max(fabsf(u), red));
}

// The compression step alone: grid (tiles, ranks), writes the message.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_quant_ef(QArgs a) {
  extern __shared__ float qred[];
  constexpr int V = Ty<DT>::V;
  const int r = blockIdx.y;
  const uint64_t tile = (uint64_t)kBlock * V;
  const uint64_t e0 = (uint64_t)blockIdx.x * tile;
  const uint64_t e1 = e0 + tile < a.M ? e0 + tile : a.M;
  if (a.vec_ok && e1 - e0 == tile) {
    const uint32_t lane = threadIdx.x;
    float x[V], e[V], v[V];
    load_ge<DT>(a, e0, r, lane, x, e);
    const uint64_t el = e0 + (uint64_t)lane * V;
    quant_lane<DT, true>(x, e, v, a.eb + (uint64_t)r * a.es + el * 4, a.qb + (uint64_t)r * a.qs + el,
                         a.sb + (uint64_t)r * a.ss + (el / kQBlock) * 4);
  } else {
    for (uint64_t b0 = e0; b0 < e1; b0 += kQBlock) {
      float u;
      const float s = quant_elem_scale<DT>(a, b0, e1, r, qred, &u);
      const uint64_t e = b0 + threadIdx.x;
      if (e < e1) {
        const float q = q_round(u, s);
        *(float*)(a.eb + (uint64_t)r * a.es + e * 4) = u - q * s;
        *(int8_t*)(a.qb + (uint64_t)r * a.qs + e) = (int8_t)(int32_t)q;
      }
      if (threadIdx.x == 0) *(float*)(a.sb + (uint64_t)r * a.ss + (b0 / kQBlock) * 4) = s;
    }
  }
}

// The reduction of the messages: every element folds the dequantized values
// of all ranks in the ring order of its chunk, and every rank gets the result.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_dequant_reduce(QArgs a) {
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  typedef typename QPack<V>::T QT;
  const int N = a.N;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const uint64_t el = t.e0 + (uint64_t)threadIdx.x * V;
    const uint64_t sb = (el / kQBlock) * 4;
    float acc[V];
    int r = (int)t.c;
    for (int j0 = 0; j0 < N; j0 += 8) {
      QT qw[8];
      float sc[8];
      int rr = r;
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // past the last rank the loads repeat valid ones
        qw[k] = *(const QT*)(a.qb + (uint64_t)rr * a.qs + el);
        sc[k] = *(const float*)(a.sb + (uint64_t)rr * a.ss + sb);
        if (j0 + k + 1 < N) rr = rr + 1 == N ? 0 : rr + 1;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (j0 + k < N) {
          float q[V];
          QPack<V>::unpack(qw[k], q);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] = (j0 + k == 0) ? q[i] * sc[k] : q[i] * sc[k] + acc[i];
        }
      r = rr;  // the first rank of the next batch (rr moved past the last load)
    }
    const u32x4 o = pack<DT>(acc);
    char* d = a.rb + t.e0 * SZ;
    for (int k = 0; k < N; ++k, d += a.rs) stg(d + threadIdx.x * 16u, o);
  } else {
    for (uint64_t e = t.e0 + threadIdx.x; e < t.e1; e += kBlock) {
      const int c = (int)chunk_of(a.M, N, e);
      float acc = 0.0f;
      for (int j = 0, r = c; j < N; ++j, r = r + 1 == N ? 0 : r + 1) {
        const float v = (float)*(const int8_t*)(a.qb + (uint64_t)r * a.qs + e) *
                        *(const float*)(a.sb + (uint64_t)r * a.ss + (e / kQBlock) * 4);
        acc = j == 0 ? v : v + acc;
      }
      for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, acc);
    }
  }
}

// Compression and reduction in one pass, no message in memory.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_quant_ef_fused(QArgs a) {
  extern __shared__ float qred[];
  constexpr int V = Ty<DT>::V;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int B = 4;  // ranks loaded ahead of their compression
  const int N = a.N;
  const Tile<V> t = a.tpc_log2 >= 0 ? tile_pow2<V>(blockIdx.x, a.tpc_log2) : tile_floor<V>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const uint32_t lane = threadIdx.x;
    const uint64_t el = t.e0 + (uint64_t)lane * V;
    float acc[V];
    int r = (int)t.c;
    for (int j0 = 0; j0 < N; j0 += B) {
      float x[B][V], e[B][V];
      int rs[B];
      int rr = r;
#pragma unroll
      for (int k = 0; k < B; ++k) {  // past the last rank the loads repeat valid ones
        rs[k] = rr;
        load_ge<DT>(a, t.e0, rr, lane, x[k], e[k]);
        if (j0 + k + 1 < N) rr = rr + 1 == N ? 0 : rr + 1;
      }
#pragma unroll
      for (int k = 0; k < B; ++k)
        if (j0 + k < N) {
          float v[V];
          quant_lane<DT, false>(x[k], e[k], v, a.eb + (uint64_t)rs[k] * a.es + el * 4, nullptr, nullptr);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] = (j0 + k == 0) ? v[i] : v[i] + acc[i];
        }
      r = rr;  // the first rank of the next batch (rr moved past the last load)
    }
    const u32x4 o = pack<DT>(acc);
    char* d = a.rb + t.e0 * SZ;
    for (int k = 0; k < N; ++k, d += a.rs) stg(d + lane * 16u, o);
  } else {
    // per block: the N scales first (they need every element of the block),
    // then each element folds in the ring order of its own chunk
    float* scl = qred + 2;
    for (uint64_t b0 = t.e0; b0 < t.e1; b0 += kQBlock) {
      for (int r = 0; r < N; ++r) {
        float u;
        const float s = quant_elem_scale<DT>(a, b0, t.e1, r, qred, &u);
        if (threadIdx.x == 0) scl[r] = s;
      }
      __syncthreads();
      const uint64_t e = b0 + threadIdx.x;
      if (e < t.e1) {
        const int c = (int)chunk_of(a.M, N, e);
        float acc = 0.0f;
        for (int j = 0, r = c; j < N; ++j, r = r + 1 == N ? 0 : r + 1) {
          float* ep = (float*)(a.eb + (uint64_t)r * a.es + e * 4);
          const float u = ld1<DT>(a.gb + (uint64_t)r * a.gs + e * SZ) + *ep;
          const float v = q_round(u, scl[r]) * scl[r];
          *ep = u - v;
          acc = j == 0 ? v : v + acc;
        }
        for (int r = 0; r < N; ++r) st1<DT>(a.rb + (uint64_t)r * a.rs + e * SZ, acc);
      }
      __syncthreads();
    }
  }
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

// LDS reservation of a fused AllReduce that folds all N ranks of a tile and
// stores N results (2N vector accesses per workgroup).  A bf16 lane unpacks,
// folds and rounds eight elements per 16-byte vector (fp32: four), so from 8
// ranks on it wants more bytes in flight: at N = 8 in rows 256 KiB beyond
// the payload apart, 3 workgroups per CU against the byte rule's 2 took the
// ring from 6.19-6.21 to 6.43 TB/s and the trees, double tree and 2-port
// ring up 2.5-3.5% (halving-doubling 6.17 against 6.02); at N = 16 the rule
// gives 2 either way.
// (`blocks` > 0 overrides the choice.)
static unsigned ar_fused_lds(const Red& r, int blocks) {
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
static unsigned rs_fused_lds(const Red& r) {
  if (r.blocks_per_cu > 0) return lds_for_blocks_per_cu(r.blocks_per_cu);
  const int b = r.N < 8 ? default_blocks_per_cu(kVecBytes * (r.N + 1), kSkewedTarget, 1) : r.N <= 12 ? 4 : 3;
  return lds_for_blocks_per_cu(one_round_blocks(num_tiles(r.M, r.dt), b));
}

hipError_t launch_ring_fused(const Red& r) {
  const FusedArgs a = fused_args(r);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
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
      r.rs_mode ? rs_fused_lds(r)
      : runtime_n ? lds_for_blocks_per_cu(r.blocks_per_cu > 0 ? r.blocks_per_cu
                                                              : one_round_blocks(num_tiles(r.M, r.dt),
                                                                                 batched_ring_blocks_per_cu(r.N, r.dt)))
                  : ar_fused_lds(r, ring_bpc);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    switch (r.N) {
      case 2: hipLaunchKernelGGL((k_ring_fused<DT, OP, 2>), grid, blk, lds, r.st, a); break;
      case 3: hipLaunchKernelGGL((k_ring_fused<DT, OP, 3>), grid, blk, lds, r.st, a); break;
      case 4: hipLaunchKernelGGL((k_ring_fused<DT, OP, 4>), grid, blk, lds, r.st, a); break;
      case 8: hipLaunchKernelGGL((k_ring_fused<DT, OP, 8>), grid, blk, lds, r.st, a); break;
      case 16: hipLaunchKernelGGL((k_ring_fused<DT, OP, 16>), grid, blk, lds, r.st, a); break;
      default: hipLaunchKernelGGL((k_ring_fused<DT, OP, 0>), grid, blk, lds, r.st, a); break;
    }
    return hipGetLastError();
  });
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
      hipLaunchKernelGGL((k_tree_fused<DT, OP, NR, TREE_HD>), grid, blk, lds, r.st, a);       \
    else                                                                                      \
      hipLaunchKernelGGL((k_tree_fused<DT, OP, NR, TREE_BFLY>), grid, blk, lds, r.st, a);     \
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
  case NN: hipLaunchKernelGGL((k_btree_fused<DT, OP, NN>), grid, blk, lds, r.st, a); break;
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
      hipLaunchKernelGGL((k_tree_fused<DT, OP, NR, TREE_HD>), grid, blk, lds, r.st, a);       \
    else                                                                                      \
      hipLaunchKernelGGL((k_tree_fused<DT, OP, NR, TREE_BFLY>), grid, blk, lds, r.st, a);     \
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
      hipLaunchKernelGGL((k_dbt_fused<DT, OP, NR, true>), grid, blk, lds, r.st, a);            \
    else                                                                                       \
      hipLaunchKernelGGL((k_dbt_fused<DT, OP, NR, false>), grid, blk, lds, r.st, a);           \
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
      case 4: hipLaunchKernelGGL((k_ring2_fused<DT, OP, 4, true>), grid, blk, lds, r.st, a); break;
      case 8: hipLaunchKernelGGL((k_ring2_fused<DT, OP, 8, true>), grid, blk, lds, r.st, a); break;
      case 16: hipLaunchKernelGGL((k_ring2_fused<DT, OP, 16, true>), grid, blk, lds, r.st, a); break;
      default:
        if (r.N <= 16) hipLaunchKernelGGL((k_ring2_fused<DT, OP, 16, false>), grid, blk, lds, r.st, a);
        else hipLaunchKernelGGL((k_ring2_fused<DT, OP, 0, false>), grid, blk, lds, r.st, a);
    }
    return hipGetLastError();
  });
}

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
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = lds_for_blocks_per_cu(r.blocks_per_cu > 0 ? r.blocks_per_cu
                                                                 : one_round_blocks(num_tiles(r.M, r.dt), hier_blocks_per_cu(r.N)));
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    hipLaunchKernelGGL((k_hier_fused<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

namespace {
QArgs q_args(const QLaunch& L) {
  QArgs a;
  a.gb = L.g; a.gs = L.gs;
  a.eb = L.e; a.es = L.es;
  a.qb = L.q; a.qs = L.qs;
  a.sb = L.s; a.ss = L.ss;
  a.rb = L.r; a.rs = L.rs;
  a.M = L.M; a.N = L.N; a.vec_ok = L.vec_ok;
  a.tpc_log2 = L.bnd ? pow2_tiles_per_chunk(L.M, L.N, L.dt, L.vec_ok) : -1;
  for (int c = 0; c <= L.N; ++c) a.bnd[c] = L.bnd ? L.bnd[c] : 0;
  return a;
}
// dynamic LDS: the occupancy reservation (the caller's, else `dflt`
// workgroups per CU), and at least the element-wise paths' reduction words and
// per-rank scales
unsigned q_lds(int blocks_per_cu, int dflt) {
  const unsigned lds = lds_for_blocks_per_cu(blocks_per_cu > 0 ? blocks_per_cu : dflt);
  const unsigned need = (2 + kMaxRanks) * 4;
  return lds < need ? need : lds;
}
// Default workgroups per CU, swept on the MI355X at 8 ranks x 67,108,864
// elements (1 to 16 per CU): the compression step streams best at 16 for
// float32 gradients (1065 us against 1262 at 8) and 8 for bf16 (1040 us
// against 1068 at 16), the reduction of the messages at 8 (float32) / 6
// (bf16), the fused kernel, which keeps four ranks' loads in flight, at 4
// (float32) / 3 (bf16).
int quant_blocks_per_cu(int dt) { return dt == DT_F32 ? 16 : 8; }
int dequant_blocks_per_cu(int dt) { return dt == DT_F32 ? 8 : 6; }
int qfused_blocks_per_cu(int dt) { return dt == DT_F32 ? 4 : 3; }
}  // namespace

hipError_t launch_quant_ef(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16)) return hipErrorInvalidValue;
  const QArgs a = q_args(L);
  const dim3 grid((unsigned)num_tiles(L.M, L.dt), (unsigned)L.N), blk(kBlock);
  const unsigned lds = q_lds(L.blocks_per_cu, quant_blocks_per_cu(L.dt));
  if (L.dt == DT_F32) hipLaunchKernelGGL((k_quant_ef<DT_F32>), grid, blk, lds, L.st, a);
  else hipLaunchKernelGGL((k_quant_ef<DT_BF16>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

hipError_t launch_dequant_reduce(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16) || !L.bnd) return hipErrorInvalidValue;
  const QArgs a = q_args(L);
  const dim3 grid((unsigned)num_tiles(L.M, L.dt)), blk(kBlock);
  const unsigned lds = q_lds(L.blocks_per_cu, dequant_blocks_per_cu(L.dt));
  if (L.dt == DT_F32) hipLaunchKernelGGL((k_dequant_reduce<DT_F32>), grid, blk, lds, L.st, a);
  else hipLaunchKernelGGL((k_dequant_reduce<DT_BF16>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

hipError_t launch_quant_ef_fused(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16) || !L.bnd) return hipErrorInvalidValue;
  const QArgs a = q_args(L);
  const dim3 grid((unsigned)num_tiles(L.M, L.dt)), blk(kBlock);
  const unsigned lds = q_lds(L.blocks_per_cu, qfused_blocks_per_cu(L.dt));
  if (L.dt == DT_F32) hipLaunchKernelGGL((k_quant_ef_fused<DT_F32>), grid, blk, lds, L.st, a);
  else hipLaunchKernelGGL((k_quant_ef_fused<DT_BF16>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

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
    hipLaunchKernelGGL((k_gsteps<DT, OP>), grid, blk, lds, r.st, a);
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
    hipLaunchKernelGGL((k_ring_pass<DT, OP>), grid, blk, lds, r.st, a);
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
  hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(256), 0, r.st, bar, 2 + 2 * a.npass);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid(a.nclaims), blk(kBlock);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    hipLaunchKernelGGL((k_ring_queue<DT, OP>), grid, blk, lds, r.st, a);
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
    hipLaunchKernelGGL((k_hd_rs_step<DT, OP>), grid, blk, lds, r.st, a);
    return hipGetLastError();
  });
}

hipError_t launch_bfly_step(const Red& r, int d, int first, int last, int acc_in_recv) {
  const StepArgs a = step_args(r, d, first, last, acc_in_recv);
  const dim3 grid((unsigned)num_tiles(r.M, r.dt)), blk(kBlock);
  const unsigned lds = occupancy_lds(r.blocks_per_cu, kVecBytes * 2 * r.N, kSkewedTarget);
  return by_dt_op(r.dt, r.op, [&](auto dt, auto op) {
    constexpr int DT = decltype(dt)::value, OP = decltype(op)::value;
    hipLaunchKernelGGL((k_bfly_step<DT, OP>), grid, blk, lds, r.st, a);
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
  if (g.esize == 2) hipLaunchKernelGGL((k_ring_ag_pass<2>), grid, blk, lds, g.st, a);
  else hipLaunchKernelGGL((k_ring_ag_pass<4>), grid, blk, lds, g.st, a);
  return hipGetLastError();
}

// The standalone AllGather (one load, N stores per tile) follows the
// write-heavy byte rule, capped at 10 workgroups per CU below 6 ranks and at
// 8 from 6 on: the rule's 11-16 overfill the write queues (fp32, 2 GiB per
// buffer: N = 4 6.35 TB/s at 10 against 5.46 at the rule's 14; N = 2 6.44
// against 5.82 at 16; N = 6 6.28 at 8 against 5.91 at 10).
hipError_t launch_ag_fused(const Gat& g) {
  Gat c = g;
  if (c.blocks_per_cu <= 0) {
    const int b = default_blocks_per_cu(kVecBytes * (uint64_t)(g.N + 1), kSkewedTarget, 1);
    const int cap = g.N < 6 ? 10 : 8;
    c.blocks_per_cu = one_round_blocks(gat_tiles(g), b > cap ? cap : b);
  }
  return launch_ring_ag_pass(c, 0, g.N - 1);
}

hipError_t launch_hd_ag_step(const Gat& g, int d, int first) {
  const GatArgs a = gat_args(g, d, first);
  const dim3 grid(gat_tiles(g)), blk(kBlock);
  const unsigned lds = occupancy_lds(g.blocks_per_cu, kVecBytes * 2 * d, kSkewedTarget);
  if (g.esize == 2) hipLaunchKernelGGL((k_hd_ag_step<2>), grid, blk, lds, g.st, a);
  else hipLaunchKernelGGL((k_hd_ag_step<4>), grid, blk, lds, g.st, a);
  return hipGetLastError();
}

hipError_t launch_bcast(const char* src, Side dst, int N, int skip, uint64_t nbytes, int vec_ok,
                        int blocks_per_cu, hipStream_t st) {
  BcArgs a;
  a.src = src; a.db = dst.base; a.ds = dst.stride; a.nbytes = nbytes;
  a.N = N; a.skip = skip; a.vec_ok = vec_ok;
  const dim3 grid((unsigned)((nbytes + kBcastTile - 1) / kBcastTile)), blk(kCopyBlock);
  const int nw = skip >= 0 ? N - 1 : N;
  const unsigned lds = occupancy_lds(blocks_per_cu, kBcastTile * (nw + 1), kBcastTarget);
  hipLaunchKernelGGL(k_bcast, grid, blk, lds, st, a);
  return hipGetLastError();
}

hipError_t launch_copies(const CopyDesc* d, int n, int esize, int blocks_per_cu, hipStream_t st) {
  CopyArgs a;
  a.n = 0; a.esize = esize; a.vecmask = 0; a.tpre[0] = 0;
  for (int i = 0; i < n && i < kMaxDesc; ++i) {
    if (d[i].bytes == 0) continue;
    const int j = a.n++;
    a.src[j] = d[i].src; a.dst[j] = d[i].dst; a.bytes[j] = d[i].bytes;
    a.tpre[j + 1] = a.tpre[j] + (d[i].bytes + kCopyTile - 1) / kCopyTile;
    if ((((uintptr_t)d[i].src | (uintptr_t)d[i].dst | d[i].bytes) & 15u) == 0) a.vecmask |= 1ull << j;
  }
  if (a.n == 0) return hipSuccess;
  const dim3 grid((unsigned)a.tpre[a.n]), blk(kCopyBlock);
  const unsigned lds = blocks_per_cu > 0 ? lds_for_blocks_per_cu(blocks_per_cu) : 0;
  hipLaunchKernelGGL(k_copies, grid, blk, lds, st, a);
  return hipGetLastError();
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
        case 4: hipLaunchKernelGGL((k_fused_seg<DT, OP, 4, ALG_RING>), grid, blk, lds, L.st, a); break;
        case 8: hipLaunchKernelGGL((k_fused_seg<DT, OP, 8, ALG_RING>), grid, blk, lds, L.st, a); break;
        case 16: hipLaunchKernelGGL((k_fused_seg<DT, OP, 16, ALG_RING>), grid, blk, lds, L.st, a); break;
        default: hipLaunchKernelGGL((k_fused_seg<DT, OP, 0, ALG_RING>), grid, blk, lds, L.st, a); break;
      }
    } else {
#define CC_SEG_CASE(NR)                                                                        \
  case NR:                                                                                     \
    if (L.alg == ALG_HD)                                                                       \
      hipLaunchKernelGGL((k_fused_seg<DT, OP, NR, ALG_HD>), grid, blk, lds, L.st, a);          \
    else                                                                                       \
      hipLaunchKernelGGL((k_fused_seg<DT, OP, NR, ALG_BFLY>), grid, blk, lds, L.st, a);        \
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
