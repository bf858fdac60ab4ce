// INT8 compression with error feedback and the AllReduce of the compressed
// contributions (textbook ch. 6 "集合通信": 量化：降低精度, 梯度通信的分块量化,
// 错误反馈与残差累积).

#include "cc_device.h"

namespace cc {
namespace {

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
};

// The compression kernels give every lane 4 consecutive elements of a rank,
// whatever the gradient type: the error accumulators (float32, 4 bytes per
// element) are then one 16-byte load and store per lane, and every store
// instruction of a wavefront writes one contiguous KiB (bf16 gradients and
// results move 8 bytes per lane, 512 contiguous bytes per instruction).  With
// 8 bf16 elements per lane the accumulators took two 16-byte stores per lane
// 32 bytes apart, each instruction covering half of every line it touched,
// and the DRAM saw 6% more write traffic than the kernel's output.
constexpr int kQLane = 4;
constexpr uint64_t kQTile = (uint64_t)kBlock * kQLane;  // 512 elements
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ void ld4(const char* p, float* x) {
  if constexpr (DT == DT_F32) {
    unpack<DT_F32>(ldg(p), x);
  } else {
    const u32x2 w = __builtin_nontemporal_load((const u32x2*)p);
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}
template <int DT>
__device__ __forceinline__ void st4(char* p, const float* x) {
  if constexpr (DT == DT_F32) {
    stg(p, pack<DT_F32>(x));
  } else {
    u32x2 w;
    w.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
    w.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
    __builtin_nontemporal_store(w, (u32x2*)p);
  }
}

__device__ __forceinline__ float q_scale(float m) { return m / 127.0f; }
// q = round-half-even(u / s) clamped to [-127, 127], as the integer it is
// (through int32: rint of a small negative ratio is -0.0, an int8 has no
// signed zero, and v = q s must then be +0).
// The quotient is needed only to the integer it rounds to.  u times the
// hardware reciprocal of s is within 2.5e-5 of the correctly rounded u / s
// (|u / s| <= 127 (1 + 2^-24); v_rcp_f32 within 1 ulp, the product within
// half an ulp); where that estimate lies more than 1e-4 away from every
// half-integer both round to the same integer, and elsewhere -- ties, NaN,
// infinities, and scales below 2^-100 whose reciprocal would not be normal --
// the IEEE division decides.  The results are those of the division alone.
__device__ __forceinline__ float q_round(float u, float s) {
  if (s == 0.0f) return 0.0f;
  const float est = u * __builtin_amdgcn_rcpf(s);
  const float frac = fabsf(est - __builtin_truncf(est));
  float r = __builtin_rintf(est);
  if (__builtin_expect(!(s >= 0x1p-100f && fabsf(frac - 0.5f) > 1e-4f), 0)) r = __builtin_rintf(u / s);
  return (float)(int32_t)(r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r));
}

// The value of another lane of the same 16-lane row, by DPP (no LDS trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max over the 32 lanes of a half-wavefront (one 128-element block at 4
// elements per lane), in every lane of it: within quads by DPP quad
// permutations (lanes i^1, i^2), across the quads of a 16-lane row by the
// half-row and row mirrors, and across the two rows by a swizzle that swaps
// lanes i and i^16.  A shuffle per step (ds_bpermute) cost an LDS round trip
// and a wait each time.  The maximum does not depend on the order.
__device__ __forceinline__ float half_wave_max(float m) {
  m = fmaxf(m, dpp_mov<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_mov<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_mov<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_mov<0x140>(m));  // row_mirror
  return fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x401F)));  // xor 16
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

// The compression of one lane's V elements of one rank (fast path): returns
// v and writes e, and the int8 values and the block scale when Q is set.
template <bool Q>
__device__ __forceinline__ void quant_lane(const float* x, const float* e, float* v, char* ep, char* qp, char* sp) {
  constexpr int V = kQLane;
  float u[V], m = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    u[i] = x[i] + e[i];
    m = fmaxf(m, fabsf(u[i]));
  }
  static_assert(kQBlock / V == 32, "a block is half a wavefront");
  m = half_wave_max(m);
  const float s = q_scale(m);
  float q[V], en[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    q[i] = q_round(u[i], s);
    v[i] = q[i] * s;
    en[i] = u[i] - v[i];
  }
  stw_vec<DT_F32>(ep, en);
  if constexpr (Q) {
    *(typename QPack<V>::T*)qp = QPack<V>::pack(q);
    if ((threadIdx.x & (kQBlock / V - 1)) == 0) *(float*)sp = s;
  }
}

template <int DT>
__device__ __forceinline__ void load_ge(const QArgs& a, uint64_t e0, int r, uint32_t lane, float* x, float* e) {
  constexpr int SZ = Ty<DT>::SZ;
  const uint64_t el = e0 + (uint64_t)lane * kQLane;
  ld4<DT>(a.gb + (uint64_t)r * a.gs + el * SZ, x);
  unpack<DT_F32>(ldg(a.eb + (uint64_t)r * a.es + el * 4), e);
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
  constexpr int V = kQLane;
  const int r = blockIdx.y;
  const uint64_t e0 = (uint64_t)blockIdx.x * kQTile;
  const uint64_t e1 = e0 + kQTile < a.M ? e0 + kQTile : a.M;
  if (a.vec_ok && e1 - e0 == kQTile) {
    const uint32_t lane = threadIdx.x;
    float x[V], e[V], v[V];
    load_ge<DT>(a, e0, r, lane, x, e);
    const uint64_t el = e0 + (uint64_t)lane * V;
    quant_lane<true>(x, e, v, a.eb + (uint64_t)r * a.es + el * 4, a.qb + (uint64_t)r * a.qs + el,
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
//
// A workgroup of kDqThreads threads takes a tile of kDqTile elements of every
// rank, 4 per thread.  The int8 values come in with 16-byte loads (a thread
// loads 16 values of one rank) and are staged in LDS, 8 ranks at a time;
// after the barrier each thread folds its 4 elements over those ranks and,
// at the end, stores its 4 results to every rank with one store each, so
// that every store instruction of a wavefront writes consecutive output (1
// KiB for float32 results).  Measured on the MI355X (8 ranks x 67,108,864,
// rows 256 MiB apart, three interleaved runs on one GPU): 1024-element tiles
// in the XCD order below 5.78 TB/s with float32 results and 6.04 with bf16;
// 2048-element tiles 5.63 and 5.86 in launch order, 5.49 and 6.02 in XCD
// order; the earlier design (128 threads of 16 elements, each storing 4
// times per rank after a wave-local LDS transpose) 5.75 and 5.71.
constexpr uint64_t kDqTile = 1024;
constexpr int kDqThreads = (int)(kDqTile / 4);
constexpr int kDqBatch = 8;                                   // ranks staged per pass
constexpr unsigned kDqLds = kDqBatch * (unsigned)kDqTile;     // their int8 values

// Workgroups go to the 8 XCDs in turn (workgroup b to XCD b mod 8), each XCD
// with its own L2.  The kDqLine tiles whose block scales share one 128-byte
// line are given to workgroups of one XCD, so that the line is fetched once:
// workgroup b = 8 slot + x takes tile ((slot / G) 8 + x) G + slot mod G, G =
// kDqLine, over the whole groups of 8 G tiles; the rest keep their index.
constexpr uint32_t kDqLine = (uint32_t)(32 * kQBlock / kDqTile);
__device__ __forceinline__ uint64_t dq_tile(uint32_t b, uint64_t tiles) {
  const uint64_t whole = tiles / (8 * kDqLine) * (8 * kDqLine);
  if (b >= whole) return b;
  const uint32_t x = b & 7u, slot = b >> 3;
  return ((uint64_t)(slot / kDqLine) * 8 + x) * kDqLine + slot % kDqLine;
}

template <int DT>
__global__ __launch_bounds__(kDqThreads) void k_dequant_reduce(QArgs a) {
  extern __shared__ uint32_t qst[];  // [kDqBatch][kDqTile / 4] words of 4 int8 values
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int LPR = (int)(kDqTile / 16);  // loading threads per rank
  constexpr int RPL = kDqThreads / LPR;      // ranks per load instruction
  const int N = a.N;
  const uint64_t t0 = dq_tile(blockIdx.x, gridDim.x) * kDqTile;
  const uint64_t t1 = t0 + kDqTile < a.M ? t0 + kDqTile : a.M;
  const uint32_t c0 = chunk_of(a.M, N, t0);
  if (a.vec_ok && t1 - t0 == kDqTile && c0 == chunk_of(a.M, N, t1 - 1)) {
    const uint32_t tid = threadIdx.x, ll = tid % LPR, ls = tid / LPR;
    const uint64_t e4 = t0 + (uint64_t)tid * 4;  // this thread's 4 elements
    const uint64_t sb = (e4 / kQBlock) * 4;
    float acc[4];
    int r = (int)c0;  // rank of the batch's first slot
    for (int j0 = 0; j0 < N; j0 += kDqBatch) {
      const int nb = N - j0 < kDqBatch ? N - j0 : kDqBatch;
      if (j0) __syncthreads();  // the previous batch is read out of LDS
      u32x4 w[kDqBatch / RPL];
#pragma unroll
      for (int q = 0; q < kDqBatch / RPL; ++q) {
        const int k = q * RPL + (int)ls;
        if (k < nb) {
          const int rk = r + k < N ? r + k : r + k - N;
          w[q] = ldg(a.qb + (uint64_t)rk * a.qs + t0 + (uint64_t)ll * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < kDqBatch / RPL; ++q) {
        const int k = q * RPL + (int)ls;
        if (k < nb) *(u32x4*)(qst + k * (int)(kDqTile / 4) + ll * 4) = w[q];
      }
      float sc[kDqBatch];
#pragma unroll
      for (int k = 0; k < kDqBatch; ++k)
        if (k < nb) {
          const int rk = r + k < N ? r + k : r + k - N;
          sc[k] = *(const float*)(a.sb + (uint64_t)rk * a.ss + sb);
        }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kDqBatch; ++k)
        if (k < nb) {
          const uint32_t qw = qst[k * (int)(kDqTile / 4) + tid];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float q = (float)(int8_t)(qw >> (8 * i));
            acc[i] = (j0 + k == 0) ? q * sc[k] : q * sc[k] + acc[i];
          }
        }
      r = r + nb < N ? r + nb : r + nb - N;
    }
    char* d = a.rb + e4 * SZ;
    for (int k = 0; k < N; ++k, d += a.rs) st4<DT>(d, acc);
  } else {
    for (uint64_t e = t0 + threadIdx.x; e < t1; e += kDqThreads) {
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

// Compression and reduction in one pass, no message in memory.  A workgroup
// takes U groups of kQTile elements (a thread's 4 elements in each) and
// walks the ranks B at a time, loading a batch's gradients and accumulators
// before it compresses them.  Measured on the MI355X (8 ranks x 67,108,864,
// rows by the rank-stride rule, two interleaved runs, best occupancy of 1-5
// workgroups per CU; TB/s of the kernel's bytes): U = 2, B = 1 5.85-5.88
// fp32 (3 per CU) and 5.91 bf16 (4); U = 1, B = 4 (the earlier form)
// 5.49-5.50 and 5.62; U = 2, B = 2 5.75-5.79 and 5.74-5.76; U = 4, B = 1
// 5.53 and 5.56-5.59; U = 4, B = 2 5.38 and 5.53-5.56.
constexpr int kQfU = 2, kQfB = 1;
template <int DT, int U>
__global__ __launch_bounds__(kBlock) void k_quant_ef_fused(QArgs a) {
  extern __shared__ float qred[];
  constexpr int V = kQLane;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int B = kQfB;  // ranks loaded ahead of their compression
  const int N = a.N;
  const Tile<V * U> t = a.tpc_log2 >= 0 ? tile_pow2<V * U>(blockIdx.x, a.tpc_log2)
                                        : tile_floor<V * U>(blockIdx.x, a.M, N, a.vec_ok);
  if (t.fast) {
    const uint32_t lane = threadIdx.x;
    float acc[U][V];
    int r = (int)t.c;
    for (int j0 = 0; j0 < N; j0 += B) {
      float x[B][U][V], e[B][U][V];
      int rs[B];
      int rr = r;
#pragma unroll
      for (int k = 0; k < B; ++k) {  // past the last rank the loads repeat valid ones
        rs[k] = rr;
#pragma unroll
        for (int u = 0; u < U; ++u) load_ge<DT>(a, t.e0 + u * kQTile, rr, lane, x[k][u], e[k][u]);
        if (j0 + k + 1 < N) rr = rr + 1 == N ? 0 : rr + 1;
      }
#pragma unroll
      for (int k = 0; k < B; ++k)
        if (j0 + k < N) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint64_t el = t.e0 + u * kQTile + (uint64_t)lane * V;
            float v[V];
            quant_lane<false>(x[k][u], e[k][u], v, a.eb + (uint64_t)rs[k] * a.es + el * 4, nullptr, nullptr);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[u][i] = (j0 + k == 0) ? v[i] : v[i] + acc[u][i];
          }
        }
      r = rr;  // the first rank of the next batch (rr moved past the last load)
    }
    char* d = a.rb + (t.e0 + (uint64_t)lane * V) * SZ;
    for (int k = 0; k < N; ++k, d += a.rs)
#pragma unroll
      for (int u = 0; u < U; ++u) st4<DT>(d + u * kQTile * SZ, acc[u]);
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

}  // namespace

namespace {
QArgs q_args(const QLaunch& L) {
  QArgs a;
  a.gb = L.g; a.gs = L.gs;
  a.eb = L.e; a.es = L.es;
  a.qb = L.q; a.qs = L.qs;
  a.sb = L.s; a.ss = L.ss;
  a.rb = L.r; a.rs = L.rs;
  a.M = L.M; a.N = L.N; a.vec_ok = L.vec_ok;
  a.tpc_log2 = pow2_tiles_per_chunk_v(L.M, L.N, kQLane, L.vec_ok);
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
// elements (2 to 16 per CU): the compression step streams best at 16 (float32
// gradients 6.41 TB/s against 5.69 at 8; bf16 6.46 against 5.17 at 8), the
// reduction of the messages at 4 for float32 results and 6 for bf16 (5.78 and
// 6.05 TB/s; 5.31 and 6.05 at 6, 5.54 and 5.51 at 4), the fused kernel at 3
// for float32 and 4 for bf16 (1-5 per CU: float32 5.85-5.88 against 2.79-5.19
// at 1, 2, 4, 5; bf16 5.91 against 5.28-5.49 at 3 and 5).
int quant_blocks_per_cu(int) { return 16; }
int dequant_blocks_per_cu(int dt) { return dt == DT_F32 ? 4 : 6; }
int qfused_blocks_per_cu(int dt) { return dt == DT_F32 ? 3 : 4; }
}  // namespace

hipError_t launch_quant_ef(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16)) return hipErrorInvalidValue;
  const QArgs a = q_args(L);
  const dim3 grid((unsigned)((L.M + kQTile - 1) / kQTile), (unsigned)L.N), blk(kBlock);
  const unsigned lds = q_lds(L.blocks_per_cu, quant_blocks_per_cu(L.dt));
  if (L.dt == DT_F32) CC_LAUNCH((k_quant_ef<DT_F32>), grid, blk, lds, L.st, a);
  else CC_LAUNCH((k_quant_ef<DT_BF16>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

hipError_t launch_dequant_reduce(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16)) return hipErrorInvalidValue;
  const QArgs a = q_args(L);  // vec_ok: int8 rows, scales and results 16-byte aligned (base and stride)
  const uint64_t tiles = (L.M + kDqTile - 1) / kDqTile;
  if (tiles > 0x7fffffffull) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles), blk(kDqThreads);
  unsigned lds = q_lds(L.blocks_per_cu, dequant_blocks_per_cu(L.dt));
  if (lds < kDqLds) lds = kDqLds;
  if (L.dt == DT_F32) CC_LAUNCH((k_dequant_reduce<DT_F32>), grid, blk, lds, L.st, a);
  else CC_LAUNCH((k_dequant_reduce<DT_BF16>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

hipError_t launch_quant_ef_fused(const QLaunch& L) {
  if (L.N < 1 || L.N > kMaxRanks || (L.dt != DT_F32 && L.dt != DT_BF16)) return hipErrorInvalidValue;
  constexpr int U = kQfU;
  QArgs a = q_args(L);
  a.tpc_log2 = pow2_tiles_per_chunk_v(L.M, L.N, kQLane * U, L.vec_ok);
  const dim3 grid((unsigned)((L.M + U * kQTile - 1) / (U * kQTile))), blk(kBlock);
  const unsigned lds = q_lds(L.blocks_per_cu, qfused_blocks_per_cu(L.dt));
  if (L.dt == DT_F32) CC_LAUNCH((k_quant_ef_fused<DT_F32, U>), grid, blk, lds, L.st, a);
  else CC_LAUNCH((k_quant_ef_fused<DT_BF16, U>), grid, blk, lds, L.st, a);
  return hipGetLastError();
}

}  // namespace cc
