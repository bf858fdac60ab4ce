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

}  // namespace cc
