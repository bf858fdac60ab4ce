// Copy kernels of the collective-reduction engine: broadcast from one source
// to N rank buffers, and descriptor copies (AllToAll(v) blocks and its
// variants, rank copies).  No arithmetic.

#include "cc_device.h"

namespace cc {
namespace {

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

// ------------------------------------------------------------------ capacity-padded MoE exchange

struct MoeArgs {
  const char* sb;
  uint64_t ss;
  char* db;
  uint64_t ds;
  uint64_t rowb;
  uint32_t cap, N, E, epr;
  uint32_t dispatch, vec_ok;
  uint32_t rows_pre[kMaxRanks + 1];  // token rows of the ranks before i
  uint32_t cnt[kMoeMaxBlocks];       // [N][E] rows token rank i routes to expert e
};

// rows of token rank i that precede its rows for expert e (sorted by expert)
__device__ __forceinline__ uint32_t moe_disp(const MoeArgs& a, uint32_t i, uint32_t e) {
  uint32_t d = 0;
  for (uint32_t x = 0; x < e; ++x) d += a.cnt[i * a.E + x];
  return d;
}

// Workgroup b writes output row b.  Dispatch: rows in the expert side's order
// (expert rank j, then token rank i and local expert l, then slot s): slot s
// of block (i, l) holds token row disp(i, e) + s when s < cnt(i, e), else
// zeros.  Combine: token rank i's rows in order: row r of expert e's rows
// comes back from slot r - disp(i, e) of block (i, l) on expert rank j when
// that slot was kept (below the capacity), else zeros.  The indices are
// uniform across the workgroup (scalar registers); the row is then a plain
// streaming copy.
__global__ __launch_bounds__(kCopyBlock) void k_moe_rows(MoeArgs a) {
  const uint32_t idx = blockIdx.x;
  const char* src = nullptr;
  char* dst;
  if (a.dispatch) {
    const uint32_t b = idx / a.cap, s = idx - b * a.cap;
    const uint32_t per_rank = a.N * a.epr;
    const uint32_t j = b / per_rank, rem = b - j * per_rank;
    const uint32_t i = rem / a.epr, l = rem - i * a.epr;
    const uint32_t e = j * a.epr + l;
    dst = a.db + (uint64_t)j * a.ds + ((uint64_t)rem * a.cap + s) * a.rowb;
    if (s < a.cnt[i * a.E + e]) src = a.sb + (uint64_t)i * a.ss + ((uint64_t)moe_disp(a, i, e) + s) * a.rowb;
  } else {
    uint32_t i = 0;
    while (i + 1 < a.N && a.rows_pre[i + 1] <= idx) ++i;
    const uint32_t r = idx - a.rows_pre[i];
    uint32_t e = 0, d = 0;
    while (e + 1 < a.E && d + a.cnt[i * a.E + e] <= r) d += a.cnt[i * a.E + e++];
    const uint32_t s = r - d;
    dst = a.db + (uint64_t)i * a.ds + (uint64_t)r * a.rowb;
    if (s < a.cap) {
      const uint32_t j = e / a.epr, l = e - j * a.epr;
      src = a.sb + (uint64_t)j * a.ss + ((uint64_t)(i * a.epr + l) * a.cap + s) * a.rowb;
    }
  }
  if (a.vec_ok) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (src) {
#pragma unroll 4
      for (uint64_t o = (uint64_t)threadIdx.x * 16; o < a.rowb; o += kCopyTile) stg(dst + o, ldg(src + o));
    } else {
      for (uint64_t o = (uint64_t)threadIdx.x * 16; o < a.rowb; o += kCopyTile) stg(dst + o, z);
    }
  } else {
    for (uint64_t o = threadIdx.x; o < a.rowb; o += kCopyBlock) dst[o] = src ? src[o] : (char)0;
  }
}

}  // namespace

bool moe_rows_fit(int N, int E, uint64_t cap, const uint64_t* cnt) {
  if (N < 1 || N > kMaxRanks || E < N || E % N || (uint64_t)N * E > (uint64_t)kMoeMaxBlocks) return false;
  if (cap == 0 || cap > 0xffffffffull) return false;
  uint64_t rows = 0;
  for (int i = 0; i < N; ++i) {
    uint64_t ri = 0;
    for (int e = 0; e < E; ++e) {
      if (cnt[(size_t)i * E + e] > 0xffffffffull) return false;
      ri += cnt[(size_t)i * E + e];
    }
    rows += ri;
  }
  // one workgroup of kCopyBlock threads per output row: the grid's x size and
  // its work-items within 31 and 32 bits
  const uint64_t lim = 0xffffffffull / kCopyBlock;
  return rows <= lim && (uint64_t)N * E * cap <= lim;
}

hipError_t launch_moe_rows(const MoeLaunch& L) {
  if (!moe_rows_fit(L.N, L.E, L.cap, L.cnt)) return hipErrorInvalidValue;
  MoeArgs a;
  a.sb = L.src; a.ss = L.ss; a.db = L.dst; a.ds = L.ds; a.rowb = L.rowb;
  a.cap = (uint32_t)L.cap; a.N = (uint32_t)L.N; a.E = (uint32_t)L.E; a.epr = (uint32_t)(L.E / L.N);
  a.dispatch = (uint32_t)L.dispatch;
  a.vec_ok = ((((uintptr_t)L.src | (uintptr_t)L.dst | L.ss | L.ds | L.rowb) & 15u) == 0);
  a.rows_pre[0] = 0;
  for (int i = 0; i < L.N; ++i) {
    uint64_t ri = 0;
    for (int e = 0; e < L.E; ++e) {
      a.cnt[i * L.E + e] = (uint32_t)L.cnt[(size_t)i * L.E + e];
      ri += L.cnt[(size_t)i * L.E + e];
    }
    a.rows_pre[i + 1] = a.rows_pre[i] + (uint32_t)ri;
  }
  const uint64_t rows = L.dispatch ? (uint64_t)L.N * L.E * L.cap : a.rows_pre[L.N];
  if (rows == 0 || L.rowb == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), blk(kCopyBlock);
  // 8 workgroups per CU by default: the C = 1.25 dispatch of 8 ranks x 4096
  // tokens (top-8 of 64 experts, rows of 14,336 bytes) ran at 5.66 TB/s
  // against 5.49 at full occupancy, the combine at 5.72 against 5.56
  const unsigned lds = lds_for_blocks_per_cu(L.blocks_per_cu > 0 ? L.blocks_per_cu : 8);
  CC_LAUNCH(k_moe_rows, grid, blk, lds, L.st, a);
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
  CC_LAUNCH(k_bcast, grid, blk, lds, st, a);
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
  CC_LAUNCH(k_copies, grid, blk, lds, st, a);
  return hipGetLastError();
}

}  // namespace cc
