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

constexpr int kCopyVecs = 2;                                  // 16-byte vectors per thread and tile
constexpr uint64_t kCopyRow = (uint64_t)kCopyBlock * 16;       // one vector per thread
constexpr uint64_t kCopyTile = kCopyRow * kCopyVecs;           // 4 KiB

// Flat tiling over a list of copies: workgroup b copies tile (b - tpre[k]) of
// descriptor k (found by binary search), so skewed block sizes still spread
// over the whole chip.  A thread moves two vectors, both loaded before either
// is stored, at 12 workgroups per CU by default.  Measured on the MI355X (the
// MoE dispatch, 8 ranks x 4096 tokens x top-8, rows of 7168 bf16; dropless /
// capacity-padded at C = 1.25, direct): one vector per thread (2 KiB tiles)
// at full occupancy 6.08-6.12 / 5.62-5.66 TB/s (pairwise); two vectors at
// full occupancy 6.38 / 5.94-5.99, at 12 per CU 6.53-6.55 / 6.24-6.28 (the
// combine 6.20-6.23 against 5.99-6.00); four vectors 6.06-6.34 / 5.70; 256
// threads of one vector 6.16-6.22 dropless.
constexpr int kCopiesBlocksPerCu = 12;

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
      for (uint64_t o = o0 + (uint64_t)threadIdx.x * 16; o < o1; o += kCopyRow) stg(dst + o, z);
    } else {
      for (uint64_t o = o0 + threadIdx.x; o < o1; o += kCopyBlock) dst[o] = 0;
    }
  } else if ((a.vecmask >> k) & 1) {
    const uint64_t p = o0 + (uint64_t)threadIdx.x * 16;
    u32x4 w[kCopyVecs];
#pragma unroll
    for (int u = 0; u < kCopyVecs; ++u)
      if (p + u * kCopyRow < o1) w[u] = ldg(src + p + u * kCopyRow);
#pragma unroll
    for (int u = 0; u < kCopyVecs; ++u)
      if (p + u * kCopyRow < o1) stg(dst + p + u * kCopyRow, w[u]);
  } else {
    for (uint64_t o = o0 + threadIdx.x; o < o1; o += kCopyBlock) dst[o] = src[o];
  }
}

}  // namespace

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
  const unsigned lds = lds_for_blocks_per_cu(blocks_per_cu > 0 ? blocks_per_cu : kCopiesBlocksPerCu);
  CC_LAUNCH(k_copies, grid, blk, lds, st, a);
  return hipGetLastError();
}

}  // namespace cc
