// C ABI of the collective-reduction engine: argument validation, schedule
// planning and kernel dispatch.  Declared in include/cc.h.

#include "../../include/cc.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "cc_api_internal.h"
#include "cc_launch.h"
#include "cc_sched.h"

using namespace cc;

namespace cc {
namespace api {

thread_local std::string g_err;

cc_status_t fail(cc_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

cc_status_t ok() {
  g_err.clear();
  return CC_OK;
}

// a launch the LDS guard refused on this thread, not yet reported
thread_local std::string g_refusal;

cc_status_t hip_status(hipError_t e, const char* what) {
  if (!g_refusal.empty()) {
    std::string why;
    why.swap(g_refusal);
    return fail(CC_ERR_UNSUPPORTED, "%s: %s", what, why.c_str());
  }
  if (e == hipSuccess) return ok();
  return fail(CC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

cc_status_t device_ready() {
  static std::once_flag once;
  static int count = -1;
  std::call_once(once, [] {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
    count = n;
  });
  if (count <= 0) return fail(CC_ERR_NO_DEVICE, "no HIP device is visible");
  return CC_OK;
}

bool is_pow2(int n) { return n >= 1 && (n & (n - 1)) == 0; }
int ilog2(int n) {
  int l = 0;
  while ((1 << l) < n) ++l;
  return l;
}
bool al16(uint64_t v) { return (v & 15u) == 0; }
bool al16p(const void* p) { return al16((uint64_t)(uintptr_t)p); }
uint64_t rup(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

extern const cc_config_t kDefaultCfg = {CC_ALGO_RING, 0, nullptr, 0, 0, 0};

cc_status_t common_checks(cc_coll_t coll, int nranks, cc_dtype_t dtype, const cc_config_t* cfg) {
  if (nranks < 1 || nranks > CC_MAX_RANKS)
    return fail(CC_ERR_INVALID_ARG, "nranks=%d outside [1, %d]", nranks, CC_MAX_RANKS);
  if ((int)dtype < 0 || (int)dtype > 2) return fail(CC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if ((int)cfg->algo < 0 || (int)cfg->algo > 5) return fail(CC_ERR_INVALID_ARG, "unknown algo %d", (int)cfg->algo);
  if ((int)cfg->algo >= CC_ALGO_TREE && coll != CC_COLL_ALL_REDUCE)
    return fail(CC_ERR_UNSUPPORTED, "tree, double tree and 2-port ring are AllReduce schedules");
  if (cfg->fuse_depth < 0) return fail(CC_ERR_INVALID_ARG, "fuse_depth=%d is negative", cfg->fuse_depth);
  if (cfg->blocks_per_cu < 0) return fail(CC_ERR_INVALID_ARG, "blocks_per_cu=%d is negative", cfg->blocks_per_cu);
  if (cfg->grid_sync != 0 && cfg->grid_sync != 1)
    return fail(CC_ERR_INVALID_ARG, "grid_sync=%d is neither 0 nor 1", cfg->grid_sync);
  if (cfg->grid_sync &&
      (coll != CC_COLL_ALL_REDUCE || cfg->algo != CC_ALGO_RING || cfg->fuse_depth < 1))
    return fail(CC_ERR_UNSUPPORTED, "grid_sync runs the stepwise ring AllReduce only (algo ring, fuse_depth >= 1)");
  return CC_OK;
}

// nbytes per rank buffer; N buffers at base + r*stride must not overlap each
// other and the base must be set when there is data.
cc_status_t check_side(const cc_rankbuf_t& s, uint64_t nbytes, int N, const char* name) {
  if (nbytes == 0) return CC_OK;
  if (s.base == nullptr) return fail(CC_ERR_INVALID_ARG, "%s.base is NULL", name);
  if (N > 1 && s.rank_stride_bytes < nbytes)
    return fail(CC_ERR_INVALID_ARG, "%s.rank_stride_bytes=%zu is smaller than a rank's %llu bytes", name,
                s.rank_stride_bytes, (unsigned long long)nbytes);
  return CC_OK;
}

// Any byte shared between a rank buffer of `a` and one of `b`?
bool sides_overlap(const cc_rankbuf_t& a, uint64_t abytes, int an, const cc_rankbuf_t& b, uint64_t bbytes,
                   int bn) {
  if (abytes == 0 || bbytes == 0) return false;
  const uint64_t ab = (uint64_t)(uintptr_t)a.base, bb = (uint64_t)(uintptr_t)b.base;
  for (int i = 0; i < an; ++i) {
    const uint64_t a0 = ab + (uint64_t)i * a.rank_stride_bytes, a1 = a0 + abytes;
    for (int j = 0; j < bn; ++j) {
      const uint64_t b0 = bb + (uint64_t)j * b.rank_stride_bytes, b1 = b0 + bbytes;
      if (a0 < b1 && b0 < a1) return true;
    }
  }
  return false;
}

bool same_side(const cc_rankbuf_t& a, const cc_rankbuf_t& b) {
  return a.base == b.base && a.rank_stride_bytes == b.rank_stride_bytes;
}

}  // namespace api

void refuse_launch(const char* why) { api::g_refusal = why; }

}  // namespace cc

using namespace cc::api;

namespace {

// A launch covers num_tiles workgroups of kBlock threads: the grid's x size
// must fit 31 bits and its work-items 32 bits (HIP rejects a larger launch).
cc_status_t grid_fits(uint64_t M, int dt) {
  const uint64_t tiles = num_tiles(M, dt);
  if (tiles > 0x7fffffffull || tiles * (uint64_t)kBlock > 0xffffffffull)
    return fail(CC_ERR_INVALID_ARG, "count too large for one launch");
  return CC_OK;
}

Side side(const cc_rankbuf_t& s) { return Side{(char*)s.base, (uint64_t)s.rank_stride_bytes}; }

// floor(c*M/N), c = 0..N: the chunk boundaries every schedule uses
struct Bounds {
  uint64_t b[kMaxRanks + 1];
  Bounds(uint64_t M, int N) {
    for (int c = 0; c <= N; ++c) b[c] = (uint64_t)(((unsigned __int128)c * M) / (unsigned)N);
  }
};

// ---- AllReduce schedules that run as descriptor steps
// the descriptor-step schedule of an AllReduce, or -1 (kernels of its own)
int sched_of(int algo, int N) {
  switch (algo) {
    case CC_ALGO_TREE: return SCHED_TREE;
    case CC_ALGO_DOUBLE_TREE: return SCHED_DBT;
    case CC_ALGO_RING_2PORT: return SCHED_RING2;
    case CC_ALGO_HALVING_DOUBLING: return is_pow2(N) ? -1 : SCHED_HD_PAIRS;
    case CC_ALGO_BUTTERFLY: return is_pow2(N) ? -1 : SCHED_BFLY_PAIRS;
  }
  return -1;
}

constexpr int kDbtFusedMaxRanks = 16;

// whether an AllReduce runs descriptor steps: the stepwise form of those
// schedules, and the double tree beyond its fused kernel's rank limit
bool runs_steps(const cc_config_t& cfg, int N) {
  if (N < 2 || sched_of(cfg.algo, N) < 0) return false;
  return cfg.fuse_depth >= 1 || (cfg.algo == CC_ALGO_DOUBLE_TREE && N > kDbtFusedMaxRanks);
}

// ---- workspace sizing (bytes); M is the full per-rank vector length
uint64_t ws_need_data(cc_coll_t coll, const cc_config_t& cfg, int N, uint64_t M, int dt);

// grid_sync: the queue words take the first kBarBytes, staging follows
constexpr uint64_t kBarBytes = 512;
static_assert(kQueueWords * 4 <= kBarBytes, "queue words fit");
bool uses_barrier(const cc_config_t& cfg, int N) { return cfg.grid_sync && N > 1; }

uint64_t ws_need(cc_coll_t coll, const cc_config_t& cfg, int N, uint64_t M, int dt) {
  return (uses_barrier(cfg, N) ? kBarBytes : 0) + ws_need_data(coll, cfg, N, M, dt);
}

uint64_t ws_need_data(cc_coll_t coll, const cc_config_t& cfg, int N, uint64_t M, int dt) {
  if (N <= 1) return 0;
  const uint64_t per_elem = M * 4;
  const uint64_t per_rank = N * rup(per_elem, 256);
  // descriptor steps keep fp32 partials per rank for bf16
  if (coll == CC_COLL_ALL_REDUCE && runs_steps(cfg, N)) return dt == DT_BF16 ? per_rank : 0;
  if (cfg.fuse_depth == 0) return 0;
  const int k = std::min(cfg.fuse_depth, N - 1);
  if (coll == CC_COLL_ALL_REDUCE) {
    if (dt != DT_BF16) return 0;
    if (cfg.algo == CC_ALGO_RING) return k < N - 1 ? per_elem : 0;
    return N >= 4 ? per_rank : 0;  // halving-doubling and butterfly, fp32 partials per rank
  }
  if (coll == CC_COLL_REDUCE_SCATTER) {
    if (cfg.algo == CC_ALGO_RING) return k < N - 1 ? per_elem : 0;
    if (cfg.algo == CC_ALGO_HALVING_DOUBLING) return N >= 4 ? per_rank : 0;
  }
  return 0;
}

// The `need` bytes of workspace the call will use must be given and must
// share no byte with the send (N x sbytes) or recv (N x rbytes) buffers: the
// stepwise schedules write partial results there, grid_sync its queue words.
cc_status_t check_ws_bytes(const cc_config_t& cfg, uint64_t need, const char* sizer, const cc_rankbuf_t& send,
                           uint64_t sbytes, const cc_rankbuf_t& recv, uint64_t rbytes, int N) {
  if (need == 0) return CC_OK;
  if (cfg.workspace == nullptr || cfg.workspace_bytes < need)
    return fail(CC_ERR_INVALID_ARG, "this schedule needs %llu bytes of workspace (%s); got %zu",
                (unsigned long long)need, sizer, cfg.workspace ? cfg.workspace_bytes : (size_t)0);
  const cc_rankbuf_t ws{cfg.workspace, (size_t)need};
  if (sides_overlap(ws, need, 1, send, sbytes, N) || sides_overlap(ws, need, 1, recv, rbytes, N))
    return fail(CC_ERR_INVALID_ARG, "the workspace overlaps the send or recv buffers");
  return CC_OK;
}

cc_status_t check_ws(cc_coll_t coll, const cc_config_t& cfg, int N, uint64_t M, int dt, const cc_rankbuf_t& send,
                     uint64_t sbytes, const cc_rankbuf_t& recv, uint64_t rbytes) {
  const uint64_t need = ws_need(coll, cfg, N, M, dt);
  cc_status_t s = check_ws_bytes(cfg, need, "cc_workspace_size", send, sbytes, recv, rbytes, N);
  if (s || need == 0) return s;
  if (uses_barrier(cfg, N) && ((uintptr_t)cfg.workspace & 15u))
    return fail(CC_ERR_INVALID_ARG, "grid_sync needs a 16-byte aligned workspace");
  return CC_OK;
}

Side ws_side(const cc_config_t& cfg, uint64_t M, int N) {
  char* base = (char*)cfg.workspace;
  if (base && uses_barrier(cfg, N)) base += kBarBytes;
  return Side{base, rup(M * 4, 256)};
}

cc_status_t copy_ranks(const cc_rankbuf_t& src, const cc_rankbuf_t& dst, uint64_t nbytes, int N, int esize,
                       int blocks_per_cu, hipStream_t st) {
  std::vector<CopyDesc> d;
  for (int r = 0; r < N; ++r)
    d.push_back(CopyDesc{(const char*)src.base + (uint64_t)r * src.rank_stride_bytes,
                         (char*)dst.base + (uint64_t)r * dst.rank_stride_bytes, nbytes});
  for (size_t i = 0; i < d.size(); i += kMaxDesc) {
    const int n = (int)std::min<size_t>(kMaxDesc, d.size() - i);
    hipError_t e = launch_copies(d.data() + i, n, esize, blocks_per_cu, st);
    if (e != hipSuccess) return hip_status(e, "copy launch");
  }
  return ok();
}

cc_status_t run_all_reduce(cc_rankbuf_t send, cc_rankbuf_t recv, uint64_t M, int dt, int op, int N,
                           const cc_config_t& cfg, hipStream_t st);

// the launch arguments of a validated AllReduce over M elements, chunked (or
// segmented) at bnd[0..N]
Red red_of(cc_rankbuf_t send, cc_rankbuf_t recv, uint64_t M, const uint64_t* bnd, int dt, int op, int N,
           const cc_config_t& cfg, hipStream_t st) {
  Red r;
  r.send = side(send);
  r.recv = side(recv);
  r.ws = ws_side(cfg, M, N);
  r.M = M;
  r.bnd = bnd;
  r.blocks_per_cu = cfg.blocks_per_cu;
  r.N = N;
  r.dt = dt;
  r.op = op;
  r.rs_mode = 0;
  r.vec_ok = al16p(send.base) && al16(send.rank_stride_bytes) && al16p(recv.base) && al16(recv.rank_stride_bytes) &&
             (cfg.workspace == nullptr || al16p(cfg.workspace));
  r.st = st;
  return r;
}

// ---- hierarchical AllReduce
struct Hier {
  std::vector<int> dims;       // as given, level 0 first
  std::vector<int> p, stride;  // the levels of size > 1: sizes and rank strides
  std::vector<int> at;         // their index in dims
  int N = 1;
  int top = 0;                 // index in p of the AllReduce level; p.size() when none runs
};

constexpr int kMaxHierDims = 8;

cc_status_t hier_args(int ndims, const int* dims, Hier* h) {
  if (ndims < 1 || ndims > kMaxHierDims)
    return fail(CC_ERR_INVALID_ARG, "ndims=%d outside [1, %d]", ndims, kMaxHierDims);
  if (!dims) return fail(CC_ERR_INVALID_ARG, "dims is NULL");
  h->dims.assign(dims, dims + ndims);
  int64_t n = 1;
  for (int i = 0; i < ndims; ++i) {
    if (dims[i] < 1) return fail(CC_ERR_INVALID_ARG, "dims[%d]=%d is below 1", i, dims[i]);
    n *= dims[i];
    if (n > CC_MAX_RANKS) return fail(CC_ERR_INVALID_ARG, "the product of dims exceeds %d ranks", CC_MAX_RANKS);
  }
  h->N = (int)n;
  hier_levels(h->dims, &h->p, &h->stride);
  h->at.clear();
  for (int i = 0; i < ndims; ++i)
    if (dims[i] > 1) h->at.push_back(i);
  if ((int)h->p.size() > kMaxHierLevels)
    return fail(CC_ERR_UNSUPPORTED, "%d levels of size > 1; at most %d are supported", (int)h->p.size(),
                kMaxHierLevels);
  h->top = dims[ndims - 1] > 1 ? (int)h->p.size() - 1 : (int)h->p.size();
  return CC_OK;
}

// a lone outermost level: the flat ring AllReduce
bool hier_flat(const Hier& h) { return h.p.size() == 1 && h.top == 0; }

cc_status_t hier_cfg_checks(const cc_config_t& cfg, int N, cc_dtype_t dtype) {
  cc_status_t s = common_checks(CC_COLL_ALL_REDUCE, N, dtype, &cfg);
  if (s) return s;
  if (cfg.algo != CC_ALGO_RING)
    return fail(CC_ERR_UNSUPPORTED, "the hierarchical AllReduce runs ring schedules at every level (algo ring)");
  if (cfg.grid_sync) return fail(CC_ERR_UNSUPPORTED, "grid_sync is not available for the hierarchical AllReduce");
  return CC_OK;
}

uint64_t hier_ws(const Hier& h, const cc_config_t& cfg, uint64_t M, int dt) {
  if (h.N < 2) return 0;
  if (hier_flat(h)) return ws_need(CC_COLL_ALL_REDUCE, cfg, h.N, M, dt);
  if (cfg.fuse_depth == 0 || dt != DT_BF16) return 0;
  return (uint64_t)h.N * rup(M * 4, 256);  // fp32 partials per rank
}

// The N segments of the vector: the level-0 chunks (floor bounds), each split
// into its level-1 chunks, and so on; bnd[0..N] their bounds, seg[s] their
// chunk index at every level of size > 1 (8 bits each).
void hier_segments(const Hier& h, uint64_t M, uint64_t* bnd, uint32_t* seg) {
  struct S {
    uint64_t lo, hi;
    uint32_t code;
  };
  std::vector<S> cur{S{0, M, 0u}};
  for (size_t i = 0; i < h.p.size(); ++i) {
    std::vector<S> nx;
    const unsigned q = (unsigned)h.p[i];
    for (const S& x : cur)
      for (unsigned c = 0; c < q; ++c) {
        const uint64_t span = x.hi - x.lo;
        const uint64_t a = x.lo + (uint64_t)(((unsigned __int128)c * span) / q);
        const uint64_t b = x.lo + (uint64_t)(((unsigned __int128)(c + 1) * span) / q);
        nx.push_back(S{a, b, x.code | (c << (8 * i))});
      }
    cur.swap(nx);
  }
  for (size_t s = 0; s < cur.size(); ++s) {
    bnd[s] = cur[s].lo;
    seg[s] = cur[s].code;
  }
  bnd[cur.size()] = M;
}

}  // namespace

extern "C" {

const char* cc_version(void) { return "cc 0.1.0 (gfx950)"; }

const char* cc_status_string(cc_status_t s) {
  switch (s) {
    case CC_OK: return "CC_OK";
    case CC_ERR_INVALID_ARG: return "CC_ERR_INVALID_ARG";
    case CC_ERR_UNSUPPORTED: return "CC_ERR_UNSUPPORTED";
    case CC_ERR_NO_DEVICE: return "CC_ERR_NO_DEVICE";
    case CC_ERR_HIP: return "CC_ERR_HIP";
    default: break;
  }
  return "CC_ERR_UNKNOWN";
}

const char* cc_last_error(void) { return g_err.c_str(); }

cc_status_t cc_chunk_bounds(size_t count, int nranks, size_t* bounds) {
  if (nranks < 1 || nranks > CC_MAX_RANKS) return fail(CC_ERR_INVALID_ARG, "nranks=%d", nranks);
  if (!bounds) return fail(CC_ERR_INVALID_ARG, "bounds is NULL");
  for (int c = 0; c <= nranks; ++c)
    bounds[c] = (size_t)(((unsigned __int128)c * count) / (unsigned)nranks);
  return ok();
}

cc_status_t cc_all_reduce(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype, cc_op_t op,
                          int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_ALL_REDUCE, nranks, dtype, &cfg);
  if (s) return s;
  if ((int)op < 0 || (int)op > 2) return fail(CC_ERR_INVALID_ARG, "unknown op %d", (int)op);
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (count == 0) return ok();
  const uint64_t M = count, nb = M * es;
  if ((s = check_side(send, nb, N, "send")) || (s = check_side(recv, nb, N, "recv"))) return s;
  const bool in_place = same_side(send, recv);
  if (!in_place && sides_overlap(send, nb, N, recv, nb, N))
    return fail(CC_ERR_INVALID_ARG, "send and recv overlap without being the same buffers");
  if ((s = grid_fits(M, dt))) return s;
  if ((s = check_ws(CC_COLL_ALL_REDUCE, cfg, N, M, dt, send, nb, recv, nb))) return s;
  if ((s = device_ready())) return s;
  return run_all_reduce(send, recv, M, dt, (int)op, N, cfg, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// An AllReduce whose arguments are validated.
cc_status_t run_all_reduce(cc_rankbuf_t send, cc_rankbuf_t recv, uint64_t M, int dt, int op, int N,
                           const cc_config_t& cfg, hipStream_t st) {
  const int es = elem_size(dt);
  const uint64_t nb = M * es;
  const bool in_place = same_side(send, recv);
  if (N == 1) return in_place ? ok() : copy_ranks(send, recv, nb, 1, es, cfg.blocks_per_cu, st);

  const Bounds bd(M, N);
  Red r = red_of(send, recv, M, bd.b, dt, op, N, cfg, st);

  hipError_t e = hipSuccess;
  if (cfg.algo == CC_ALGO_RING) {
    if (cfg.fuse_depth == 0) return hip_status(launch_ring_fused(r), "ring all_reduce");
    const int k = std::min(cfg.fuse_depth, N - 1);
    if (cfg.grid_sync) return hip_status(launch_ring_queue(r, k, (unsigned*)cfg.workspace), "ring all_reduce (one launch)");
    const int pin = dt != DT_BF16;
    for (int s0 = 0; s0 < N - 1 && e == hipSuccess; s0 += k) e = launch_ring_rs_pass(r, s0, std::min(k, N - 1 - s0), pin);
    Gat g{r.send, r.recv, M, bd.b, cfg.blocks_per_cu, N, es, 0, r.vec_ok, st};
    for (int s0 = 0; s0 < N - 1 && e == hipSuccess; s0 += k) e = launch_ring_ag_pass(g, s0, std::min(k, N - 1 - s0));
    return hip_status(e, "ring all_reduce (stepwise)");
  }
  const int sch = sched_of(cfg.algo, N);
  if (sch >= 0) {
    if (runs_steps(cfg, N)) {
      const Plan p = build_plan((SchedAlg)sch, N, M);
      for (const auto& stp : p.steps)
        for (size_t i = 0; i < stp.size() && e == hipSuccess; i += kMaxGDesc)
          e = launch_gsteps(r, stp.data() + i, (int)std::min<size_t>(kMaxGDesc, stp.size() - i));
      return hip_status(e, "all_reduce (descriptor steps)");
    }
    int m = 1;
    while (2 * m <= N) m *= 2;
    switch (cfg.algo) {
      case CC_ALGO_TREE:
        return hip_status(launch_tree_shaped(r, TREE_BFLY, m == N ? m : 2 * m, N, 0), "tree all_reduce");
      case CC_ALGO_DOUBLE_TREE: return hip_status(launch_dbt_fused(r), "double tree all_reduce");
      case CC_ALGO_RING_2PORT: return hip_status(launch_ring2_fused(r), "2-port ring all_reduce");
      default:
        return hip_status(launch_tree_shaped(r, cfg.algo == CC_ALGO_HALVING_DOUBLING ? TREE_HD : TREE_BFLY, m, m, N - m),
                          "pair-folded all_reduce");
    }
  }
  const int tree = cfg.algo == CC_ALGO_HALVING_DOUBLING ? TREE_HD : TREE_BFLY;
  if (cfg.fuse_depth == 0) return hip_status(launch_tree_fused(r, tree), "tree all_reduce");
  const int acc_recv = dt != DT_BF16;
  if (tree == TREE_HD) {
    for (int d = N / 2; d >= 1 && e == hipSuccess; d /= 2) e = launch_hd_rs_step(r, d, d == N / 2, d == 1, acc_recv);
    Gat g{r.send, r.recv, M, bd.b, cfg.blocks_per_cu, N, es, 0, r.vec_ok, st};
    for (int d = 1; d < N && e == hipSuccess; d *= 2) e = launch_hd_ag_step(g, d, 0);
    return hip_status(e, "halving-doubling all_reduce (stepwise)");
  }
  for (int d = 1; d < N && e == hipSuccess; d *= 2) e = launch_bfly_step(r, d, d == 1, 2 * d == N, acc_recv);
  return hip_status(e, "butterfly all_reduce (stepwise)");
}

}  // namespace

extern "C" {

cc_status_t cc_all_reduce_buckets(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* offsets, const size_t* counts,
                                  int nbuckets, cc_dtype_t dtype, cc_op_t op, int nranks, const cc_config_t* cfgp,
                                  cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_ALL_REDUCE, nranks, dtype, &cfg);
  if (s) return s;
  if ((int)op < 0 || (int)op > 2) return fail(CC_ERR_INVALID_ARG, "unknown op %d", (int)op);
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (nbuckets < 0) return fail(CC_ERR_INVALID_ARG, "nbuckets=%d is negative", nbuckets);
  if (nbuckets == 0) return ok();
  if (!offsets || !counts) return fail(CC_ERR_INVALID_ARG, "offsets or counts is NULL");
  // buckets: non-empty ranges, pairwise disjoint, within every rank buffer
  std::vector<std::pair<uint64_t, uint64_t>> rg;
  uint64_t extent = 0, maxlen = 0;
  for (int b = 0; b < nbuckets; ++b) {
    if (counts[b] == 0) continue;
    const unsigned __int128 end = (unsigned __int128)offsets[b] + counts[b];
    if (end >> 60) return fail(CC_ERR_INVALID_ARG, "bucket %d out of range", b);
    rg.push_back({offsets[b], (uint64_t)end});
    extent = std::max(extent, (uint64_t)end);
    maxlen = std::max(maxlen, (uint64_t)counts[b]);
  }
  if (rg.empty()) return ok();
  std::vector<std::pair<uint64_t, uint64_t>> sorted = rg;
  std::sort(sorted.begin(), sorted.end());
  for (size_t i = 1; i < sorted.size(); ++i)
    if (sorted[i].first < sorted[i - 1].second) return fail(CC_ERR_INVALID_ARG, "buckets overlap");
  const uint64_t nb = extent * es;
  if ((s = check_side(send, nb, N, "send")) || (s = check_side(recv, nb, N, "recv"))) return s;
  const bool in_place = same_side(send, recv);
  if (!in_place && sides_overlap(send, nb, N, recv, nb, N))
    return fail(CC_ERR_INVALID_ARG, "send and recv overlap without being the same buffers");
  if ((s = grid_fits(maxlen, dt))) return s;
  if ((s = check_ws(CC_COLL_ALL_REDUCE, cfg, N, maxlen, dt, send, nb, recv, nb))) return s;
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  auto sub = [&](const cc_rankbuf_t& x, uint64_t off) {
    return cc_rankbuf_t{(char*)x.base + off * es, x.rank_stride_bytes};
  };
  const bool seg_alg = cfg.algo == CC_ALGO_RING ||
                       ((cfg.algo == CC_ALGO_HALVING_DOUBLING || cfg.algo == CC_ALGO_BUTTERFLY) && is_pow2(N));
  const bool one_launch = seg_alg && cfg.fuse_depth == 0 && N > 1 && N <= kMaxSegRanks && maxlen < (1ull << 31) &&
                          num_tiles(maxlen, dt) * kMaxSeg < 0x7fffffffull;
  if (!one_launch) {
    for (const auto& r : rg)
      if ((s = run_all_reduce(sub(send, r.first), sub(recv, r.first), r.second - r.first, dt, (int)op, N, cfg, st)))
        return s;
    return ok();
  }
  SegLaunch L;
  L.send = side(send);
  L.recv = side(recv);
  L.N = N;
  L.dt = dt;
  L.op = (int)op;
  L.alg = (int)cfg.algo;
  L.blocks_per_cu = cfg.blocks_per_cu;
  L.st = st;
  for (size_t i = 0; i < rg.size(); i += kMaxSeg) {
    L.nseg = (int)std::min<size_t>(kMaxSeg, rg.size() - i);
    for (int k = 0; k < L.nseg; ++k) {
      L.off[k] = rg[i + k].first;
      L.len[k] = rg[i + k].second - rg[i + k].first;
    }
    hipError_t e = launch_fused_seg(L);
    if (e != hipSuccess) return hip_status(e, "bucketed all_reduce");
  }
  return ok();
}

cc_status_t cc_bucket_plan(const size_t* sizes, int ntensors, size_t elem_bytes, size_t cap_bytes,
                           size_t align_elems, int* bucket_of, size_t* tensor_offset, size_t* bucket_offset,
                           size_t* bucket_count, int* nbuckets) {
  if (ntensors < 0) return fail(CC_ERR_INVALID_ARG, "ntensors=%d is negative", ntensors);
  if (!nbuckets) return fail(CC_ERR_INVALID_ARG, "nbuckets is NULL");
  if (ntensors > 0 && (!sizes || !bucket_of || !tensor_offset || !bucket_offset || !bucket_count))
    return fail(CC_ERR_INVALID_ARG, "NULL array");
  if (elem_bytes == 0 || align_elems == 0) return fail(CC_ERR_INVALID_ARG, "elem_bytes and align_elems must be > 0");
  // reverse order (the order gradients become ready in backward), greedy:
  // close the bucket when the next tensor would push it past the cap; a
  // tensor larger than the cap gets a bucket of its own
  int nb = 0;
  uint64_t cur_bytes = 0, pos = 0;
  for (int t = ntensors - 1; t >= 0; --t) {
    const unsigned __int128 tb = (unsigned __int128)sizes[t] * elem_bytes;
    if (tb >> 60) return fail(CC_ERR_INVALID_ARG, "tensor %d too large", t);
    if (nb == 0 || (cur_bytes > 0 && cur_bytes + (uint64_t)tb > cap_bytes)) {
      // open a new bucket at the next aligned offset
      const uint64_t start = nb == 0 ? 0 : rup(bucket_offset[nb - 1] + bucket_count[nb - 1], align_elems);
      bucket_offset[nb] = start;
      bucket_count[nb] = 0;
      pos = start;
      cur_bytes = 0;
      ++nb;
    }
    bucket_of[t] = nb - 1;
    tensor_offset[t] = pos;
    pos += sizes[t];
    bucket_count[nb - 1] += sizes[t];
    cur_bytes += (uint64_t)tb;
  }
  *nbuckets = nb;
  return ok();
}

cc_status_t cc_reduce_scatter(cc_rankbuf_t send, cc_rankbuf_t recv, size_t recvcount, cc_dtype_t dtype, cc_op_t op,
                              int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_REDUCE_SCATTER, nranks, dtype, &cfg);
  if (s) return s;
  if ((int)op < 0 || (int)op > 2) return fail(CC_ERR_INVALID_ARG, "unknown op %d", (int)op);
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (cfg.algo == CC_ALGO_BUTTERFLY) return fail(CC_ERR_UNSUPPORTED, "butterfly is defined for all_reduce only");
  if (cfg.algo == CC_ALGO_HALVING_DOUBLING && !is_pow2(N))
    return fail(CC_ERR_UNSUPPORTED, "halving-doubling needs nranks = 2^k (got %d)", N);
  if (recvcount == 0) return ok();
  const uint64_t S = recvcount, M = (uint64_t)N * S;
  if ((s = check_side(send, M * es, N, "send")) || (s = check_side(recv, S * es, N, "recv"))) return s;
  if (sides_overlap(send, M * es, N, recv, S * es, N)) return fail(CC_ERR_INVALID_ARG, "send and recv overlap");
  if ((s = grid_fits(M, dt))) return s;
  if ((s = check_ws(CC_COLL_REDUCE_SCATTER, cfg, N, M, dt, send, M * es, recv, S * es))) return s;
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  if (N == 1) return copy_ranks(send, recv, S * es, 1, es, cfg.blocks_per_cu, st);

  const Bounds bd(M, N);
  Red r;
  r.send = side(send);
  r.recv = side(recv);
  r.ws = ws_side(cfg, M, N);
  r.M = M;
  r.bnd = bd.b;
  r.blocks_per_cu = cfg.blocks_per_cu;
  r.N = N;
  r.dt = dt;
  r.op = (int)op;
  r.rs_mode = 1;
  r.vec_ok = al16p(send.base) && al16(send.rank_stride_bytes) && al16p(recv.base) && al16(recv.rank_stride_bytes) &&
             al16(S * es) && (cfg.workspace == nullptr || al16p(cfg.workspace));
  r.st = st;
  hipError_t e = hipSuccess;
  if (cfg.algo == CC_ALGO_RING) {
    if (cfg.fuse_depth == 0) return hip_status(launch_ring_fused(r), "ring reduce_scatter");
    const int k = std::min(cfg.fuse_depth, N - 1);
    for (int s0 = 0; s0 < N - 1 && e == hipSuccess; s0 += k) e = launch_ring_rs_pass(r, s0, std::min(k, N - 1 - s0), 0);
    return hip_status(e, "ring reduce_scatter (stepwise)");
  }
  if (cfg.fuse_depth == 0) return hip_status(launch_tree_fused(r, TREE_HD), "halving-doubling reduce_scatter");
  for (int d = N / 2; d >= 1 && e == hipSuccess; d /= 2) e = launch_hd_rs_step(r, d, d == N / 2, d == 1, 0);
  return hip_status(e, "halving-doubling reduce_scatter (stepwise)");
}

cc_status_t cc_all_gather(cc_rankbuf_t send, cc_rankbuf_t recv, size_t sendcount, cc_dtype_t dtype, int nranks,
                          const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_ALL_GATHER, nranks, dtype, &cfg);
  if (s) return s;
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (cfg.algo == CC_ALGO_BUTTERFLY) return fail(CC_ERR_UNSUPPORTED, "butterfly is defined for all_reduce only");
  if (cfg.algo == CC_ALGO_HALVING_DOUBLING && !is_pow2(N))
    return fail(CC_ERR_UNSUPPORTED, "halving-doubling needs nranks = 2^k (got %d)", N);
  if (sendcount == 0) return ok();
  const uint64_t S = sendcount, M = (uint64_t)N * S;
  if ((s = check_side(send, S * es, N, "send")) || (s = check_side(recv, M * es, N, "recv"))) return s;
  if (sides_overlap(send, S * es, N, recv, M * es, N)) return fail(CC_ERR_INVALID_ARG, "send and recv overlap");
  if ((s = grid_fits(M, dt))) return s;
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  if (N == 1) return copy_ranks(send, recv, S * es, 1, es, cfg.blocks_per_cu, st);
  const Bounds bd(M, N);
  Gat g;
  g.send = side(send);
  g.recv = side(recv);
  g.M = M;
  g.bnd = bd.b;
  g.blocks_per_cu = cfg.blocks_per_cu;
  g.N = N;
  g.esize = es;
  g.ag_mode = 1;
  g.vec_ok = al16p(send.base) && al16(send.rank_stride_bytes) && al16p(recv.base) && al16(recv.rank_stride_bytes) &&
             al16(S * es);
  g.st = st;
  if (cfg.fuse_depth == 0) return hip_status(launch_ag_fused(g), "all_gather");
  hipError_t e = hipSuccess;
  if (cfg.algo == CC_ALGO_RING) {
    const int k = std::min(cfg.fuse_depth, N - 1);
    for (int s0 = 0; s0 < N - 1 && e == hipSuccess; s0 += k) e = launch_ring_ag_pass(g, s0, std::min(k, N - 1 - s0));
    return hip_status(e, "ring all_gather (stepwise)");
  }
  for (int d = 1; d < N && e == hipSuccess; d *= 2) e = launch_hd_ag_step(g, d, d == 1);
  return hip_status(e, "halving-doubling all_gather (stepwise)");
}

cc_status_t cc_broadcast(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype, int root, int nranks,
                         const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_BROADCAST, nranks, dtype, &cfg);
  if (s) return s;
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (root < 0 || root >= N) return fail(CC_ERR_INVALID_ARG, "root=%d outside [0, %d)", root, N);
  if (cfg.algo == CC_ALGO_BUTTERFLY) return fail(CC_ERR_UNSUPPORTED, "butterfly is defined for all_reduce only");
  if (count == 0) return ok();
  const uint64_t nb = (uint64_t)count * es;
  if ((s = check_side(recv, nb, N, "recv"))) return s;
  if (send.base == nullptr) return fail(CC_ERR_INVALID_ARG, "send.base is NULL");
  const bool in_place = same_side(send, recv);
  const cc_rankbuf_t src_rank = {(char*)send.base + (uint64_t)root * send.rank_stride_bytes, 0};
  if (!in_place && sides_overlap(src_rank, nb, 1, recv, nb, N))
    return fail(CC_ERR_INVALID_ARG, "the root's send buffer overlaps a recv buffer");
  if (nb / 2048 > 0x7fffffffull) return fail(CC_ERR_INVALID_ARG, "count too large");
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  const char* src = (const char*)src_rank.base;
  Side dst = side(recv);
  const int vec_ok = al16p(src) && al16p(recv.base) && al16(recv.rank_stride_bytes);
  if (cfg.fuse_depth == 0 || N == 1)
    return hip_status(launch_bcast(src, dst, N, in_place ? root : -1, nb, vec_ok, cfg.blocks_per_cu, st), "broadcast");
  // stepwise: the root's own output first, then the chain or binomial steps
  hipError_t e = hipSuccess;
  auto rank_ptr = [&](int r) { return dst.base + (uint64_t)((r % N + N) % N) * dst.stride; };
  if (!in_place) {
    CopyDesc d{src, rank_ptr(root), nb};
    e = launch_copies(&d, 1, es, cfg.blocks_per_cu, st);
  }
  if (cfg.algo == CC_ALGO_RING) {
    for (int s0 = 0; s0 < N - 1 && e == hipSuccess; ++s0) {
      CopyDesc d{rank_ptr(root + s0), rank_ptr(root + s0 + 1), nb};
      e = launch_copies(&d, 1, es, cfg.blocks_per_cu, st);
    }
    return hip_status(e, "ring broadcast (stepwise)");
  }
  for (int k = 1; k < N && e == hipSuccess; k *= 2) {
    std::vector<CopyDesc> d;
    for (int rel = 0; rel < k && rel + k < N; ++rel) d.push_back(CopyDesc{rank_ptr(root + rel), rank_ptr(root + rel + k), nb});
    for (size_t i = 0; i < d.size() && e == hipSuccess; i += kMaxDesc)
      e = launch_copies(d.data() + i, (int)std::min<size_t>(kMaxDesc, d.size() - i), es, cfg.blocks_per_cu, st);
  }
  return hip_status(e, "binomial broadcast (stepwise)");
}

cc_status_t cc_all_to_all(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, size_t elem_per_row,
                          cc_dtype_t dtype, int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(CC_COLL_ALL_TO_ALL, nranks, dtype, &cfg);
  if (s) return s;
  const int N = nranks, dt = (int)dtype, es = elem_size(dt);
  if (cfg.algo != CC_ALGO_RING) return fail(CC_ERR_UNSUPPORTED, "all_to_all supports the ring/pairwise schedule only");
  if (counts == nullptr) return fail(CC_ERR_INVALID_ARG, "counts is NULL");
  if (elem_per_row == 0) return fail(CC_ERR_INVALID_ARG, "elem_per_row is 0");
  const unsigned __int128 row_bytes = (unsigned __int128)elem_per_row * es;
  std::vector<uint64_t> sdisp((size_t)N * N), rdisp((size_t)N * N), stot(N, 0), rtot(N, 0);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) {
      const unsigned __int128 b = (unsigned __int128)counts[i * N + j] * row_bytes;
      if (b >> 62) return fail(CC_ERR_INVALID_ARG, "counts[%d][%d] too large", i, j);
      sdisp[i * N + j] = stot[i];
      stot[i] += (uint64_t)b;
      if ((stot[i] >> 62)) return fail(CC_ERR_INVALID_ARG, "send size too large");
    }
  for (int j = 0; j < N; ++j)
    for (int i = 0; i < N; ++i) {
      rdisp[i * N + j] = rtot[j];
      rtot[j] += (uint64_t)((unsigned __int128)counts[i * N + j] * row_bytes);
      if ((rtot[j] >> 62)) return fail(CC_ERR_INVALID_ARG, "recv size too large");
    }
  const uint64_t smax = *std::max_element(stot.begin(), stot.end());
  const uint64_t rmax = *std::max_element(rtot.begin(), rtot.end());
  if ((s = check_side(send, smax, N, "send")) || (s = check_side(recv, rmax, N, "recv"))) return s;
  if (sides_overlap(send, smax, N, recv, rmax, N)) return fail(CC_ERR_INVALID_ARG, "send and recv overlap");
  if (smax == 0) return ok();
  if (smax / 2048 > (0x7fffffffull - kMaxDesc) / (uint64_t)N)
    return fail(CC_ERR_INVALID_ARG, "counts too large for one launch");
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  auto desc = [&](int i, int j) {
    return CopyDesc{(const char*)send.base + (uint64_t)i * send.rank_stride_bytes + sdisp[i * N + j],
                    (char*)recv.base + (uint64_t)j * recv.rank_stride_bytes + rdisp[i * N + j],
                    (uint64_t)((unsigned __int128)counts[i * N + j] * row_bytes)};
  };
  hipError_t e = hipSuccess;
  std::vector<CopyDesc> d;
  if (cfg.fuse_depth == 0) {
    for (int j = 0; j < N; ++j)
      for (int i = 0; i < N; ++i) d.push_back(desc(i, j));
    for (size_t i = 0; i < d.size() && e == hipSuccess; i += kMaxDesc)
      e = launch_copies(d.data() + i, (int)std::min<size_t>(kMaxDesc, d.size() - i), es, cfg.blocks_per_cu, st);
    return hip_status(e, "all_to_all");
  }
  for (int k = 0; k < N && e == hipSuccess; ++k) {  // pairwise: step k sends i -> i+k
    d.clear();
    for (int i = 0; i < N; ++i) d.push_back(desc(i, (i + k) % N));
    e = launch_copies(d.data(), N, es, cfg.blocks_per_cu, st);
  }
  return hip_status(e, "pairwise all_to_all");
}

cc_status_t cc_workspace_size(cc_coll_t coll, const cc_config_t* cfgp, int nranks, size_t count, cc_dtype_t dtype,
                              size_t* bytes) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = common_checks(coll, nranks, dtype, &cfg);
  if (s) return s;
  if (!bytes) return fail(CC_ERR_INVALID_ARG, "bytes is NULL");
  if ((int)coll < 0 || (int)coll > 4) return fail(CC_ERR_INVALID_ARG, "unknown collective %d", (int)coll);
  uint64_t M = count;
  if (coll == CC_COLL_REDUCE_SCATTER) M = (uint64_t)count * nranks;
  *bytes = (size_t)ws_need(coll, cfg, nranks, M, (int)dtype);
  return ok();
}

static_assert(CC_PLAN_LOCAL_SEND == GD_LOCAL_SEND && CC_PLAN_IN1 == GD_IN1 && CC_PLAN_IN1_SEND == GD_IN1_SEND &&
                  CC_PLAN_IN2 == GD_IN2 && CC_PLAN_IN2_SEND == GD_IN2_SEND && CC_PLAN_FINAL == GD_FINAL &&
                  CC_PLAN_BOTH == GD_BOTH && CC_PLAN_COPY == GD_COPY,
              "public plan flags are the kernel's");

cc_status_t cc_all_reduce_plan(cc_algo_t algo, int nranks, size_t count, cc_plan_op_t* records, size_t cap,
                               size_t* nrecords) {
  cc_config_t cfg = kDefaultCfg;
  cfg.algo = algo;
  cc_status_t s = common_checks(CC_COLL_ALL_REDUCE, nranks, CC_FLOAT32, &cfg);
  if (s) return s;
  if (!nrecords) return fail(CC_ERR_INVALID_ARG, "nrecords is NULL");
  if (nranks < 2 || sched_of(algo, nranks) < 0)
    return fail(CC_ERR_UNSUPPORTED, "this schedule runs kernels of its own (no descriptor plan)");
  const Plan p = build_plan((SchedAlg)sched_of(algo, nranks), nranks, count);
  size_t n = 0;
  for (const auto& st : p.steps) n += st.size();
  *nrecords = n;
  if (!records) return ok();
  if (cap < n) return fail(CC_ERR_INVALID_ARG, "cap=%zu is smaller than the %zu records", cap, n);
  size_t i = 0;
  for (size_t k = 0; k < p.steps.size(); ++k)
    for (const GDesc& g : p.steps[k])
      records[i++] = cc_plan_op_t{(uint32_t)k, g.flags, g.dst, g.in1, g.in2, g.lo, g.len};
  return ok();
}

cc_status_t cc_all_reduce_hierarchical(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                                       cc_op_t op, int ndims, const int* dims, const cc_config_t* cfgp,
                                       cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  Hier h;
  cc_status_t s = hier_args(ndims, dims, &h);
  if (s || (s = hier_cfg_checks(cfg, h.N, dtype))) return s;
  if ((int)op < 0 || (int)op > 2) return fail(CC_ERR_INVALID_ARG, "unknown op %d", (int)op);
  const int N = h.N, dt = (int)dtype, es = elem_size(dt);
  if (count == 0) return ok();
  const uint64_t M = count, nb = M * es;
  if ((s = check_side(send, nb, N, "send")) || (s = check_side(recv, nb, N, "recv"))) return s;
  if (!same_side(send, recv) && sides_overlap(send, nb, N, recv, nb, N))
    return fail(CC_ERR_INVALID_ARG, "send and recv overlap without being the same buffers");
  if ((s = grid_fits(M, dt))) return s;
  if ((s = check_ws_bytes(cfg, hier_ws(h, cfg, M, dt), "cc_hierarchical_workspace_size", send, nb, recv, nb, N)))
    return s;
  if ((s = device_ready())) return s;
  hipStream_t st = (hipStream_t)stream;
  if (N == 1 || hier_flat(h)) return run_all_reduce(send, recv, M, dt, (int)op, N, cfg, st);
  uint64_t bnd[kMaxRanks + 1];
  uint32_t seg[kMaxRanks];
  hier_segments(h, M, bnd, seg);
  Red r = red_of(send, recv, M, bnd, dt, (int)op, N, cfg, st);
  if (cfg.fuse_depth == 0)
    return hip_status(launch_hier_fused(r, h.p.data(), h.stride.data(), (int)h.p.size(), h.top, bnd, seg),
                      "hierarchical all_reduce");
  const Plan p = build_hier_plan(h.dims, M);
  hipError_t e = hipSuccess;
  for (const auto& stp : p.steps)
    for (size_t i = 0; i < stp.size() && e == hipSuccess; i += kMaxGDesc)
      e = launch_gsteps(r, stp.data() + i, (int)std::min<size_t>(kMaxGDesc, stp.size() - i));
  return hip_status(e, "hierarchical all_reduce (stepwise)");
}

cc_status_t cc_hierarchical_workspace_size(int ndims, const int* dims, const cc_config_t* cfgp, size_t count,
                                           cc_dtype_t dtype, size_t* bytes) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  Hier h;
  cc_status_t s = hier_args(ndims, dims, &h);
  if (s || (s = hier_cfg_checks(cfg, h.N, dtype))) return s;
  if (!bytes) return fail(CC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)hier_ws(h, cfg, count, (int)dtype);
  return ok();
}

cc_status_t cc_hierarchical_traffic(int ndims, const int* dims, size_t count, cc_dtype_t dtype, uint64_t* level_bytes,
                                    int* level_steps) {
  Hier h;
  cc_status_t s = hier_args(ndims, dims, &h);
  if (s) return s;
  if ((int)dtype < 0 || (int)dtype > 2) return fail(CC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!level_bytes || !level_steps) return fail(CC_ERR_INVALID_ARG, "NULL output");
  for (int i = 0; i < ndims; ++i) {
    level_bytes[i] = 0;
    level_steps[i] = 0;
  }
  if (h.N < 2) return ok();
  const Plan p = build_hier_plan(h.dims, count);
  const uint64_t es = elem_size((int)dtype);
  for (size_t j = 0; j < h.p.size(); ++j) {
    const auto& v = p.level_sent[j];
    level_bytes[h.at[j]] = *std::max_element(v.begin(), v.end()) * es;
    level_steps[h.at[j]] = 2 * (h.p[j] - 1);
  }
  return ok();
}

cc_status_t cc_hierarchical_plan(int ndims, const int* dims, size_t count, cc_plan_op_t* records, size_t cap,
                                 size_t* nrecords) {
  Hier h;
  cc_status_t s = hier_args(ndims, dims, &h);
  if (s) return s;
  if (!nrecords) return fail(CC_ERR_INVALID_ARG, "nrecords is NULL");
  if (h.N < 2) return fail(CC_ERR_UNSUPPORTED, "a single rank has no schedule");
  const Plan p = build_hier_plan(h.dims, count);
  size_t n = 0;
  for (const auto& st : p.steps) n += st.size();
  *nrecords = n;
  if (!records) return ok();
  if (cap < n) return fail(CC_ERR_INVALID_ARG, "cap=%zu is smaller than the %zu records", cap, n);
  size_t i = 0;
  for (size_t k = 0; k < p.steps.size(); ++k)
    for (const GDesc& g : p.steps[k])
      records[i++] = cc_plan_op_t{(uint32_t)k, g.flags, g.dst, g.in1, g.in2, g.lo, g.len};
  return ok();
}

cc_status_t cc_get_traffic(cc_coll_t coll, cc_algo_t algo, int nranks, size_t count, cc_dtype_t dtype,
                           uint64_t* max_bytes, int* steps) {
  cc_config_t cfg = kDefaultCfg;
  cfg.algo = algo;
  cc_status_t s = common_checks(coll, nranks, dtype, &cfg);
  if (s) return s;
  if (!max_bytes || !steps) return fail(CC_ERR_INVALID_ARG, "NULL output");
  const int N = nranks;
  const uint64_t es = elem_size((int)dtype);
  if (coll == CC_COLL_ALL_REDUCE && sched_of(algo, N) >= 0) {
    if (N < 2) {
      *max_bytes = 0;
      *steps = 0;
      return ok();
    }
    const Plan p = build_plan((SchedAlg)sched_of(algo, N), N, count);
    *max_bytes = *std::max_element(p.sent.begin(), p.sent.end()) * es;
    *steps = p.net_steps;
    return ok();
  }
  if (algo != CC_ALGO_RING && coll != CC_COLL_BROADCAST && !is_pow2(N))
    return fail(CC_ERR_UNSUPPORTED, "needs nranks = 2^k");
  // chunk sizes of a per-rank vector of M elements
  auto sizes = [&](uint64_t M) {
    std::vector<uint64_t> z(N);
    for (int c = 0; c < N; ++c)
      z[c] = (uint64_t)(((unsigned __int128)(c + 1) * M) / N - ((unsigned __int128)c * M) / N);
    return z;
  };
  uint64_t best = 0;
  int st = 0;
  const int L = ilog2(N);
  switch (coll) {
    case CC_COLL_ALL_REDUCE: {
      const auto z = sizes(count);
      if (algo == CC_ALGO_RING) {
        // ReduceScatter sends every chunk but (r+1); AllGather every chunk but (r+2)
        for (int r = 0; r < N; ++r) {
          uint64_t t = 0;
          for (int q = 0; q < N - 1; ++q) t += z[((r - q) % N + N) % N] + z[((r + 1 - q) % N + N) % N];
          best = std::max(best, t);
        }
        st = 2 * (N - 1);
      } else if (algo == CC_ALGO_HALVING_DOUBLING) {
        // rank i sends, per halving step with distance d, the half of its
        // range [i & ~(2d-1), +2d) that does not hold chunk i, and per
        // doubling step the range [i & ~(d-1), +d) it holds
        std::vector<uint64_t> pre(N + 1, 0);
        for (int c = 0; c < N; ++c) pre[c + 1] = pre[c] + z[c];
        auto span = [&](int b0, int len) { return pre[b0 + len] - pre[b0]; };
        for (int i = 0; i < N; ++i) {
          uint64_t t = 0;
          for (int d = N / 2; d >= 1; d /= 2) t += span((i & ~(2 * d - 1)) + ((i & d) ? 0 : d), d);
          for (int d = 1; d < N; d *= 2) t += span(i & ~(d - 1), d);
          best = std::max(best, t);
        }
        st = 2 * L;
      } else {
        best = (uint64_t)L * count;
        st = L;
      }
      break;
    }
    case CC_COLL_REDUCE_SCATTER:
    case CC_COLL_ALL_GATHER:
      // count = per-rank shard; every rank sends all chunks but one, for both schedules
      best = (uint64_t)(N - 1) * count;
      st = algo == CC_ALGO_RING ? N - 1 : L;
      if (algo == CC_ALGO_BUTTERFLY) return fail(CC_ERR_UNSUPPORTED, "butterfly is defined for all_reduce only");
      break;
    case CC_COLL_BROADCAST:
      if (algo == CC_ALGO_BUTTERFLY) return fail(CC_ERR_UNSUPPORTED, "butterfly is defined for all_reduce only");
      if (algo == CC_ALGO_RING) {
        best = N > 1 ? count : 0;
        st = N - 1;
      } else {
        best = (uint64_t)L * count;  // the root sends in every doubling step
        st = L;
      }
      break;
    case CC_COLL_ALL_TO_ALL:
      if (algo != CC_ALGO_RING) return fail(CC_ERR_UNSUPPORTED, "all_to_all supports the pairwise schedule only");
      best = (uint64_t)(N - 1) * count;  // count = elements per (source, destination) block
      st = N - 1;
      break;
    default:
      return fail(CC_ERR_INVALID_ARG, "unknown collective");
  }
  *max_bytes = best * es;
  *steps = st;
  return ok();
}

}  // extern "C"
