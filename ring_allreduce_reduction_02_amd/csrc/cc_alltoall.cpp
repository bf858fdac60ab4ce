// C ABI of the AllToAll variants around MoE routing: expert capacity, the
// capacity-padded dispatch and combine, the hierarchical (node-aggregated)
// AllToAll, and the accounting of the pairwise and hierarchical schedules.
// Declared in include/cc.h.  Every variant is a list of copy descriptors
// (k_copies; a descriptor without a source writes zeros), enqueued in phase
// or step order on the caller's stream.

#include <algorithm>
#include <vector>

#include "cc_api_internal.h"
#include "cc_launch.h"

using namespace cc;
using namespace cc::api;

namespace {

constexpr uint64_t kByteLimit = 1ull << 62;

cc_status_t run_copies(const std::vector<CopyDesc>& d, int esize, int blocks_per_cu, hipStream_t st,
                       const char* what) {
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < d.size() && e == hipSuccess; i += kMaxDesc)
    e = launch_copies(d.data() + i, (int)std::min<size_t>(kMaxDesc, d.size() - i), esize, blocks_per_cu, st);
  return hip_status(e, what);
}

cc_status_t a2a_cfg(const cc_config_t& cfg, int nranks, cc_dtype_t dtype) {
  cc_status_t s = common_checks(CC_COLL_ALL_TO_ALL, nranks, dtype, &cfg);
  if (s) return s;
  if (cfg.algo != CC_ALGO_RING)
    return fail(CC_ERR_UNSUPPORTED, "the AllToAll variants run the direct or the pairwise schedule (algo ring)");
  return CC_OK;
}

// ---- capacity-padded MoE exchange
struct Moe {
  int N = 0, E = 0, epr = 0;
  uint64_t cap = 0, rowb = 0;
  std::vector<uint64_t> cnt, kept, disp;  // [N][E], [N][E], [N][E+1] (rows)
  uint64_t token_bytes_max = 0;           // largest token-side buffer
  uint64_t expert_bytes = 0;              // expert-side buffer: E * cap rows
};

cc_status_t moe_geom(const size_t* counts, int N, int E, size_t cap, size_t elem_per_row, int es, Moe* m) {
  if (!counts) return fail(CC_ERR_INVALID_ARG, "counts is NULL");
  if (E < N || E % N) return fail(CC_ERR_INVALID_ARG, "nexperts=%d must be a positive multiple of nranks=%d", E, N);
  if (elem_per_row == 0) return fail(CC_ERR_INVALID_ARG, "elem_per_row is 0");
  const unsigned __int128 rowb = (unsigned __int128)elem_per_row * es;
  if (rowb >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "row too large");
  const unsigned __int128 eb = (unsigned __int128)E * cap * rowb;
  if (eb >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "nexperts * capacity rows too large");
  m->N = N;
  m->E = E;
  m->epr = E / N;
  m->cap = cap;
  m->rowb = (uint64_t)rowb;
  m->expert_bytes = (uint64_t)eb;
  m->cnt.assign((size_t)N * E, 0);
  m->kept.assign((size_t)N * E, 0);
  m->disp.assign((size_t)N * (E + 1), 0);
  for (int i = 0; i < N; ++i) {
    unsigned __int128 rows = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t c = counts[(size_t)i * E + e];
      m->cnt[(size_t)i * E + e] = c;
      m->kept[(size_t)i * E + e] = std::min<uint64_t>(c, cap);
      m->disp[(size_t)i * (E + 1) + e] = (uint64_t)rows;
      rows += c;
      if (rows * rowb >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "rank %d sends too many rows", i);
    }
    m->disp[(size_t)i * (E + 1) + E] = (uint64_t)rows;
    m->token_bytes_max = std::max(m->token_bytes_max, (uint64_t)(rows * rowb));
  }
  return CC_OK;
}

// Descriptors moving block (token rank i, expert e) between the token side
// (rows at disp[i][e]) and the expert side (rank e / epr, slot block
// (i * epr + e % epr) * cap): kept rows copied, the rest zero-filled on the
// receiving side.
void moe_block(const Moe& m, const cc_rankbuf_t& tok, const cc_rankbuf_t& exp, int i, int e, bool dispatch,
               std::vector<CopyDesc>* d) {
  const int j = e / m.epr, l = e % m.epr;
  const uint64_t n = m.kept[(size_t)i * m.E + e], c = m.cnt[(size_t)i * m.E + e];
  char* tb = (char*)tok.base + (uint64_t)i * tok.rank_stride_bytes + m.disp[(size_t)i * (m.E + 1) + e] * m.rowb;
  char* xb = (char*)exp.base + (uint64_t)j * exp.rank_stride_bytes + ((uint64_t)i * m.epr + l) * m.cap * m.rowb;
  if (dispatch) {
    if (n) d->push_back(CopyDesc{tb, xb, n * m.rowb});
    if (m.cap > n) d->push_back(CopyDesc{nullptr, xb + n * m.rowb, (m.cap - n) * m.rowb});
  } else {
    if (n) d->push_back(CopyDesc{xb, tb, n * m.rowb});
    if (c > n) d->push_back(CopyDesc{nullptr, tb + n * m.rowb, (c - n) * m.rowb});
  }
}

typedef std::vector<std::vector<CopyDesc>> Steps;

cc_status_t launch_steps(const Steps& steps, int esize, int blocks_per_cu, hipStream_t st, const char* what) {
  for (const auto& d : steps) {
    cc_status_t s = run_copies(d, esize, blocks_per_cu, st, what);
    if (s) return s;
  }
  return ok();
}

// Validates a padded dispatch (or combine) and builds its copies, one list
// per step: every transfer at once for fuse_depth 0, else the pairwise steps.
cc_status_t moe_build(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts, size_t capacity,
                      size_t elem_per_row, cc_dtype_t dtype, int nranks, const cc_config_t& cfg, bool dispatch,
                      Steps* steps) {
  cc_status_t s = a2a_cfg(cfg, nranks, dtype);
  if (s) return s;
  const int N = nranks, es = elem_size((int)dtype);
  Moe m;
  if ((s = moe_geom(counts, N, nexperts, capacity, elem_per_row, es, &m))) return s;
  const cc_rankbuf_t& tok = dispatch ? send : recv;
  const cc_rankbuf_t& exp = dispatch ? recv : send;
  if ((s = check_side(tok, m.token_bytes_max, N, dispatch ? "send" : "recv")) ||
      (s = check_side(exp, m.expert_bytes, N, dispatch ? "recv" : "send")))
    return s;
  if (sides_overlap(tok, m.token_bytes_max, N, exp, m.expert_bytes, N))
    return fail(CC_ERR_INVALID_ARG, "send and recv overlap");
  steps->clear();
  if (cfg.fuse_depth == 0) {
    steps->emplace_back();
    auto& d = steps->back();
    if (dispatch) {
      for (int j = 0; j < N; ++j)
        for (int i = 0; i < N; ++i)
          for (int l = 0; l < m.epr; ++l) moe_block(m, tok, exp, i, j * m.epr + l, true, &d);
    } else {
      for (int i = 0; i < N; ++i)
        for (int e = 0; e < m.E; ++e) moe_block(m, tok, exp, i, e, false, &d);
    }
    return CC_OK;
  }
  // pairwise: at step k the sender r serves the pair (r, r + k)
  for (int k = 0; k < N; ++k) {
    steps->emplace_back();
    for (int r = 0; r < N; ++r) {
      const int q = (r + k) % N;
      const int i = dispatch ? r : q, j = dispatch ? q : r;  // token rank, expert rank
      for (int l = 0; l < m.epr; ++l) moe_block(m, tok, exp, i, j * m.epr + l, dispatch, &steps->back());
    }
  }
  return CC_OK;
}

// ---- AllToAll(v) geometry: per-block byte counts and displacements
struct A2A {
  int N = 0;
  std::vector<uint64_t> b, sd, rd;  // [N][N] bytes i -> j, send displacement on i, recv displacement on j
  uint64_t smax = 0, rmax = 0;
};

cc_status_t a2a_geom(const size_t* counts, int N, size_t elem_per_row, int es, A2A* g) {
  if (!counts) return fail(CC_ERR_INVALID_ARG, "counts is NULL");
  if (elem_per_row == 0) return fail(CC_ERR_INVALID_ARG, "elem_per_row is 0");
  const unsigned __int128 rowb = (unsigned __int128)elem_per_row * es;
  g->N = N;
  g->b.assign((size_t)N * N, 0);
  g->sd.assign((size_t)N * N, 0);
  g->rd.assign((size_t)N * N, 0);
  std::vector<unsigned __int128> st(N, 0), rt(N, 0);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) {
      const unsigned __int128 x = (unsigned __int128)counts[(size_t)i * N + j] * rowb;
      if (x >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "counts[%d][%d] too large", i, j);
      g->b[(size_t)i * N + j] = (uint64_t)x;
      g->sd[(size_t)i * N + j] = (uint64_t)st[i];
      st[i] += x;
      if (st[i] >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "send size too large");
    }
  for (int j = 0; j < N; ++j)
    for (int i = 0; i < N; ++i) {
      g->rd[(size_t)i * N + j] = (uint64_t)rt[j];
      rt[j] += g->b[(size_t)i * N + j];
      if (rt[j] >= kByteLimit) return fail(CC_ERR_INVALID_ARG, "recv size too large");
    }
  for (int r = 0; r < N; ++r) {
    g->smax = std::max(g->smax, (uint64_t)st[r]);
    g->rmax = std::max(g->rmax, (uint64_t)rt[r]);
  }
  return CC_OK;
}

// ---- hierarchical AllToAll: staging layout of the node-pair payloads
struct Hier2 {
  int P = 0, L = 0, G = 0;
  // payload of ordered node pair (n, n2), n2 != n: offset in a staging area,
  // and the offset of block (source local l, destination local l2) in it
  std::vector<uint64_t> pair_off;  // [G][G]
  std::vector<uint64_t> sub_off;   // [P][P] (source rank, destination rank) for inter-node blocks
  uint64_t inter = 0;              // bytes of all payloads
};

void hier2_layout(const A2A& g, int L, Hier2* h) {
  h->P = g.N;
  h->L = L;
  h->G = g.N / L;
  h->pair_off.assign((size_t)h->G * h->G, 0);
  h->sub_off.assign((size_t)g.N * g.N, 0);
  uint64_t at = 0;
  for (int n = 0; n < h->G; ++n)
    for (int n2 = 0; n2 < h->G; ++n2) {
      if (n2 == n) continue;
      h->pair_off[(size_t)n * h->G + n2] = at;
      uint64_t in = 0;
      for (int l = 0; l < L; ++l)
        for (int l2 = 0; l2 < L; ++l2) {
          const int i = n * L + l, j = n2 * L + l2;
          h->sub_off[(size_t)i * g.N + j] = in;
          in += g.b[(size_t)i * g.N + j];
        }
      at += in;
    }
  h->inter = at;
}

uint64_t hier2_ws(const Hier2& h) { return h.inter ? 2 * rup(h.inter, 256) : 0; }

cc_status_t hier2_args(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype, int nranks, int local_size,
                       A2A* g, Hier2* h) {
  if (nranks < 1 || nranks > CC_MAX_RANKS) return fail(CC_ERR_INVALID_ARG, "nranks=%d", nranks);
  if ((int)dtype < 0 || (int)dtype > 2) return fail(CC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (local_size < 1 || nranks % local_size)
    return fail(CC_ERR_INVALID_ARG, "local_size=%d must divide nranks=%d", local_size, nranks);
  cc_status_t s = a2a_geom(counts, nranks, elem_per_row, elem_size((int)dtype), g);
  if (s) return s;
  hier2_layout(*g, local_size, h);
  return CC_OK;
}

bool steps_empty(const Steps& steps) {
  for (const auto& d : steps)
    if (!d.empty()) return false;
  return true;
}

// Validates a hierarchical AllToAll and builds its three phases.
cc_status_t hier2_build(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, size_t elem_per_row,
                        cc_dtype_t dtype, int nranks, int local_size, const cc_config_t& cfg, Steps* steps) {
  cc_status_t s = a2a_cfg(cfg, nranks, dtype);
  if (s) return s;
  A2A g;
  Hier2 h;
  if ((s = hier2_args(counts, elem_per_row, dtype, nranks, local_size, &g, &h))) return s;
  const int P = nranks, L = local_size, G = P / L;
  if ((s = check_side(send, g.smax, P, "send")) || (s = check_side(recv, g.rmax, P, "recv"))) return s;
  if (sides_overlap(send, g.smax, P, recv, g.rmax, P)) return fail(CC_ERR_INVALID_ARG, "send and recv overlap");
  const uint64_t need = hier2_ws(h);
  if (need && (cfg.workspace == nullptr || cfg.workspace_bytes < need))
    return fail(CC_ERR_INVALID_ARG,
                "this exchange needs %llu bytes of workspace (cc_all_to_all_hierarchical_workspace_size); got %zu",
                (unsigned long long)need, cfg.workspace ? cfg.workspace_bytes : (size_t)0);
  if (need) {
    const cc_rankbuf_t ws{cfg.workspace, need};
    if (sides_overlap(ws, need, 1, send, g.smax, P) || sides_overlap(ws, need, 1, recv, g.rmax, P))
      return fail(CC_ERR_INVALID_ARG, "the workspace overlaps send or recv");
  }
  char* A = (char*)cfg.workspace;                          // payloads at the aggregators
  char* B = need ? A + rup(h.inter, 256) : nullptr;        // payloads at the receivers
  auto sp = [&](int i, int j) {
    return (const char*)send.base + (uint64_t)i * send.rank_stride_bytes + g.sd[(size_t)i * P + j];
  };
  auto rp = [&](int i, int j) { return (char*)recv.base + (uint64_t)j * recv.rank_stride_bytes + g.rd[(size_t)i * P + j]; };
  auto at = [&](char* area, int i, int j) {
    return area + h.pair_off[(size_t)(i / L) * G + j / L] + h.sub_off[(size_t)i * P + j];
  };
  steps->assign(3, {});
  // 1. aggregate: blocks inside the node go to their destination, blocks
  //    for another node into that node pair's payload
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j) {
      const uint64_t n = g.b[(size_t)i * P + j];
      if (n) (*steps)[0].push_back(CopyDesc{sp(i, j), i / L == j / L ? rp(i, j) : at(A, i, j), n});
    }
  // 2. exchange: one transfer per ordered node pair
  for (int n = 0; n < G; ++n)
    for (int n2 = 0; n2 < G; ++n2) {
      if (n2 == n) continue;
      const uint64_t o = h.pair_off[(size_t)n * G + n2];
      uint64_t bytes = 0;
      for (int l = 0; l < L; ++l)
        for (int l2 = 0; l2 < L; ++l2) bytes += g.b[(size_t)(n * L + l) * P + n2 * L + l2];
      if (bytes) (*steps)[1].push_back(CopyDesc{A + o, B + o, bytes});
    }
  // 3. distribute inside the destination node
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j) {
      const uint64_t n = g.b[(size_t)i * P + j];
      if (n && i / L != j / L) (*steps)[2].push_back(CopyDesc{at(B, i, j), rp(i, j), n});
    }
  return CC_OK;
}

}  // namespace

extern "C" {

cc_status_t cc_moe_capacity(int nranks, size_t tokens, int topk, int nexperts, int factor_num, int factor_den,
                            size_t* capacity) {
  if (nranks < 1 || topk < 1 || nexperts < 1 || factor_num < 1 || factor_den < 1)
    return fail(CC_ERR_INVALID_ARG, "nranks, topk, nexperts and the factor must be positive");
  if (!capacity) return fail(CC_ERR_INVALID_ARG, "capacity is NULL");
  const unsigned __int128 num = (unsigned __int128)nranks * tokens * (unsigned)topk * (unsigned)factor_num;
  const unsigned __int128 den = (unsigned __int128)(unsigned)nexperts * (unsigned)factor_den;
  const unsigned __int128 c = (num + den - 1) / den;
  if (c >> 62) return fail(CC_ERR_INVALID_ARG, "capacity too large");
  *capacity = (size_t)c;
  return ok();
}

}  // extern "C"

namespace {

// The padded dispatch (or combine): validated and planned by moe_build, then
// run as copy descriptors step by step (direct: one step; pairwise: N).  A
// one-launch row kernel (one workgroup per output row) was measured against
// this and lost once the copy kernel moved two vectors per thread: C = 1.25
// dispatch 5.60 TB/s against 6.24-6.27, zero fill 5.36-5.42 against 6.17.
cc_status_t moe_exchange(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts, size_t capacity,
                         size_t elem_per_row, cc_dtype_t dtype, int nranks, const cc_config_t& cfg, bool dispatch,
                         hipStream_t st) {
  Steps steps;
  cc_status_t s = moe_build(send, recv, counts, nexperts, capacity, elem_per_row, dtype, nranks, cfg, dispatch, &steps);
  if (s) return s;
  if (steps_empty(steps)) return ok();
  if ((s = device_ready())) return s;
  return launch_steps(steps, elem_size((int)dtype), cfg.blocks_per_cu, st,
                      dispatch ? "padded MoE dispatch" : "padded MoE combine");
}

}  // namespace

extern "C" {

cc_status_t cc_moe_dispatch_padded(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts,
                                   size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                   const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  return moe_exchange(send, recv, counts, nexperts, capacity, elem_per_row, dtype, nranks, cfg, true,
                      (hipStream_t)stream);
}

cc_status_t cc_moe_combine_padded(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts, int nexperts,
                                  size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                  const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  return moe_exchange(send, recv, counts, nexperts, capacity, elem_per_row, dtype, nranks, cfg, false,
                      (hipStream_t)stream);
}

cc_status_t cc_all_to_all_plan(cc_a2a_kind_t kind, cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts,
                               int nexperts, size_t capacity, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                               int local_size, const cc_config_t* cfgp, cc_copy_op_t* records, size_t cap,
                               size_t* nrecords) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  if (!nrecords) return fail(CC_ERR_INVALID_ARG, "nrecords is NULL");
  Steps steps;
  cc_status_t s;
  switch (kind) {
    case CC_A2A_MOE_DISPATCH:
    case CC_A2A_MOE_COMBINE:
      s = moe_build(send, recv, counts, nexperts, capacity, elem_per_row, dtype, nranks, cfg,
                    kind == CC_A2A_MOE_DISPATCH, &steps);
      break;
    case CC_A2A_HIERARCHICAL:
      s = hier2_build(send, recv, counts, elem_per_row, dtype, nranks, local_size, cfg, &steps);
      break;
    default:
      return fail(CC_ERR_INVALID_ARG, "unknown exchange kind %d", (int)kind);
  }
  if (s) return s;
  size_t n = 0;
  for (const auto& d : steps) n += d.size();
  *nrecords = n;
  if (!records) return ok();
  if (cap < n) return fail(CC_ERR_INVALID_ARG, "cap=%zu is smaller than the %zu records", cap, n);
  size_t i = 0;
  for (size_t k = 0; k < steps.size(); ++k)
    for (const CopyDesc& c : steps[k])
      records[i++] = cc_copy_op_t{(uint32_t)k, 0u, (uint64_t)(uintptr_t)c.src, (uint64_t)(uintptr_t)c.dst, c.bytes};
  return ok();
}

cc_status_t cc_all_to_all_hierarchical_workspace_size(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype,
                                                      int nranks, int local_size, size_t* bytes) {
  A2A g;
  Hier2 h;
  cc_status_t s = hier2_args(counts, elem_per_row, dtype, nranks, local_size, &g, &h);
  if (s) return s;
  if (!bytes) return fail(CC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)hier2_ws(h);
  return ok();
}

cc_status_t cc_all_to_all_hierarchical(cc_rankbuf_t send, cc_rankbuf_t recv, const size_t* counts,
                                       size_t elem_per_row, cc_dtype_t dtype, int nranks, int local_size,
                                       const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  Steps steps;
  cc_status_t s = hier2_build(send, recv, counts, elem_per_row, dtype, nranks, local_size, cfg, &steps);
  if (s) return s;
  if (steps_empty(steps)) return ok();
  if ((s = device_ready())) return s;
  return launch_steps(steps, elem_size((int)dtype), cfg.blocks_per_cu, (hipStream_t)stream,
                      "hierarchical all_to_all");
}

cc_status_t cc_all_to_all_traffic(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                  int local_size, int* flows, uint64_t* total_bytes, uint64_t* max_rank_bytes) {
  A2A g;
  Hier2 h;
  cc_status_t s = hier2_args(counts, elem_per_row, dtype, nranks, local_size, &g, &h);
  if (s) return s;
  if (!flows || !total_bytes || !max_rank_bytes) return fail(CC_ERR_INVALID_ARG, "NULL output");
  const int P = nranks, L = local_size, G = P / L;
  std::vector<std::vector<uint64_t>> sent(4, std::vector<uint64_t>(P, 0));
  for (int k = 0; k < 4; ++k) {
    flows[k] = 0;
    total_bytes[k] = 0;
  }
  auto add = [&](int ph, int src, int dst, uint64_t n) {
    if (src == dst || n == 0) return;
    ++flows[ph];
    total_bytes[ph] += n;
    sent[ph][src] += n;
  };
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j) add(0, i, j, g.b[(size_t)i * P + j]);
  for (int i = 0; i < P; ++i) {
    const int n = i / L;
    for (int j = 0; j < P; ++j)
      if (j / L == n) add(1, i, j, g.b[(size_t)i * P + j]);
    for (int n2 = 0; n2 < G; ++n2) {
      if (n2 == n) continue;
      uint64_t rows = 0;
      for (int l2 = 0; l2 < L; ++l2) rows += g.b[(size_t)i * P + n2 * L + l2];
      add(1, i, n * L + n2 % L, rows);
    }
  }
  for (int n = 0; n < G; ++n)
    for (int n2 = 0; n2 < G; ++n2) {
      if (n2 == n) continue;
      uint64_t bytes = 0;
      for (int l = 0; l < L; ++l)
        for (int l2 = 0; l2 < L; ++l2) {
          const int i = n * L + l, j = n2 * L + l2;
          bytes += g.b[(size_t)i * P + j];
          add(3, n2 * L + n % L, j, g.b[(size_t)i * P + j]);
        }
      add(2, n * L + n2 % L, n2 * L + n % L, bytes);
    }
  for (int k = 0; k < 4; ++k) max_rank_bytes[k] = *std::max_element(sent[k].begin(), sent[k].end());
  return ok();
}

cc_status_t cc_all_to_all_step_bytes(const size_t* counts, size_t elem_per_row, cc_dtype_t dtype, int nranks,
                                     uint64_t* step_max, uint64_t* step_total) {
  if (nranks < 1 || nranks > CC_MAX_RANKS) return fail(CC_ERR_INVALID_ARG, "nranks=%d", nranks);
  if ((int)dtype < 0 || (int)dtype > 2) return fail(CC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!step_max || !step_total) return fail(CC_ERR_INVALID_ARG, "NULL output");
  A2A g;
  cc_status_t s = a2a_geom(counts, nranks, elem_per_row, elem_size((int)dtype), &g);
  if (s) return s;
  const int N = nranks;
  for (int k = 0; k < N; ++k) {
    step_max[k] = 0;
    step_total[k] = 0;
    for (int i = 0; i < N; ++i) {
      const uint64_t n = g.b[(size_t)i * N + (i + k) % N];
      step_max[k] = std::max(step_max[k], n);
      step_total[k] += n;
    }
  }
  return ok();
}

}  // extern "C"
