// C ABI of the block-wise INT8 compression with error feedback and of the
// AllReduce of the compressed contributions.  Declared in include/cc.h.

#include <algorithm>

#include "cc_api_internal.h"
#include "cc_launch.h"

using namespace cc;
using namespace cc::api;

namespace {

uint64_t q_blocks(uint64_t M) { return (M + kQBlock - 1) / kQBlock; }

cc_status_t q_checks(int nranks, cc_dtype_t dtype, const cc_config_t& cfg, uint64_t M) {
  cc_status_t s = common_checks(CC_COLL_ALL_REDUCE, nranks, dtype, &cfg);
  if (s) return s;
  if (dtype != CC_FLOAT32 && dtype != CC_BFLOAT16)
    return fail(CC_ERR_UNSUPPORTED, "INT8 compression takes float32 or bf16 gradients");
  if (cfg.algo != CC_ALGO_RING)
    return fail(CC_ERR_UNSUPPORTED, "the compressed AllReduce folds in the ring order (algo ring)");
  if (cfg.grid_sync) return fail(CC_ERR_UNSUPPORTED, "grid_sync is not available here");
  // the compression kernels tile by 512 elements (4 per lane): the grid's
  // work-items must fit 32 bits
  const uint64_t tiles = (M + 511) / 512;
  if (tiles * (uint64_t)kBlock > 0xffffffffull) return fail(CC_ERR_INVALID_ARG, "count too large for one launch");
  return CC_OK;
}

bool al(const cc_rankbuf_t& b) { return al16p(b.base) && al16(b.rank_stride_bytes); }

struct Side2 {
  const cc_rankbuf_t* b;
  uint64_t n;
  const char* name;
};

// every pair of the listed buffers disjoint, except pairs marked same-allowed
cc_status_t disjoint(const Side2* s, int n, int N, int same_a = -1, int same_b = -1) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j) {
      if (i == same_a && j == same_b && same_side(*s[i].b, *s[j].b)) continue;
      if (sides_overlap(*s[i].b, s[i].n, N, *s[j].b, s[j].n, N))
        return fail(CC_ERR_INVALID_ARG, "%s and %s overlap", s[i].name, s[j].name);
    }
  return CC_OK;
}

QLaunch q_launch(const cc_rankbuf_t& g, const cc_rankbuf_t& e, const cc_rankbuf_t& q, const cc_rankbuf_t& s,
                 const cc_rankbuf_t& r, uint64_t M, int N, int dt, int vec_ok,
                 const cc_config_t& cfg, cc_stream_t st) {
  return QLaunch{(const char*)g.base, g.rank_stride_bytes, (char*)e.base, e.rank_stride_bytes,
                 (char*)q.base,       q.rank_stride_bytes, (char*)s.base, s.rank_stride_bytes,
                 (char*)r.base,       r.rank_stride_bytes, M, N, dt, vec_ok, cfg.blocks_per_cu,
                 (hipStream_t)st};
}

// workspace of the two-kernel form: int8 values, then scales, rank-strided
uint64_t ws_q_stride(uint64_t M) { return rup(M, 256); }
uint64_t ws_s_stride(uint64_t M) { return rup(4 * q_blocks(M), 256); }
uint64_t ws_bytes(int N, uint64_t M) { return (uint64_t)N * (ws_q_stride(M) + ws_s_stride(M)); }

}  // namespace

extern "C" {

cc_status_t cc_quantize_ef(cc_rankbuf_t grad, cc_rankbuf_t err, cc_rankbuf_t q, cc_rankbuf_t scales, size_t count,
                           cc_dtype_t dtype, int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  const uint64_t M = count;
  cc_status_t s = q_checks(nranks, dtype, cfg, M);
  if (s) return s;
  if (M == 0) return ok();
  const int N = nranks, es = elem_size((int)dtype);
  const Side2 sd[] = {{&grad, M * es, "grad"}, {&err, M * 4, "err"}, {&q, M, "q"}, {&scales, 4 * q_blocks(M), "scales"}};
  for (const Side2& x : sd)
    if ((s = check_side(*x.b, x.n, N, x.name))) return s;
  if ((s = disjoint(sd, 4, N))) return s;
  if ((s = device_ready())) return s;
  const int vec_ok = al(grad) && al(err) && al(q) && al(scales);
  const cc_rankbuf_t none{nullptr, 0};
  return hip_status(launch_quant_ef(q_launch(grad, err, q, scales, none, M, N, (int)dtype, vec_ok, cfg,
                                             stream)),
                    "int8 quantize with error feedback");
}

cc_status_t cc_all_reduce_dequant(cc_rankbuf_t q, cc_rankbuf_t scales, cc_rankbuf_t recv, size_t count,
                                  cc_dtype_t dtype, int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  const uint64_t M = count;
  cc_status_t s = q_checks(nranks, dtype, cfg, M);
  if (s) return s;
  if (M == 0) return ok();
  const int N = nranks, es = elem_size((int)dtype);
  const Side2 sd[] = {{&q, M, "q"}, {&scales, 4 * q_blocks(M), "scales"}, {&recv, M * es, "recv"}};
  for (const Side2& x : sd)
    if ((s = check_side(*x.b, x.n, N, x.name))) return s;
  if ((s = disjoint(sd, 3, N))) return s;
  if ((s = device_ready())) return s;
  const int vec_ok = al(q) && al(scales) && al(recv);
  const cc_rankbuf_t none{nullptr, 0};
  return hip_status(launch_dequant_reduce(q_launch(none, none, q, scales, recv, M, N, (int)dtype, vec_ok, cfg,
                                                   stream)),
                    "all_reduce of int8 messages");
}

cc_status_t cc_all_reduce_int8_ef(cc_rankbuf_t grad, cc_rankbuf_t err, cc_rankbuf_t recv, size_t count,
                                  cc_dtype_t dtype, int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  const uint64_t M = count;
  cc_status_t s = q_checks(nranks, dtype, cfg, M);
  if (s) return s;
  if (M == 0) return ok();
  const int N = nranks, es = elem_size((int)dtype);
  const Side2 sd[] = {{&grad, M * es, "grad"}, {&recv, M * es, "recv"}, {&err, M * 4, "err"}};
  for (const Side2& x : sd)
    if ((s = check_side(*x.b, x.n, N, x.name))) return s;
  if ((s = disjoint(sd, 3, N, 0, 1))) return s;  // grad and recv may be the same buffers
  const uint64_t need = cfg.fuse_depth == 0 ? 0 : ws_bytes(N, M);
  if (need && (cfg.workspace == nullptr || cfg.workspace_bytes < need))
    return fail(CC_ERR_INVALID_ARG, "this schedule needs %llu bytes of workspace (cc_int8_ef_workspace_size); got %zu",
                (unsigned long long)need, cfg.workspace ? cfg.workspace_bytes : (size_t)0);
  cc_rankbuf_t qb{nullptr, 0}, sb{nullptr, 0};
  if (need) {
    qb = cc_rankbuf_t{cfg.workspace, (size_t)ws_q_stride(M)};
    sb = cc_rankbuf_t{(char*)cfg.workspace + (uint64_t)N * ws_q_stride(M), (size_t)ws_s_stride(M)};
    const cc_rankbuf_t ws{cfg.workspace, (size_t)need};
    for (const Side2& x : sd)
      if (sides_overlap(ws, need, 1, *x.b, x.n, N))
        return fail(CC_ERR_INVALID_ARG, "the workspace overlaps %s", x.name);
  }
  if ((s = device_ready())) return s;
  if (!need) {
    const int vec_ok = al(grad) && al(err) && al(recv);
    return hip_status(launch_quant_ef_fused(q_launch(grad, err, qb, sb, recv, M, N, (int)dtype, vec_ok, cfg,
                                                     stream)),
                      "int8 all_reduce with error feedback");
  }
  const int vec_ok = al(grad) && al(err) && al(recv) && al(qb) && al(sb);
  hipError_t e = launch_quant_ef(q_launch(grad, err, qb, sb, recv, M, N, (int)dtype, vec_ok, cfg, stream));
  if (e == hipSuccess) e = launch_dequant_reduce(q_launch(grad, err, qb, sb, recv, M, N, (int)dtype, vec_ok, cfg, stream));
  return hip_status(e, "int8 all_reduce with error feedback (two kernels)");
}

cc_status_t cc_int8_ef_workspace_size(const cc_config_t* cfgp, int nranks, size_t count, cc_dtype_t dtype,
                                      size_t* bytes) {
  const cc_config_t& cfg = cfgp ? *cfgp : kDefaultCfg;
  cc_status_t s = q_checks(nranks, dtype, cfg, count);
  if (s) return s;
  if (!bytes) return fail(CC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = cfg.fuse_depth == 0 || count == 0 ? 0 : (size_t)ws_bytes(nranks, count);
  return ok();
}

cc_status_t cc_int8_message_bytes(size_t count, size_t* bytes) {
  if (!bytes) return fail(CC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)(count + 4 * q_blocks(count));
  return ok();
}

}  // extern "C"
