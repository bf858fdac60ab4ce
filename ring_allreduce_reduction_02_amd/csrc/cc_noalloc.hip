// cc_all_reduce_noalloc: cc_all_reduce with its staging in a fixed device
// array of this library instead of a caller-owned workspace, for callers that
// cannot allocate device memory.  Declared in include/cc.h.
//
// The array, `scratch`, is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy for the life of the process.  Host code
// never uses the name `scratch` as an address (on the host it names a
// stand-in, not device memory); the device address of the current GPU's copy
// comes from hipGetSymbolAddress, taken once per device on the first call
// made with that device current, and is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/cc.h"
#include "cc_api_internal.h"

using namespace cc::api;

static_assert(CC_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size is a multiple of its alignment");

static __device__ __align__(256) unsigned char scratch[CC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

// The device address of the current GPU's `scratch`, looked up once per device.
cc_status_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CC_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(CC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return CC_OK;
}

}  // namespace

extern "C" cc_status_t cc_all_reduce_noalloc(cc_rankbuf_t send, cc_rankbuf_t recv, size_t count, cc_dtype_t dtype,
                                             cc_op_t op, int nranks, const cc_config_t* cfgp, cc_stream_t stream) {
  cc_config_t cfg = cfgp ? *cfgp : kDefaultCfg;
  if (cfg.workspace != nullptr || cfg.workspace_bytes != 0)
    return fail(CC_ERR_INVALID_ARG, "cc_all_reduce_noalloc takes no workspace (cfg.workspace must be NULL, 0 bytes)");
  size_t need = 0;
  cc_status_t s = cc_workspace_size(CC_COLL_ALL_REDUCE, &cfg, nranks, count, dtype, &need);
  if (s) return s;
  if (need > (size_t)CC_NOALLOC_SCRATCH_BYTES)
    return fail(CC_ERR_INVALID_ARG,
                "this schedule needs %zu bytes of staging; the library's fixed scratch holds %zu "
                "(use cc_all_reduce with a workspace)",
                need, (size_t)CC_NOALLOC_SCRATCH_BYTES);
  if (need > 0 && count > 0 && nranks > 1) {
    if ((s = device_ready())) return s;
    void* p = nullptr;
    if ((s = scratch_ptr(&p))) return s;
    cfg.workspace = p;
    cfg.workspace_bytes = CC_NOALLOC_SCRATCH_BYTES;
  }
  return cc_all_reduce(send, recv, count, dtype, op, nranks, &cfg, stream);
}
