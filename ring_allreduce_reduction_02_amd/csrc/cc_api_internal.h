// Argument checks and status reporting shared by the C-ABI source files
// (defined in cc_api.cpp).  Host-side only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cc.h"

namespace cc {
namespace api {

// set the thread's last-error text and return s
cc_status_t fail(cc_status_t s, const char* fmt, ...);
// clear the last-error text and return CC_OK
cc_status_t ok();
// CC_OK, or CC_ERR_HIP naming `what`
cc_status_t hip_status(hipError_t e, const char* what);
// CC_ERR_NO_DEVICE when no HIP device is visible
cc_status_t device_ready();

bool is_pow2(int n);
int ilog2(int n);
bool al16(uint64_t v);
bool al16p(const void* p);
uint64_t rup(uint64_t v, uint64_t a);

// {CC_ALGO_RING, 0, NULL, 0, 0, 0}: what a NULL cc_config_t* means
extern const cc_config_t kDefaultCfg;

// rank count, dtype and the config fields every collective validates
cc_status_t common_checks(cc_coll_t coll, int nranks, cc_dtype_t dtype, const cc_config_t* cfg);
// nbytes per rank buffer: base set when there is data, stride covering a rank
cc_status_t check_side(const cc_rankbuf_t& s, uint64_t nbytes, int N, const char* name);
// any byte shared between a rank buffer of a and one of b
bool sides_overlap(const cc_rankbuf_t& a, uint64_t abytes, int an, const cc_rankbuf_t& b, uint64_t bbytes, int bn);
bool same_side(const cc_rankbuf_t& a, const cc_rankbuf_t& b);

}  // namespace api
}  // namespace cc
