// The launch guard's rule, free of HIP so that a host test can compile it: a
// workgroup's static LDS (its kernel's __shared__ declarations) plus the
// dynamic reservation (the occupancy cap) must not exceed the device's
// per-workgroup limit.  A launch beyond it faulted the GPU once, when a
// kernel with a 4-byte static word was given the whole 160 KiB reservation.
#pragma once

// true when the workgroup's LDS fits; an unknown limit (<= 0) leaves the
// decision to the runtime
inline bool lds_fits(unsigned static_bytes, unsigned dynamic_bytes, int lds_per_block) {
  if (lds_per_block <= 0) return true;
  return (unsigned long long)static_bytes + dynamic_bytes <= (unsigned long long)lds_per_block;
}
