// lsa_forward_noalloc: lsa_forward with its workspace in a file-scope device array, for
// callers that cannot allocate device memory (code under HIP graph capture, serving
// loops that forbid allocation, harnesses that forbid it).
//
// The array `scratch` below is LSA_NOALLOC_SCRATCH_BYTES of device memory that every GPU
// the library runs on holds until the process ends.  In host code its name is only a
// host-side stand-in: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is handed to
// kernels.  Every call on one GPU shares the array, so calls that overlap on one GPU (on
// different streams, or from several host threads without ordering) race.  No kernel of
// lsa_forward needs its workspace cleared beforehand: every counter it uses is cleared
// by a kernel of the same call, so the contents left by an earlier call do no harm.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lsa.h"

#define LSA_API extern "C" __attribute__((visibility("default")))

static __device__ __align__(256) unsigned char scratch[LSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The current device's address of `scratch`, looked up on its first use on that device.
lsa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LSA_ERR_HIP;
  if (dev >= kMaxDevices) return LSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LSA_OK;
}

}  // namespace

LSA_API lsa_status lsa_forward_noalloc(const lsa_forward_args* a, void* stream) {
  // sizes first: a call whose chunk (the requested chunk_rows, else one row) needs more
  // than the array is rejected before anything is looked up or launched
  int64_t rows = 0;
  int32_t split = 0;
  const lsa_status st = lsa_forward_plan(a, LSA_NOALLOC_SCRATCH_BYTES, &rows, &split);
  if (st != LSA_OK) return st;
  if (rows == 0) return LSA_OK;  // nothing to do
  void* ws = nullptr;
  const lsa_status sa = scratch_address(&ws);
  if (sa != LSA_OK) return sa;
  return lsa_forward(a, ws, LSA_NOALLOC_SCRATCH_BYTES, stream);
}
