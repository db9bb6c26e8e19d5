// msa_backward_noalloc: msa_backward with its scratch in a static device
// array instead of a caller-provided buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as an address: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept.  All calls on one GPU share its array, so
// calls that overlap on one GPU (different streams, or threads) race; the
// backward's preprocess clears everything that must start at zero on every
// call, so a call never sees the previous call's contents.
#include <hip/hip_runtime.h>

#include <mutex>

#include "msa_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of this device's copy of `scratch` (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" int msa_backward_noalloc(const msa_problem* p, const void* q, const void* k, const void* v,
                                    const void* out, const void* dout, const float* lse,
                                    const int32_t* cu_seqlens, const int32_t* sched, void* dq, void* dk,
                                    void* dv, void* stream) {
  size_t need = 0;
  const int st = msa_backward_scratch_bytes(p, &need);
  if (st != MSA_OK) return st;
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_SCRATCH_LIMIT;
  void* ptr = nullptr;
  const int sa = scratch_address(&ptr);
  if (sa != MSA_OK) return sa;
  return msa_backward(p, q, k, v, out, dout, lse, cu_seqlens, sched, ptr, dq, dk, dv, stream);
}
