// q4_noalloc.hip -- q4_linear for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): the same layer, with the workspace taken from a
// file-scope device array instead of a caller-provided buffer.
//
// The array exists once per GPU the library runs on, from the load of the
// code object to the end of the process.  Its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and kept;
// host code never uses the array's name as an address, only that pointer.
// Nothing here allocates or frees memory.  Every call on a GPU shares that
// GPU's array: calls that overlap in time on one GPU (other streams, other
// threads) race on it.  No kernel of the layer needs its workspace cleared
// (every byte it reads there was written earlier in the same call), so the
// array's contents from earlier calls never matter.
#include <hip/hip_runtime.h>

#include <mutex>

#include "q4linear.h"

static __device__ __align__(256) unsigned char scratch[Q4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The device address of the current device's array (looked up on its first
// use on that device).
q4_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q4_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return Q4_OK;
}

}  // namespace

extern "C" q4_status q4_linear_noalloc(const float* x, int64_t ldx, const uint8_t* qw,
                                       int64_t ldq, const float* scales, int64_t lds,
                                       int64_t group_size, const float* bias, float* out,
                                       int64_t ldo, int64_t M, int64_t N, int64_t K,
                                       int32_t nibble_order, int32_t math, void* stream,
                                       int32_t* path_out) {
  if (path_out) *path_out = Q4_PATH_NONE;
  // Invalid sizes need no workspace here; q4_linear then reports them.
  const size_t need = q4_linear_workspace_bytes(M, N, K, group_size, math);
  void* ws = nullptr;
  if (need > 0) {
    if (need > (size_t)Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_WORKSPACE;
    const q4_status st = scratch_on_current_device(&ws);
    if (st != Q4_OK) return st;
  }
  // q4_linear checks every argument before it queues anything, and checks
  // the workspace against the plan's need
  return q4_linear(x, ldx, qw, ldq, scales, lds, group_size, bias, out, ldo, M, N, K,
                   nibble_order, math, ws, need > 0 ? (size_t)Q4_NOALLOC_SCRATCH_BYTES : 0,
                   stream, path_out);
}
