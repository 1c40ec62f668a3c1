// tile_gather_backward for callers that cannot allocate device memory.
//
// The grouped execution of the gather backward needs scratch memory (segment
// offsets, term lists, count tables).  tile_gather_backward takes it from the
// caller as a workspace; this entry point takes it from `scratch`, a static
// device array of the library, so a caller under stream capture, in a tight
// serving loop or in a harness that forbids hipMalloc passes only its inputs
// and outputs.  Every GPU the library runs on holds its own copy of the array
// (STG_STATIC_SCRATCH_BYTES) from the moment the array is first looked up on
// it until the process ends.  All calls on one GPU share that copy, and the
// kernels initialise every part of it they read, so nothing from an earlier
// call leaks into a later one; calls that overlap in time on one GPU (on
// different streams, or from different host threads without ordering) race
// on it.
//
// Host code never passes `scratch` itself: in host code that name is a
// host-side shadow, not a device address.  The device address comes from
// hipGetSymbolAddress, once per device, with that device current.
#include <atomic>
#include <mutex>

#include "stg_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[STG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// device address of `scratch` on the current device
int scratch_address(const char* name, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return stg::fail(STG_ERR_LAUNCH, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return stg::fail(STG_ERR_UNSUPPORTED, "%s: device %d out of range", name, dev);
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return stg::fail(STG_ERR_LAUNCH, "%s: no device address for the static scratch array: %s", name,
                         hipGetErrorString(e));
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return STG_OK;
}

}  // namespace

extern "C" int tile_gather_backward_static(const stg_tensor* a_grad, const int32_t* indices, int64_t n_indices,
                                           const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                                           const stg_tensor* grad_out, void* stream) {
  stg::clear_error();
  const char* name = "tile_gather_backward_static";
  const int64_t need = tile_gather_backward_workspace(a_grad, n_indices, tile_shape, axis);
  if (need < 0) return (int)-need;
  if (need > STG_STATIC_SCRATCH_BYTES)
    return stg::fail(STG_ERR_RANGE, "%s: %lld bytes of scratch needed, the static array holds %lld", name,
                     (long long)need, (long long)STG_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    // the array looked up is the current device's: a stream of another
    // device would run the kernels against an address that is not theirs
    if (stream) {
      int cur = -1, sdev = -1;
      hipError_t e = hipGetDevice(&cur);
      if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
      if (e != hipSuccess) return stg::fail(STG_ERR_LAUNCH, "%s: stream device: %s", name, hipGetErrorString(e));
      if (sdev != cur)
        return stg::fail(STG_ERR_INVALID, "%s: the stream is on device %d, the current device is %d", name, sdev, cur);
    }
    const int rc = scratch_address(name, &ws);
    if (rc) return rc;
  }
  return tile_gather_backward(a_grad, indices, n_indices, tile_shape, offset, axis, grad_out, ws,
                              need > 0 ? STG_STATIC_SCRATCH_BYTES : 0, stream);
}
