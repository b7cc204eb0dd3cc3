// sattn_indexed_fwd_noalloc: the indexed call for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The split-K partials go to `scratch`, a fixed file-scope device array that every GPU the
// library runs on holds until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with hipGetSymbolAddress
// (the device current at the first call) and only that address is ever handed to a kernel.
// Everything else (validation, kernels, merge) is sattn_indexed_fwd's.
//
// Nothing in the scratch has to start at any value: each call writes every partial it reads.
// Calls that overlap on one GPU share its scratch and race; calls ordered on one stream do not.
#include <mutex>

#include "sattn.h"
#include "sattn_kernels.hpp"

namespace {

constexpr size_t kScratchBytes = SATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void *ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// Device address of this device's copy of `scratch`, looked up at the first call on the device.
void *scratch_on_current_device(hipStream_t stream, sattn_status *st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    *st = SATTN_ERR_LAUNCH;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = SATTN_ERR_UNSUPPORTED;
    return nullptr;
  }
  // The scratch address is the current device's: a stream of another device would hand its
  // kernels an address that is not theirs.
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) {
      *st = SATTN_ERR_UNSUPPORTED;
      return nullptr;
    }
  }
  DeviceScratch &d = g_scratch[dev];
  std::call_once(d.once, [&d]() { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
  if (d.err != hipSuccess || d.ptr == nullptr) {
    *st = SATTN_ERR_LAUNCH;
    return nullptr;
  }
  *st = SATTN_OK;
  return d.ptr;
}

}  // namespace

extern "C" sattn_status sattn_indexed_fwd_noalloc(const sattn_indexed_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (a->num_splits > 1 && a->batch > 0 && a->q_len > 0 && a->num_heads > 0 && a->head_dim > 0 &&
      sattn_indexed_workspace_size(a->batch, a->q_len, a->num_heads, a->head_dim, a->num_splits) > kScratchBytes)
    return SATTN_ERR_SCRATCH_LIMIT;  // before the device is touched
  if (a->num_splits <= 1) return sattn::indexed_fwd_with_workspace(a, nullptr, 0, stream);
  sattn_status st;
  void *ws = scratch_on_current_device(stream, &st);
  if (!ws) return st;
  return sattn::indexed_fwd_with_workspace(a, ws, kScratchBytes, stream);
}
