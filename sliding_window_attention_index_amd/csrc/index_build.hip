// Top-k lists for the indexed path, built on the device.
//
// Problem (DeepSeek-V4 CSA/HCA article, §2.3 and §3.3): a query's list is its
// sliding-window indices followed by its compressed-region indices, as
// absolute rows of a cache laid out as [window ring | compressed rows];
// position p lives in ring slot p % window, and compressed row c exists once
// position (c + 1) * ratio - 1 has been seen.  Unused entries are -1.
//
// The lists are pure integer functions of (position, entry), so the kernel is
// a store stream: one thread writes four consecutive entries of one list
// (one 16-byte store when rows allow it), HBM-write bound.
#include <algorithm>

#include "sattn_device.hpp"
#include "sattn_kernels.hpp"

namespace sattn {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;

__device__ __forceinline__ int entry(int64_t p, int k, const BuildIdxParams &a) {
  if (k < a.window) {
    const int64_t q = (p - a.window + 1 > 0 ? p - a.window + 1 : 0) + k;  // k-th position of the window
    return (p >= 0 && q <= p) ? static_cast<int>(q % a.window) : -1;
  }
  const int64_t c = k - a.window;  // compressed row c
  return (a.ratio > 0 && (c + 1) * a.ratio - 1 <= p) ? static_cast<int>(a.window + c) : -1;
}

template <bool kVec>
__global__ __launch_bounds__(256) void build_topk_idxs_kernel(BuildIdxParams a) {
  const int K = a.window + a.n_comp;
  const int64_t per_row = (K + 3) / 4;
  const int64_t total = static_cast<int64_t>(a.batch) * a.q_len * per_row;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / per_row;  // query row b * q_len + t
    const int k0 = static_cast<int>(i - r * per_row) * 4;
    const int64_t b = r / a.q_len;
    const int64_t p = static_cast<int64_t>(a.start_pos[b]) + (r - b * a.q_len);
    int32_t *dst = a.out + r * K + k0;
    if constexpr (kVec) {
      const i32x4 v = {entry(p, k0, a), entry(p, k0 + 1, a), entry(p, k0 + 2, a), entry(p, k0 + 3, a)};
      *reinterpret_cast<i32x4 *>(dst) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k0 + j < K) dst[j] = entry(p, k0 + j, a);
    }
  }
}

}  // namespace

hipError_t launch_build_topk_idxs(const BuildIdxParams &a, hipStream_t stream) {
  const int K = a.window + a.n_comp;
  const int64_t total = static_cast<int64_t>(a.batch) * a.q_len * ((K + 3) / 4);
  if (total == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, static_cast<int64_t>(cus) * 16);
  const bool vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15u) == 0;
  if (vec)
    hipLaunchKernelGGL(build_topk_idxs_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(build_topk_idxs_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sattn
