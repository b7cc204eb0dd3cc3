// Top-k lists for the indexed path, built on the device.
//
// Problem (DeepSeek-V4 CSA/HCA article, §2.3 and §3.3): a query's list is its
// sliding-window indices followed by its compressed-region indices, as
// absolute rows of a cache laid out as [window ring | compressed rows];
// position p lives in ring slot p % window, and compressed row c exists once
// position (c + 1) * ratio - 1 has been seen.  Unused entries are -1.
//
// The lists are pure integer functions of (position, entry), so the kernels are
// store streams.  Lists of at least 256 entries with 16-byte aligned rows: one
// wave per piece of a list (up to 4 KB) works out the list's window start, ring
// slot and number of visible compressed rows once, then each lane writes 16-byte
// chunks with a compare and a select per entry; many small pieces keep enough
// stores in flight.  Other shapes: one thread per four
// consecutive entries of one list.
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

// One wave per piece of kPiece 16-byte chunks of a list (K % 4 == 0, 16-byte aligned rows).
constexpr int kPiece = 256;
__global__ __launch_bounds__(256) void build_topk_idxs_rows(BuildIdxParams a) {
  const int W = a.window;
  const int K = W + a.n_comp;
  const int per_row = K / 4;
  const int pieces = (per_row + kPiece - 1) / kPiece;
  const int64_t items = static_cast<int64_t>(a.batch) * a.q_len * pieces;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = static_cast<int>(threadIdx.x & 63);
  for (int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + wave; w < items; w += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t r = w / pieces;
    const int ch0 = static_cast<int>(w - r * pieces) * kPiece;
    const int ch1 = per_row < ch0 + kPiece ? per_row : ch0 + kPiece;
    const int64_t b = r / a.q_len;
    const int64_t p = static_cast<int64_t>(a.start_pos[b]) + (r - b * a.q_len);
    // Window part: entry k is position q0 + k, listed (as ring slot (q0 + k) % W) while q0 + k <= p,
    // that is for k < nw.  Compressed part: row c is visible once (c + 1) ratio - 1 <= p, that is
    // for c < (p + 1) / ratio.
    const int64_t q0 = p - W + 1 > 0 ? p - W + 1 : 0;
    const int nw = p < 0 ? 0 : static_cast<int>(p + 1 < W ? p + 1 : W);
    const int s0 = W > 0 ? static_cast<int>(q0 % W) : 0;
    const int64_t vis = a.ratio > 0 && p >= 0 ? (p + 1) / a.ratio : 0;
    const int nc = static_cast<int>(vis < a.n_comp ? vis : a.n_comp);
    int32_t *dst = a.out + r * K;
    for (int ch = ch0 + lane; ch < ch1; ch += 64) {
      i32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * ch + j;
        if (k < W) {
          const int slot = s0 + k >= W ? s0 + k - W : s0 + k;
          v[j] = k < nw ? slot : -1;
        } else {
          v[j] = k - W < nc ? k : -1;  // row W + c of the cache is entry W + c
        }
      }
      *reinterpret_cast<i32x4 *>(dst + 4 * ch) = v;
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
  const bool vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15u) == 0;
  if (vec && K >= 256) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.q_len * ((K / 4 + kPiece - 1) / kPiece);
    const int64_t wgs = std::min<int64_t>((items + 3) / 4, static_cast<int64_t>(cus) * 1024);  // ~one piece per wave
    if (trace_on())
      trace("build_topk_idxs_rows grid=%lld block=256 pieces=%lld lists=%lld entries=%d", static_cast<long long>(wgs),
            static_cast<long long>(items), static_cast<long long>(a.batch) * a.q_len, K);
    hipLaunchKernelGGL(build_topk_idxs_rows, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, static_cast<int64_t>(cus) * 16);
  if (trace_on())
    trace("build_topk_idxs_kernel<vec=%d> grid=%lld block=256 lists=%lld entries=%d", vec ? 1 : 0,
          static_cast<long long>(blocks), static_cast<long long>(a.batch) * a.q_len, K);
  if (vec)
    hipLaunchKernelGGL(build_topk_idxs_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(build_topk_idxs_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sattn
