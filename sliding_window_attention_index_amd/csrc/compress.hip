// Gated pooling of the compressor (DeepSeek-V4 CSA/HCA article, §5.1): each compressed row is
// the sum over a window's entries of kv times softmax(score + ape), the softmax taken over the
// window's entries separately for every feature.  Without overlap a window is its `ratio`
// tokens; with overlap (kv and score carry 2 d features per token) window w also takes the
// previous window's tokens with their first d features, its own tokens contributing their last
// d features (the article's overlap transform); window 0 has no previous window.
//
// Memory-bound: every projected feature of every token is read once.  One thread per (batch,
// window, 8 features): the 16 threads of a 128-wide row read 16-byte runs of each token row,
// and the softmax runs online over the entries in fp32 (running max, rescaled sum and weighted
// sum), so every entry is loaded once.  For the usual ratios (1, 2, 4, and 8 in bf16) all
// loads of a window are in flight together.
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"

namespace sattn {
namespace {

template <typename T>
__device__ __forceinline__ void store8(T *p, const float v[8]);
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16 *p, const float v[8]) {
  const bf16x8 w = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                    static_cast<__bf16>(v[3]), static_cast<__bf16>(v[4]), static_cast<__bf16>(v[5]),
                    static_cast<__bf16>(v[6]), static_cast<__bf16>(v[7])};
  *reinterpret_cast<bf16x8 *>(p) = w;
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float v[8]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Eight consecutive elements as loaded (16 bytes of bf16, 32 bytes of fp32), widened at use.
template <typename T>
struct Raw8;
template <>
struct Raw8<__bf16> {
  u32x4 w;
  __device__ __forceinline__ void load(const __bf16 *p) { w = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ void unpack(float out[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const f32x4 *>(p);
    b = *reinterpret_cast<const f32x4 *>(p + 4);
  }
  __device__ __forceinline__ void unpack(float out[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  }
};

// Online softmax state of 8 features over a window's entries.
struct Pool8 {
  float m[8], l[8], acc[8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m[e] = kNegInf;
      l[e] = 0.0f;
      acc[e] = 0.0f;
    }
  }
  // One entry: scores s + a (natural units), values v.
  __device__ __forceinline__ void add(const float s[8], const float a[8], const float v[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (s[e] + a[e]) * kLog2e;
      const float m_new = fmaxf(m[e], x);
      const float r = fast_exp2(m[e] - m_new);  // 0 on the first entry (m = -inf)
      const float q = fast_exp2(x - m_new);
      l[e] = l[e] * r + q;
      acc[e] = acc[e] * r + q * v[e];
      m[e] = m_new;
    }
  }
};

// R > 0: the window length is a compile-time constant and every load of a window is issued
// before any is used (the latency of one round trip per window instead of one per token).
// R == 0: any ratio, one token at a time.
template <typename T, int R>
__global__ __launch_bounds__(256) void compress_pool_kernel(CompressParams p) {
  const int d = p.head_dim;
  const int g8 = d / 8;
  const int ratio = R > 0 ? R : p.ratio;
  const int n_out = p.seq_len / ratio;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= static_cast<int64_t>(p.batch) * n_out * g8) return;
  const int f0 = static_cast<int>(gid % g8) * 8;
  const int64_t bw = gid / g8;
  const int w = static_cast<int>(bw % n_out);
  const int64_t b = bw / n_out;
  const int coff = p.overlap ? 2 : 1;
  const int64_t tok = static_cast<int64_t>(coff) * d;  // elements between tokens
  const T *kv = static_cast<const T *>(p.kv) + b * p.seq_len * tok;
  const T *sc = static_cast<const T *>(p.score) + b * p.seq_len * tok;
  const T *ape = static_cast<const T *>(p.ape);
  const int lo = p.overlap ? d : 0;  // feature offset of a window's own tokens
  const bool prev = p.overlap && w > 0;

  Pool8 pool;
  pool.init();
  if constexpr (R > 0) {
    // entries 0 .. R-1: previous window (first half), R .. 2R-1: own tokens; the raw 8-element
    // runs of score and kv stay packed until used (ape is tiny and read at use).
    Raw8<T> s[2 * R], v[2 * R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t t = static_cast<int64_t>(w) * R + i;
      s[R + i].load(sc + t * tok + lo + f0);
      v[R + i].load(kv + t * tok + lo + f0);
      if (prev) {
        s[i].load(sc + (t - R) * tok + f0);
        v[i].load(kv + (t - R) * tok + f0);
      }
    }
    float sf[8], vf[8], af[8];
    if (prev) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        s[i].unpack(sf);
        v[i].unpack(vf);
        load8(ape + static_cast<int64_t>(i) * tok + f0, af);
        pool.add(sf, af, vf);
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      s[R + i].unpack(sf);
      v[R + i].unpack(vf);
      load8(ape + static_cast<int64_t>(i) * tok + lo + f0, af);
      pool.add(sf, af, vf);
    }
  } else {
    float s[8], v[8], a[8];
    if (prev) {
      for (int i = 0; i < ratio; ++i) {
        const int64_t t = static_cast<int64_t>(w - 1) * ratio + i;
        load8(sc + t * tok + f0, s);
        load8(kv + t * tok + f0, v);
        load8(ape + static_cast<int64_t>(i) * tok + f0, a);
        pool.add(s, a, v);
      }
    }
    for (int i = 0; i < ratio; ++i) {
      const int64_t t = static_cast<int64_t>(w) * ratio + i;
      load8(sc + t * tok + lo + f0, s);
      load8(kv + t * tok + lo + f0, v);
      load8(ape + static_cast<int64_t>(i) * tok + lo + f0, a);
      pool.add(s, a, v);
    }
  }
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = pool.acc[e] / pool.l[e];
  store8(static_cast<T *>(p.out) + (b * p.out_batch_stride + w) * d + f0, o);
}

template <typename T>
hipError_t launch_t(const CompressParams &p, dim3 grid, hipStream_t stream) {
  if (trace_on())
    trace("compress_pool_kernel<%s, ratio=%d> grid=%u block=256 rows=%lld head_dim=%d overlap=%d",
          sizeof(T) == 2 ? "bf16" : "fp32", p.ratio, grid.x, static_cast<long long>(p.batch) * (p.seq_len / p.ratio),
          p.head_dim, p.overlap);
  switch (p.ratio) {
    case 1: hipLaunchKernelGGL((compress_pool_kernel<T, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((compress_pool_kernel<T, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((compress_pool_kernel<T, 4>), grid, dim3(256), 0, stream, p); break;
    case 8:  // fp32 runs of eight tokens would not fit the registers: one token at a time
      if (sizeof(T) == 2) hipLaunchKernelGGL((compress_pool_kernel<T, 8>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((compress_pool_kernel<T, 0>), grid, dim3(256), 0, stream, p);
      break;
    default: hipLaunchKernelGGL((compress_pool_kernel<T, 0>), grid, dim3(256), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress_pool(const CompressParams &p, int elem_type, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(p.batch) * (p.seq_len / p.ratio) * (p.head_dim / 8);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  return elem_type == kF32 ? launch_t<float>(p, grid, stream) : launch_t<__bf16>(p, grid, stream);
}

}  // namespace sattn
