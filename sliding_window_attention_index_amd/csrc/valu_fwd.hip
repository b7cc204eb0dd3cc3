// Generic VALU kernels: any head_dim <= 256 (multiple of 8), fp32 or bf16,
// any head grouping.  One wave64 per (query token, head).
//
// The key set is walked in chunks of 64: lane j owns key j of the chunk for
// the logits (full dot product against q staged in LDS), the chunk's maximum
// and sum come from wave reductions, and for the weighted sum of values the
// lanes own output dimensions (lane, lane+64, ...) while the 64 keys'
// weights are broadcast one by one.  This is the online-softmax update of
// the DeepSeek-V4 article §4.3 (running max, rescale factor exp(old-new),
// running sum, rescaled accumulator) carried in base 2.
//
// Sinks (vLLM PR #49815 report, `_fwd_kernel` sink branch):
//   key-0 bias: sink*log2(e) is added to the logit of key 0 when present;
//   null logit: the state starts at m = sink*log2(e), l = 1.
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"

namespace sattn {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxHeadDim = 256;

// Make LDS writes of this wave visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t readlane64(int64_t x, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32), j);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

struct RowResult {
  float acc[kMaxHeadDim / 64];
  float m, l;
};

// Online softmax of one (query, head) row over a key set described by `keys`:
// keys(slot, &row_offset, &is_key0) -> valid, for slot in [0, count).
template <typename T, typename KeyFn>
__device__ __forceinline__ void attend_row(const T *__restrict__ qrow, const T *__restrict__ kmat,
                                           const T *__restrict__ vmat, int count, KeyFn keys, int D,
                                           float scale_log2, float sink2, bool key0_bias, bool null_sink,
                                           float *__restrict__ q_lds, RowResult &res) {
  const int lane = lane_id();
  for (int d = lane; d < D; d += 64) q_lds[d] = load_elem(qrow + d);
  wave_lds_sync();

  const int nc = (D + 63) / 64;
  res.m = null_sink ? sink2 : kNegInf;
  res.l = null_sink ? 1.0f : 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxHeadDim / 64; ++c) res.acc[c] = 0.0f;

  for (int base = 0; base < count; base += 64) {
    const int slot = base + lane;
    int64_t roff = 0;
    bool is0 = false;
    const bool valid = slot < count && keys(slot, roff, is0);
    float s = kNegInf;
    if (valid) {
      const T *krow = kmat + roff;
      float dot = 0.0f;
      for (int d = 0; d < D; d += 8) {
        float kk[8];
        load8(krow + d, kk);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf(q_lds[d + i], kk[i], dot);
      }
      s = dot * scale_log2;
      if (key0_bias && is0) s += sink2;
    }
    const float m_new = fmaxf(res.m, wave_max(s));
    if (m_new == kNegInf) continue;  // nothing attended yet (wave-uniform)
    const float alpha = fast_exp2(res.m - m_new);
    const float p = valid ? fast_exp2(s - m_new) : 0.0f;
    res.l = res.l * alpha + wave_sum(p);
#pragma unroll
    for (int c = 0; c < kMaxHeadDim / 64; ++c) res.acc[c] *= alpha;
    const int nk = min(64, count - base);
    for (int j = 0; j < nk; ++j) {
      const float pj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p), j));
      if (pj == 0.0f) continue;  // masked or underflowed key: no contribution
      const int64_t rj = readlane64(roff, j);
      const T *vrow = vmat + rj;
#pragma unroll
      for (int c = 0; c < kMaxHeadDim / 64; ++c) {
        const int d = lane + 64 * c;
        if (c < nc && d < D) res.acc[c] = fmaf(pj, load_elem(vrow + d), res.acc[c]);
      }
    }
    res.m = m_new;
  }
}

template <typename T>
__device__ __forceinline__ void write_row(const RowResult &r, int D, T *__restrict__ orow, float *lse_slot) {
  const int lane = lane_id();
  const float inv = r.l > 0.0f ? 1.0f / r.l : 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxHeadDim / 64; ++c) {
    const int d = lane + 64 * c;
    if (d < D) store_elem(orow + d, r.acc[c] * inv);
  }
  if (lse_slot && lane == 0) *lse_slot = r.l > 0.0f ? (r.m + log2f(r.l)) * kLn2 : kNegInf;
}

template <typename T>
__global__ __launch_bounds__(64 * kWavesPerBlock) void window_fwd_valu(WindowParams p) {
  __shared__ float q_lds[kWavesPerBlock][kMaxHeadDim];
  const int wave = threadIdx.x >> 6;
  const int seq = blockIdx.y;
  const int h = blockIdx.z;
  const int a = p.cu_seqlens[seq];
  const int L = p.cu_seqlens[seq + 1] - a;
  const int i = blockIdx.x * kWavesPerBlock + wave;
  if (i >= L) return;
  const int D = p.head_dim, Hkv = p.num_kv_heads, g = h / p.group;
  int lo = p.window_left < 0 ? 0 : max(0, i - p.window_left);
  int hi = p.window_right < 0 ? L - 1 : min(L - 1, i + p.window_right);
  const int count = max(0, hi - lo + 1);
  const T *q = static_cast<const T *>(p.q);
  const T *k = static_cast<const T *>(p.k);
  const T *v = static_cast<const T *>(p.v);
  auto keys = [&](int slot, int64_t &roff, bool &is0) {
    const int j = lo + slot;
    roff = (static_cast<int64_t>(a + j) * Hkv + g) * D;
    is0 = j == 0;
    return true;
  };
  const float sink2 = p.sink_mode != kSinkNone ? p.sinks[h] * kLog2e : 0.0f;
  RowResult r;
  const int64_t qoff = (static_cast<int64_t>(a + i) * p.num_heads + h) * D;
  attend_row<T>(q + qoff, k, v, count, keys, D, p.scale_log2, sink2, p.sink_mode == kSinkKey0,
                p.sink_mode == kSinkNull, q_lds[wave], r);
  write_row<T>(r, D, static_cast<T *>(p.o) + qoff,
               p.lse ? p.lse + static_cast<int64_t>(a + i) * p.num_heads + h : nullptr);
}

template <typename T>
__global__ __launch_bounds__(64 * kWavesPerBlock) void indexed_fwd_valu(IndexedParams p) {
  __shared__ float q_lds[kWavesPerBlock][kMaxHeadDim];
  const int wave = threadIdx.x >> 6;
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const int64_t bt = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (bt >= BM) return;
  const int h = blockIdx.y;
  const int part = blockIdx.z;
  const int D = p.head_dim, N = p.kv_len, K = p.topk;
  const int64_t b = bt / p.q_len;
  const int kb = part * p.part_len;
  const int count = max(0, min(K, kb + p.part_len) - kb);
  const int32_t *list = p.idx + bt * K + kb;
  auto keys = [&](int slot, int64_t &roff, bool &is0) {
    const int x = list[slot];
    roff = (b * N + x) * static_cast<int64_t>(D);
    is0 = x == 0;
    return x >= 0 && x < N;
  };
  const bool partial = p.num_parts > 1;
  const float sink2 = p.sink_mode != kSinkNone ? p.sinks[h] * kLog2e : 0.0f;
  const T *kvp = static_cast<const T *>(p.kv);
  RowResult r;
  const int64_t qoff = (bt * p.num_heads + h) * D;
  attend_row<T>(static_cast<const T *>(p.q) + qoff, kvp, kvp, count, keys, D, p.scale_log2, sink2,
                p.sink_mode == kSinkKey0, !partial && p.sink_mode == kSinkNull, q_lds[wave], r);
  if (partial) {
    const int64_t row = (static_cast<int64_t>(part) * BM + bt) * p.num_heads + h;
    write_row<float>(r, D, p.part_o + row * D, p.part_lse + row);
  } else {
    write_row<T>(r, D, static_cast<T *>(p.o) + qoff, p.lse ? p.lse + bt * p.num_heads + h : nullptr);
  }
}

// Attention mass per block of list entries, normalised by a given log-sum-exp (nano-vllm XAttention
// offload note, technical details: the third stage normalises with the merged global statistics and
// sums per block).  Generic shapes: one wave per (query, head); for block c the lanes take 64 of
// its entries at a time, a valid entry contributes exp2(s - lse * log2(e)) with s its logit in base
// 2 (key-0 bias included), and a wave sum gives the block's mass.  Every block is written.
template <typename T>
__global__ __launch_bounds__(64 * kWavesPerBlock) void block_mass_valu(IndexedParams p) {
  __shared__ float q_lds[kWavesPerBlock][kMaxHeadDim];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const int64_t bt = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (bt >= BM) return;
  const int h = blockIdx.y;
  const int D = p.head_dim, N = p.kv_len, K = p.topk, bk = p.block_keys;
  const int64_t b = bt / p.q_len;
  const int64_t rh = bt * p.num_heads + h;
  const T *qrow = static_cast<const T *>(p.q) + rh * D;
  float *ql = q_lds[wave];
  for (int d = lane; d < D; d += 64) ql[d] = load_elem(qrow + d);
  wave_lds_sync();
  const int32_t *list = p.idx + bt * K;
  const T *kvb = static_cast<const T *>(p.kv) + b * static_cast<int64_t>(N) * D;
  const float lse2 = p.lse_in[rh] * kLog2e;
  const float bias2 = p.sink_mode == kSinkKey0 ? p.sinks[h] * kLog2e : 0.0f;
  float *out = p.mass + rh * p.n_bins;
  for (int c = 0; c < p.n_bins; ++c) {
    const int lo = c * bk, hi = min(K, lo + bk);
    float part = 0.0f;
    for (int base = lo; base < hi; base += 64) {
      const int slot = base + lane;
      const int x = slot < hi ? list[slot] : -1;
      if (x >= 0 && x < N) {
        const T *krow = kvb + static_cast<int64_t>(x) * D;
        float dot = 0.0f;
        for (int d = 0; d < D; d += 8) {
          float kk[8];
          load8(krow + d, kk);
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = fmaf(ql[d + i], kk[i], dot);
        }
        float s = dot * p.scale_log2;
        if (x == 0) s += bias2;
        part += fast_exp2(s - lse2);
      }
    }
    const float tot = wave_sum(part);
    if (lane == 0) out[c] = tot;
  }
}

// Merge of per-chunk partial results: M = max(lse_c, sink), W = sum exp(lse_c - M) [+ exp(sink - M)].
// One thread per (row, head, 4 consecutive dims): the parts' log-sum-exps first (maximum, then
// weights), then every part's 16-byte slice of o in flight together.  [P3] technical details:
// per-chunk softmax statistics combined into global ones; the null sink enters the denominator
// once.
template <typename T>
__global__ __launch_bounds__(256) void merge4_kernel(MergeParams p) {
  const int D4 = p.head_dim / 4;
  const int64_t RH = static_cast<int64_t>(p.rows) * p.num_heads;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= RH * D4) return;
  const int64_t rh = gid / D4;
  const int q = static_cast<int>(gid - rh * D4);
  const int hh = static_cast<int>(rh % p.num_heads);
  const int S = p.num_parts;
  const bool null_sink = p.sink_mode == kSinkNull;
  T *orow = static_cast<T *>(p.o) + rh * p.head_dim + 4 * q;
  const float *o4 = p.part_o + rh * p.head_dim + 4 * q;
  // One pass, eight parts at a time: every load of a group is issued before any is used, and the
  // running (M, W, acc) is rescaled when a group raises the maximum.
  float M = null_sink ? p.sinks[hh] : kNegInf;
  float W = null_sink ? 1.0f : 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kG = 8;
  for (int c0 = 0; c0 < S; c0 += kG) {
    float lv[kG];
    f32x4 ov[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int c = min(c0 + j, S - 1);  // a clamped duplicate is given weight 0 below
      lv[j] = c0 + j < S ? p.part_lse[c * RH + rh] : kNegInf;
      ov[j] = *reinterpret_cast<const f32x4 *>(o4 + c * RH * p.head_dim);
    }
    float gm = lv[0];
#pragma unroll
    for (int j = 1; j < kG; ++j) gm = fmaxf(gm, lv[j]);
    if (gm > M) {  // new maximum: rescale what has been summed
      const float r = M == kNegInf ? 0.0f : expf(M - gm);
      W *= r;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= r;
      M = gm;
    }
    if (M == kNegInf) continue;
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const float w = expf(lv[j] - M);  // 0 for an empty part (lse = -inf)
      W += w;
      if (w > 0.0f) {  // an empty part contributes nothing, whatever its o holds
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, ov[j][e], acc[e]);
      }
    }
  }
  if (M == kNegInf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_elem(orow + e, 0.0f);
    if (p.lse && q == 0) p.lse[rh] = kNegInf;
    return;
  }
  const float inv = 1.0f / W;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_elem(orow + e, acc[e] * inv);
  if (p.lse && q == 0) p.lse[rh] = M + logf(W);
}

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t RH = static_cast<int64_t>(p.rows) * p.num_heads;
  const int64_t rh = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (rh >= RH) return;
  const int h = static_cast<int>(rh % p.num_heads);
  const int D = p.head_dim;
  const bool null_sink = p.sink_mode == kSinkNull;
  float M = kNegInf;
  for (int c = 0; c < p.num_parts; ++c) M = fmaxf(M, p.part_lse[c * RH + rh]);
  const float sink = null_sink ? p.sinks[h] : kNegInf;
  M = fmaxf(M, sink);
  T *orow = static_cast<T *>(p.o) + rh * D;
  if (M == kNegInf) {
    for (int d = lane; d < D; d += 64) store_elem(orow + d, 0.0f);
    if (p.lse && lane == 0) p.lse[rh] = kNegInf;
    return;
  }
  float acc[kMaxHeadDim / 64] = {};
  float W = 0.0f;
  for (int c = 0; c < p.num_parts; ++c) {
    const float w = expf(p.part_lse[c * RH + rh] - M);
    if (w == 0.0f) continue;
    W += w;
    const float *oc = p.part_o + (c * RH + rh) * D;
#pragma unroll
    for (int j = 0; j < kMaxHeadDim / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < D) acc[j] = fmaf(w, oc[d], acc[j]);
    }
  }
  if (null_sink) W += expf(sink - M);
  const float inv = 1.0f / W;
#pragma unroll
  for (int j = 0; j < kMaxHeadDim / 64; ++j) {
    const int d = lane + 64 * j;
    if (d < D) store_elem(orow + d, acc[j] * inv);
  }
  if (p.lse && lane == 0) p.lse[rh] = M + logf(W);
}

}  // namespace

hipError_t launch_window_valu(const WindowParams &p, int elem_type, hipStream_t stream) {
  const dim3 grid((p.max_seqlen + kWavesPerBlock - 1) / kWavesPerBlock, p.num_seqs, p.num_heads);
  if (trace_on())
    trace("window_fwd_valu<%s> grid=%ux%ux%u block=%d head_dim=%d group=%d window=(%d, %d) sink_mode=%d",
          elem_type == kF32 ? "fp32" : "bf16", grid.x, grid.y, grid.z, 64 * kWavesPerBlock, p.head_dim, p.group,
          p.window_left, p.window_right, p.sink_mode);
  if (elem_type == kF32)
    hipLaunchKernelGGL(window_fwd_valu<float>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  else
    hipLaunchKernelGGL(window_fwd_valu<__bf16>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_indexed_valu(const IndexedParams &p, int elem_type, hipStream_t stream) {
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const dim3 grid(static_cast<unsigned>((BM + kWavesPerBlock - 1) / kWavesPerBlock), p.num_heads, p.num_parts);
  if (trace_on())
    trace("indexed_fwd_valu<%s> grid=%ux%ux%u block=%d head_dim=%d slices=%d of %d entries topk=%d sink_mode=%d",
          elem_type == kF32 ? "fp32" : "bf16", grid.x, grid.y, grid.z, 64 * kWavesPerBlock, p.head_dim, p.num_parts,
          p.part_len, p.topk, p.sink_mode);
  if (elem_type == kF32)
    hipLaunchKernelGGL(indexed_fwd_valu<float>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  else
    hipLaunchKernelGGL(indexed_fwd_valu<__bf16>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_block_mass_valu(const IndexedParams &p, int elem_type, hipStream_t stream) {
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const dim3 grid(static_cast<unsigned>((BM + kWavesPerBlock - 1) / kWavesPerBlock), p.num_heads);
  if (trace_on())
    trace("block_mass_valu<%s> grid=%ux%u block=%d head_dim=%d block_keys=%d bins=%d", elem_type == kF32 ? "fp32" : "bf16",
          grid.x, grid.y, 64 * kWavesPerBlock, p.head_dim, p.block_keys, p.n_bins);
  if (elem_type == kF32)
    hipLaunchKernelGGL(block_mass_valu<float>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  else
    hipLaunchKernelGGL(block_mass_valu<__bf16>, grid, dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams &p, hipStream_t stream) {
  const int64_t RH = static_cast<int64_t>(p.rows) * p.num_heads;
  const bool vec = (reinterpret_cast<uintptr_t>(p.part_o) & 15u) == 0;  // head_dim % 8 == 0 always
  if (vec) {
    const int64_t threads = RH * (p.head_dim / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (trace_on())
      trace("merge4_kernel<%s> grid=%lld block=256 parts=%d rows=%d heads=%d head_dim=%d sink_mode=%d",
            p.out_type == kF32 ? "fp32" : "bf16", static_cast<long long>(blocks), p.num_parts, p.rows, p.num_heads,
            p.head_dim, p.sink_mode);
    if (p.out_type == kF32)
      hipLaunchKernelGGL(merge4_kernel<float>, grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(merge4_kernel<__bf16>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((RH + 3) / 4));
  if (trace_on())
    trace("merge_kernel<%s> grid=%u block=256 parts=%d rows=%d heads=%d head_dim=%d sink_mode=%d",
          p.out_type == kF32 ? "fp32" : "bf16", grid.x, p.num_parts, p.rows, p.num_heads, p.head_dim, p.sink_mode);
  if (p.out_type == kF32)
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<__bf16>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sattn
