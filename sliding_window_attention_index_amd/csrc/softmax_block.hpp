// Online-softmax step on one 32-key block held in the accumulator of
// S^T = K . Q^T (v_mfma_f32_32x32x16_bf16), shared by the MFMA kernels.
//
// Layout: lane (n, h) of the wave holds 16 logits of row n (one query-head
// row); element r is block position 8*(r/4) + 4h + r%4.  The other 16 keys
// of the row are in lane n + 32*(1-h).
//
// Update (DeepSeek-V4 article §4.3: running max, rescale factor
// exp(old_max - new_max), running sum, rescaled accumulator), carried in
// base 2 with the softmax scale folded into one FMA before the exponential.
// The running max is kept in raw logit units (scale > 0 keeps the order).
// The accumulator is rescaled only when the max grows by more than 2^8 in
// probability terms; otherwise probabilities are taken against the stale max
// (they stay <= 256), which cancels exactly in acc / l.
// The denominator sums the fp32 probabilities (the bf16-rounded copies feed
// only the PV product), which keeps the log-sum-exp at fp32 accuracy.
#pragma once

#include "sattn_device.hpp"

namespace sattn {

constexpr float kRescaleLog2 = 8.0f;

struct RowSoftmax {
  float m;  // running max, raw logit units (-inf: nothing seen)
  float l;  // this lane's share of the denominator (the lane pair sums to l)
};

// Bitmask of valid block positions [lo, hi] (relative to the block start), clipped to 0..31.
__device__ __forceinline__ uint32_t range_bits(int lo, int hi) {
  const uint32_t upto = hi >= 31 ? 0xffffffffu : (hi < 0 ? 0u : (2u << hi) - 1u);
  const uint32_t from = lo <= 0 ? 0xffffffffu : (lo > 31 ? 0u : ~((1u << lo) - 1u));
  return upto & from;
}

// Set logits whose block position bit is clear to -inf.  `bits` is the
// 32-bit validity mask of the block; h selects this lane's key quads.
__device__ __forceinline__ void mask_block(f32x16 &st, uint32_t bits, int h) {
  const uint32_t bh = bits >> (4 * h);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = 8 * (r >> 2) + (r & 3);
    const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(bh), pos, 1));
    st[r] = __uint_as_float((keep & __float_as_uint(st[r])) | (~keep & 0xff800000u));
  }
}

// Add `bias` (raw units) to the logits whose block position bit is set.
__device__ __forceinline__ void bias_block(f32x16 &st, uint32_t bits, int h, float bias) {
  const uint32_t bh = bits >> (4 * h);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = 8 * (r >> 2) + (r & 3);
    if ((bh >> pos) & 1u) st[r] += bias;
  }
}

__device__ __forceinline__ float block_max(const f32x16 &st) {
  float a = fmaxf(st[0], st[1]);
  float b = fmaxf(st[2], st[3]);
#pragma unroll
  for (int r = 4; r < 16; r += 2) {
    a = fmaxf(a, st[r]);
    b = fmaxf(b, st[r + 1]);
  }
  return halves_max(fmaxf(a, b));
}

// Returns true (wave-uniform) if the accumulators must be rescaled by `alpha`
// before this block's probabilities are accumulated; updates rs.m then.
__device__ __forceinline__ bool softmax_need_rescale(RowSoftmax &rs, float bm, float c, float &alpha) {
  const float m_new = fmaxf(rs.m, bm);
  const bool grow = (m_new - rs.m) * c > kRescaleLog2;  // -inf old max always grows when m_new is finite
  if (__ballot(grow)) {
    // Old -inf -> 0.  A row that has still seen nothing (old and new max both -inf) keeps its
    // state: its l and accumulator are 0 (or l = 1 for a null sink of -inf), and -inf - -inf
    // would make the factor NaN.  Rows of one wave reach their first key at different blocks.
    alpha = m_new == kNegInf ? 1.0f : fast_exp2((rs.m - m_new) * c);
    rs.l *= alpha;
    rs.m = m_new;
    return true;
  }
  alpha = 1.0f;
  return false;
}

// Probabilities of the block against the running max, packed as the two
// bf16x8 B operands of the PV product (keys of MFMA step t are elements
// 8t..8t+7), and their sum added to rs.l.
__device__ __forceinline__ void softmax_probs(const f32x16 &st, RowSoftmax &rs, float c, bf16x8 (&pb)[2]) {
  const float mc = rs.m == kNegInf ? 0.0f : rs.m * c;
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float e0 = fast_exp2(fmaf(st[8 * t + j], c, -mc));
      const float e1 = fast_exp2(fmaf(st[8 * t + j + 1], c, -mc));
      l0 += e0;
      l1 += e1;
      pb[t][j] = static_cast<__bf16>(e0);
      pb[t][j + 1] = static_cast<__bf16>(e1);
    }
  }
  rs.l += l0 + l1;
}

}  // namespace sattn
