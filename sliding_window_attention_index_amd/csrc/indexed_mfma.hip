// Top-k index-gathered attention over a single shared K=V head (bf16, MFMA).
//
// Problem (DeepSeek-V4 CSA/HCA article, §4.1-§4.4): every query has a list of
// absolute cache rows (-1 = unused); all query heads share one cache row per
// token, which is both the key and the value.  The article's kernel gathers
// a chunk of listed rows into shared memory so that both products become
// dense GEMMs, then runs the online softmax over chunks and adds the
// per-head null-logit sink to the denominator at the end.
//
// gfx950 mapping (one wave64 per task = one query, 32*HB of its heads, one
// slice of its list):
//   * S^T = KV . Q^T with v_mfma_f32_32x32x16_bf16.  The M dimension is 32
//     gathered keys, N is 32 heads, K runs over head_dim.  Lane (n, h) loads
//     head_dim/2 contiguous elements of key n's row straight from global
//     memory into the A-operand registers (the contraction order over
//     head_dim is permuted identically in A and B, so each lane reads one
//     contiguous half-row: 16-byte loads, no LDS round trip for QK).
//   * The accumulator layout of S^T puts 16 keys of one head in each lane and
//     the other 16 in lane ^ 32, so the row max / row sum need one
//     v_permlane32_swap instead of a 32-lane reduction.
//   * The same registers are written to a per-wave LDS tile, and the PV
//     product O^T = KV^T . P^T reads KV^T with ds_read_b64_tr_b16 (four keys
//     of one dimension per lane).  P^T is the S^T accumulator converted to
//     bf16 in place: the keys of MFMA step t are the accumulator registers
//     8t..8t+7, and the transposed reads fetch exactly those keys.
//   * The O^T accumulator holds one head per lane, so rescaling by the
//     per-head factor is a per-lane multiply; it is skipped unless the
//     running maximum grows by more than 2^8 (the stale maximum cancels in
//     o = acc / l, and p <= 256 stays exact enough in bf16/fp32).
//   * Gathers for block b+1 are issued before block b is computed.
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kPad = 16;  // LDS row padding (bf16 elements): keeps the transposed reads conflict-free

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

template <int D, int HB>
__global__ __launch_bounds__(256) void indexed_fwd_mfma(IndexedParams p) {
  constexpr int S = D / 16;   // MFMA steps over head_dim
  constexpr int DB = D / 32;  // 32-wide blocks of output dims
  constexpr int LDSS = D + kPad;
  __shared__ __attribute__((aligned(16))) __bf16 tiles[4][kBlockKeys * LDSS];

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int h = lane >> 5;   // half of the wave: which half of head_dim / which key quads
  const int n = lane & 31;   // key row (A operand) / head column (B operand and outputs)
  const int H = p.num_heads, N = p.kv_len, K = p.topk;
  const int n_hg = H / (32 * HB);
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (task >= BM * n_hg * p.num_parts) return;
  const int hg = static_cast<int>(task % n_hg);
  const int64_t rest = task / n_hg;
  const int64_t bt = rest % BM;
  const int part = static_cast<int>(rest / BM);
  const int64_t b = bt / p.q_len;
  const int head0 = hg * 32 * HB;
  const bool partial = p.num_parts > 1;
  const bool key0 = p.sink_mode == kSinkKey0;
  const bool null_sink = !partial && p.sink_mode == kSinkNull;

  // B operand of S^T: q[bt, head0 + 32hb + n, h*D/2 + 8s .. +8].
  bf16x8 qf[HB][S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + (bt * H + head0 + n) * D + h * (D / 2);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int s = 0; s < S; ++s) qf[hb][s] = *reinterpret_cast<const bf16x8 *>(qrow + hb * 32 * D + s * 8);
  }
  const float c = p.scale_log2;  // > 0 on this path
  float sink_raw[HB];  // sink in raw logit units (the running max is kept unscaled)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) sink_raw[hb] = p.sinks ? p.sinks[head0 + hb * 32 + n] * kLog2e / c : 0.0f;

  f32x16 acc[HB][DB];
  RowSoftmax rs[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[hb][db] = f32x16{};
    rs[hb].m = null_sink ? sink_raw[hb] : kNegInf;
    rs[hb].l = (null_sink && h == 0) ? 1.0f : 0.0f;  // the pair of lanes sharing a head splits l
  }

  const int kb = part * p.part_len;
  const int ke = min(K, kb + p.part_len);
  const int nblk = (max(0, ke - kb) + kBlockKeys - 1) / kBlockKeys;
  const int32_t *list = p.idx + bt * K;
  const __bf16 *kvb = static_cast<const __bf16 *>(p.kv) + b * static_cast<int64_t>(N) * D + h * (D / 2);
  __bf16 *tile = tiles[wave];

  bf16x8 cur[S], nxt[S];
  bool cur_valid = false, cur_zero = false, nxt_valid = false, nxt_zero = false;
  auto fetch = [&](int blk, bf16x8(&dst)[S], bool &valid, bool &is0) {
    const int slot = kb + blk * kBlockKeys + n;
    const int x = slot < ke ? list[slot] : -1;
    valid = x >= 0 && x < N;
    is0 = valid && x == 0;
    if (valid) {
      const __bf16 *row = kvb + static_cast<int64_t>(x) * D;
#pragma unroll
      for (int s = 0; s < S; ++s) dst[s] = *reinterpret_cast<const bf16x8 *>(row + s * 8);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) dst[s] = bf16x8{};
    }
  };
  if (nblk > 0) fetch(0, cur, cur_valid, cur_zero);

  const int g16 = lane >> 4, i16 = lane & 15;
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + 1 < nblk) fetch(blk + 1, nxt, nxt_valid, nxt_zero);
    const uint32_t vmask = static_cast<uint32_t>(__ballot(cur_valid));
    const uint32_t zmask = key0 ? static_cast<uint32_t>(__ballot(cur_zero)) : 0u;

    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < S; ++s) *reinterpret_cast<bf16x8 *>(tile + n * LDSS + h * (D / 2) + s * 8) = cur[s];

    if (vmask != 0u) {
      f32x16 st[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        st[hb] = f32x16{};
#pragma unroll
        for (int s = 0; s < S; ++s) st[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[s], qf[hb][s], st[hb], 0, 0, 0);
      }
      // Accumulator element r of lane (n, h) is key 8*(r/4) + 4h + r%4 of head n.
      bf16x8 pb[HB][2];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if (zmask) bias_block(st[hb], zmask, h, sink_raw[hb]);
        if (vmask != 0xffffffffu) mask_block(st[hb], vmask, h);
        float alpha;
        if (softmax_need_rescale(rs[hb], block_max(st[hb]), c, alpha)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[hb][db] *= alpha;
        }
        softmax_probs(st[hb], rs[hb], c, pb[hb]);
      }

      wave_lds_sync();
      // O^T[d][head] += KV^T[d][keys] . P^T[keys][head]; step tt covers keys 16tt..16tt+15 with
      // lane half h holding keys 16tt+4h+{0..3} and 16tt+8+4h+{0..3}.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int ka = 16 * tt + 4 * h + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = 32 * db + 16 * (g16 & 1) + (i16 & 3) * 4;
          const bf16x4 ra = lds_read_tr(tile + ka * LDSS + col);
          const bf16x4 rb = lds_read_tr(tile + (ka + 8) * LDSS + col);
          const bf16x8 a = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            acc[hb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[hb][tt], acc[hb][db], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) cur[s] = nxt[s];
    cur_valid = nxt_valid;
    cur_zero = nxt_zero;
  }

  // Epilogue: o = acc / l, lse = ln(2) * (m + log2 l).  Lane (n, h) holds dims 32db + 8i + 4h + {0..3}.
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = head0 + hb * 32 + n;
    const float l_tot = halves_sum(rs[hb].l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = l_tot > 0.0f ? (rs[hb].m * c + log2f(l_tot)) * kLn2 : kNegInf;
    if (partial) {
      const int64_t row = (static_cast<int64_t>(part) * BM + bt) * H + head;
      float *dst = p.part_o + row * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = {acc[hb][db][4 * i] * inv, acc[hb][db][4 * i + 1] * inv, acc[hb][db][4 * i + 2] * inv,
                           acc[hb][db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4 *>(dst + 32 * db + 8 * i) = v;
        }
      if (h == 0) p.part_lse[row] = lse_v;
    } else {
      __bf16 *dst = static_cast<__bf16 *>(p.o) + (bt * H + head) * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x4 v = {static_cast<__bf16>(acc[hb][db][4 * i] * inv),
                            static_cast<__bf16>(acc[hb][db][4 * i + 1] * inv),
                            static_cast<__bf16>(acc[hb][db][4 * i + 2] * inv),
                            static_cast<__bf16>(acc[hb][db][4 * i + 3] * inv)};
          *reinterpret_cast<bf16x4 *>(dst + 32 * db + 8 * i) = v;
        }
      if (p.lse && h == 0) p.lse[bt * H + head] = lse_v;
    }
  }
}

template <int D, int HB>
hipError_t launch(const IndexedParams &p, hipStream_t stream) {
  const int n_hg = p.num_heads / (32 * HB);
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * n_hg * p.num_parts;
  const int64_t blocks = (tasks + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((indexed_fwd_mfma<D, HB>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool indexed_mfma_supported(const IndexedParams &p) {
  return p.scale_log2 > 0.0f && (p.head_dim == 64 || p.head_dim == 128) && p.num_heads % 32 == 0;
}

hipError_t launch_indexed_mfma(const IndexedParams &p, hipStream_t stream) {
  const bool hb2 = p.num_heads % 64 == 0;
  if (p.head_dim == 128) return hb2 ? launch<128, 2>(p, stream) : launch<128, 1>(p, stream);
  return hb2 ? launch<64, 2>(p, stream) : launch<64, 1>(p, stream);
}

}  // namespace sattn
