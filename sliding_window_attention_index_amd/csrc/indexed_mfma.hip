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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_list_rsrc(const int32_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

template <int D>
__global__ __launch_bounds__(256) void indexed_fwd_mfma(IndexedParams p) {
  constexpr int S = D / 16;   // MFMA steps over head_dim
  constexpr int DB = D / 32;  // 32-wide blocks of output dims
  constexpr int LDSS = D + kPad;
  __shared__ __attribute__((aligned(16))) __bf16 tiles[4][kBlockKeys * LDSS];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5;   // half of the wave: which half of head_dim / which key quads
  const int n = lane & 31;   // key row (A operand) / head column (B operand and outputs)
  const int H = p.num_heads, N = p.kv_len, K = p.topk;
  const int n_hg = H / 32;
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (task >= BM * n_hg * p.num_parts) return;
  const int hg = static_cast<int>(task % n_hg);
  const int64_t rest = task / n_hg;
  const int64_t bt = rest % BM;
  const int part = static_cast<int>(rest / BM);
  const int64_t b = bt / p.q_len;
  const int head0 = hg * 32;
  const bool partial = p.num_parts > 1;
  const bool key0 = p.sink_mode == kSinkKey0;
  const bool null_sink = !partial && p.sink_mode == kSinkNull;

  // B operand of S^T: q[bt, head0 + n, h*D/2 + 8s .. +8].
  bf16x8 qf[S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + (bt * H + head0 + n) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 8);
  }
  const float c = p.scale_log2;  // > 0 on this path
  const float sink_raw = p.sinks ? p.sinks[head0 + n] * kLog2e / c : 0.0f;  // raw logit units

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  RowSoftmax rs;
  rs.m = null_sink ? sink_raw : kNegInf;
  rs.l = (null_sink && h == 0) ? 1.0f : 0.0f;  // the pair of lanes sharing a head splits l

  const int kb = part * p.part_len;
  const int ke = min(K, kb + p.part_len);
  const int nblk = (max(0, ke - kb) + kBlockKeys - 1) / kBlockKeys;
  // List entries through a bounds-checked buffer resource (reads past the list return 0; entries
  // past the slice are turned into -1 explicitly).
  const __amdgpu_buffer_rsrc_t lrs = make_list_rsrc(p.idx + bt * K, static_cast<uint32_t>(K) * 4u);
  // This batch row's cache through a buffer resource: a lane without a row reads past its end
  // and gets zeros.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(static_cast<const void *>(static_cast<const __bf16 *>(p.kv) + b * static_cast<int64_t>(N) * D)),
      static_cast<short>(0), static_cast<int>(static_cast<uint32_t>(N) * D * 2u), 0x00020000);
  __bf16 *tile = tiles[wave];

  // Index of this lane's row in block blk (-1: none).
  auto load_idx = [&](int blk) -> int {
    const int slot = kb + blk * kBlockKeys + n;
    const int x = __builtin_amdgcn_raw_buffer_load_b32(lrs, static_cast<uint32_t>(slot) * 4u, 0, 0);
    return slot < ke ? x : -1;
  };
  // Gather the lane's half row of block blk's row x (zero if x is not a row).
  struct Gathered {
    bf16x8 v[S];
    uint32_t vmask, zmask;  // rows that exist; rows that are cache row 0
  };
  auto gather = [&](int x, Gathered &g) {
    const bool valid = x >= 0 && x < N;
    g.vmask = static_cast<uint32_t>(__ballot(valid));
    g.zmask = key0 ? static_cast<uint32_t>(__ballot(valid && x == 0)) : 0u;
    const uint32_t off = valid ? static_cast<uint32_t>(x) * (D * 2u) + h * D : 0xfffff000u;
#pragma unroll
    for (int s = 0; s < S; ++s)
      g.v[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, off + s * 16u, 0, 0));
  };

  const int g16 = lane >> 4, i16 = lane & 15;
  auto compute = [&](const Gathered &g) {
    if (g.vmask == 0u) return;
    wave_lds_sync();  // the previous block's transposed reads are done
#pragma unroll
    for (int s = 0; s < S; ++s) *reinterpret_cast<bf16x8 *>(tile + n * LDSS + h * (D / 2) + s * 8) = g.v[s];
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g.v[s], qf[s], st, 0, 0, 0);
    // Accumulator element r of lane (n, h) is key 8*(r/4) + 4h + r%4 of head n.
    if (g.zmask) bias_block(st, g.zmask, h, sink_raw);
    if (g.vmask != 0xffffffffu) mask_block(st, g.vmask, h);
    float alpha;
    if (softmax_need_rescale(rs, block_max(st), c, alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    bf16x8 pb[2];
    softmax_probs(st, rs, c, pb);
    wave_lds_sync();  // the rows written above are visible to the whole wave
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
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[tt], acc[db], 0, 0, 0);
      }
    }
  };

  // Pipeline: the indices of blocks b+1..b+4 are in flight or held in a 4-entry ring, the rows of
  // block b+1 are gathered while block b is computed (two row buffers used in turn).
  int ix[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ix[j] = load_idx(j);
  Gathered ga, gb;
  if (nblk > 0) gather(ix[0], ga);
  ix[0] = load_idx(4);
  auto step = [&](int blk, const Gathered &cur, Gathered &nxt, int &ixs) {
    if (blk + 1 < nblk) {
      gather(ixs, nxt);  // block blk + 1
      ixs = load_idx(blk + 5);
    }
    compute(cur);
  };
  for (int b0 = 0; b0 < nblk; b0 += 4) {
    step(b0, ga, gb, ix[1]);
    if (b0 + 1 < nblk) step(b0 + 1, gb, ga, ix[2]);
    if (b0 + 2 < nblk) step(b0 + 2, ga, gb, ix[3]);
    if (b0 + 3 < nblk) step(b0 + 3, gb, ga, ix[0]);
  }

  // Epilogue: o = acc / l, lse = ln(2) * (m + log2 l).  Lane (n, h) holds dims 32db + 8i + 4h + {0..3}.
  const int head = head0 + n;
  const float l_tot = halves_sum(rs.l);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (rs.m * c + log2f(l_tot)) * kLn2 : kNegInf;
  if (partial) {
    const int64_t row = (static_cast<int64_t>(part) * BM + bt) * H + head;
    float *dst = p.part_o + row * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv,
                         acc[db][4 * i + 3] * inv};
        *reinterpret_cast<f32x4 *>(dst + 32 * db + 8 * i) = v;
      }
    if (h == 0) p.part_lse[row] = lse_v;
  } else {
    __bf16 *dst = static_cast<__bf16 *>(p.o) + (bt * H + head) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x4 v = {static_cast<__bf16>(acc[db][4 * i] * inv), static_cast<__bf16>(acc[db][4 * i + 1] * inv),
                          static_cast<__bf16>(acc[db][4 * i + 2] * inv),
                          static_cast<__bf16>(acc[db][4 * i + 3] * inv)};
        *reinterpret_cast<bf16x4 *>(dst + 32 * db + 8 * i) = v;
      }
    if (p.lse && h == 0) p.lse[bt * H + head] = lse_v;
  }
}

template <int D>
hipError_t launch(const IndexedParams &p, hipStream_t stream) {
  const int n_hg = p.num_heads / 32;
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * n_hg * p.num_parts;
  const int64_t blocks = (tasks + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((indexed_fwd_mfma<D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool indexed_mfma_supported(const IndexedParams &p) {
  // One batch row's cache and list are addressed with 32-bit buffer offsets.
  const int64_t cache_bytes = static_cast<int64_t>(p.kv_len) * p.head_dim * 2;
  return p.scale_log2 > 0.0f && (p.head_dim == 64 || p.head_dim == 128) && p.num_heads % 32 == 0 &&
         cache_bytes < (int64_t(1) << 31) - 4096 && static_cast<int64_t>(p.topk) * 4 < (int64_t(1) << 31);
}

hipError_t launch_indexed_mfma(const IndexedParams &p, hipStream_t stream) {
  return p.head_dim == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace sattn
