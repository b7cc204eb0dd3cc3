// Top-k lists chosen by a synthetic indexer (DeepSeek-V4 CSA/HCA article, §2.3: the indexer,
// fed the low-rank query qr, picks the compressed-region indices of each query; the window
// indices come first).  The article gives neither the scoring nor the weights; here compressed
// row c scores qr[b, t] . kidx[b, c] with a per-row index key, only rows visible at the query's
// position compete, the `topk` highest scores win (ties to the lower row), and the winners are
// listed as cache rows window + c in increasing c after the window part, then -1.
//
// gfx950 mapping: one workgroup per 32 queries of a batch row.  A 32-candidate score tile is
// S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = index keys read straight from memory, B = the
// 32 queries' qr in registers); lane (n, h) holds 16 candidates of query n.  Every candidate
// score becomes an order-preserving 32-bit key, and the k-th largest key of each query is found
// exactly by a radix select: four passes of 8 bits, each a histogram in LDS (LDS atomics; rows
// padded by one word so that the 32 queries' equal digits fall in different banks) over the
// candidates that still match the digits found so far, then a suffix scan of each histogram by
// one wave (4 bins a lane) finds the digit.  A counting pass and an ordered collection pass then
// write the winners in increasing row order (32-bit masks in candidate order, ties to the lower
// row).  NW waves split a workgroup's candidate tiles.  Scores are recomputed in every pass
// instead of stored: 32 x 8192 scores would not fit in LDS, and the index keys are L2-resident.
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"

namespace sattn {
namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_ix(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Order-preserving key of a float (larger float, larger key; -0 is taken as +0).
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Candidate position (within a 32-candidate tile) of accumulator element r of a lane in half h.
__device__ __forceinline__ int cand_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ uint32_t other_half(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane_id() < 32 ? r[1] : r[0];
}

constexpr int kHistStride = 257;
constexpr int kIndexerWaves = 8;

// Inclusive suffix sum over the lanes of a wave: lane l gets x[l] + x[l + 1] + ... + x[63].
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(x), off, 64));
    if (l + off < 64) x += y;
  }
  return x;
}

template <int S, int NW>
__global__ __launch_bounds__(64 * NW) void indexer_topk_kernel(IndexerParams a) {
  static_assert(32 % NW == 0, "queries split evenly over the waves");
  __shared__ uint32_t hist[32 * kHistStride];
  __shared__ uint32_t cnt_gt[NW][32], cnt_eq[NW][32];
  __shared__ uint32_t prefix[32], krem[32], total[32];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * 32;
  const int M = a.q_len, R = a.rank, W = a.window, K = a.window + a.topk;
  const int64_t sp = a.start_pos[b];

  // This lane's query (n) and how many compressed rows it sees.
  const int t = t0 + n;
  const bool q_ok = t < M;
  const int64_t p = sp + t;
  auto visible_rows = [&](int64_t pos) -> int {
    if (a.ratio <= 0 || pos < 0) return 0;
    const int64_t v = (pos + 1) / a.ratio;
    return static_cast<int>(v < a.n_comp ? v : a.n_comp);
  };
  const int vis = q_ok ? visible_rows(p) : 0;
  const int t_last = min(M, t0 + 32) - 1;
  const int c_wg = visible_rows(sp + t_last);  // the tile's last query sees the most rows
  const int n_tiles = (c_wg + 31) / 32;
  const int tile_lo = n_tiles * wave / NW, tile_hi = n_tiles * (wave + 1) / NW;

  // B operand: qr[b, t, 16 s + 8 h .. + 8] (queries past M read 0).
  const __bf16 *qb = static_cast<const __bf16 *>(a.qr) + static_cast<int64_t>(b) * M * R;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc_ix(qb, static_cast<uint32_t>(M) * R * 2);
  bf16x8 qf[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, static_cast<uint32_t>(t * R + 16 * s + 8 * h) * 2, 0, 0));
  const __bf16 *kb = static_cast<const __bf16 *>(a.kidx) + static_cast<int64_t>(b) * a.n_comp * R;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc_ix(kb, static_cast<uint32_t>(a.n_comp) * R * 2);

  // Keys of the 16 candidates this lane holds in tile `tile` (invisible ones flagged).
  auto tile_keys = [&](int tile, uint32_t (&key)[16], uint32_t &vmask) {
    const int c0 = tile * 32;
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 kf = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, static_cast<uint32_t>((c0 + n) * R + 16 * s + 8 * h) * 2, 0, 0));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
    }
    vmask = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      key[r] = score_key(st[r]);
      if (c0 + cand_of(r, h) < vis) vmask |= 1u << r;
    }
  };

  if (threadIdx.x < 32) {
    prefix[threadIdx.x] = 0;
    const int tq = t0 + static_cast<int>(threadIdx.x);
    const int v = tq < M ? visible_rows(sp + tq) : 0;
    krem[threadIdx.x] = static_cast<uint32_t>(min(a.topk, v));
    total[threadIdx.x] = static_cast<uint32_t>(min(a.topk, v));
  }

  // ---- radix select: the k-th largest key of each query, 8 bits per pass ----
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 32 * kHistStride; i += 64 * NW) hist[i] = 0;
    __syncthreads();
    const uint32_t pre = prefix[n];
    const bool want = krem[n] > 0;
    for (int tile = tile_lo; tile < tile_hi; ++tile) {
      uint32_t key[16], vmask;
      tile_keys(tile, key, vmask);  // wave-wide: lane n also supplies candidate row c0 + n
      if (!want) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool match = (vmask >> r) & 1u && (pass == 0 || (key[r] >> (shift + 8)) == pre);
        if (match) atomicAdd(&hist[n * kHistStride + ((key[r] >> shift) & 255u)], 1u);
      }
    }
    __syncthreads();
    // The digit of the need-th largest key: the largest d whose suffix count reaches need.
    for (int q = wave; q < 32; q += NW) {
      const uint32_t need = __builtin_amdgcn_readfirstlane(krem[q]);
      if (need == 0) continue;
      const uint32_t *hq = hist + q * kHistStride + 4 * lane;  // bins 4 lane .. 4 lane + 3
      const uint32_t c0 = hq[0], c1 = hq[1], c2 = hq[2], c3 = hq[3];
      const uint32_t incl = wave_suffix_sum(c0 + c1 + c2 + c3);
      const uint64_t reach = __ballot(incl >= need);  // lanes 0 .. l*: the suffix never grows with l
      const int ls = reach ? 63 - __builtin_clzll(reach) : 0;
      uint32_t above = incl - (c0 + c1 + c2 + c3);
      int d = 4 * lane;
      if (above + c3 >= need) d += 3;
      else if (above + c3 + c2 >= need) { above += c3; d += 2; }
      else if (above + c3 + c2 + c1 >= need) { above += c3 + c2; d += 1; }
      else above += c3 + c2 + c1;
      const uint32_t above_s = __builtin_amdgcn_readlane(above, ls);
      const uint32_t d_s = __builtin_amdgcn_readlane(static_cast<uint32_t>(d), ls);
      if (lane == 0) {
        krem[q] = need - above_s;
        prefix[q] = (prefix[q] << 8) | d_s;
      }
    }
    __syncthreads();
  }

  // ---- count the winners above the threshold and the ties at it, per wave ----
  const uint32_t T = prefix[n];  // the k-th largest key
  const uint32_t need_eq = krem[n];  // ties at T to take
  const bool any = total[n] > 0;
  {
    uint32_t gt = 0, eq = 0;
    for (int tile = tile_lo; tile < tile_hi; ++tile) {
      uint32_t key[16], vmask;
      tile_keys(tile, key, vmask);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool v = (vmask >> r) & 1u;
        gt += (v && key[r] > T) ? 1u : 0u;
        eq += (v && key[r] == T) ? 1u : 0u;
      }
    }
    gt += other_half(gt);
    eq += other_half(eq);
    if (h == 0) {
      cnt_gt[wave][n] = gt;
      cnt_eq[wave][n] = eq;
    }
  }
  __syncthreads();

  // ---- collect the winners in increasing row order ----
  // Every lane runs this pass, also for queries without candidates: lane n loads candidate row
  // c0 + n of each tile for all 32 queries (the A operand), so only the stores depend on the query.
  int32_t *orow = a.out + (static_cast<int64_t>(b) * M + t) * K + W;
  const uint32_t lim = any ? total[n] : 0u;  // the counts below add up to it; the bound guards the row
  {
    uint32_t base = 0, eq_before = 0;
    for (int w = 0; w < wave; ++w) {
      const uint32_t e = cnt_eq[w][n];
      const uint32_t left = need_eq > eq_before ? need_eq - eq_before : 0u;
      base += cnt_gt[w][n] + (e < left ? e : left);
      eq_before += e;
    }
    for (int tile = tile_lo; tile < tile_hi; ++tile) {
      uint32_t key[16], vmask;
      tile_keys(tile, key, vmask);
      uint32_t g = 0, e = 0;  // 32-bit masks in candidate order
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool v = (vmask >> r) & 1u;
        if (v && key[r] > T) g |= 1u << cand_of(r, h);
        if (v && key[r] == T) e |= 1u << cand_of(r, h);
      }
      g |= other_half(g);
      e |= other_half(e);
      const uint32_t left = need_eq > eq_before ? need_eq - eq_before : 0u;
      uint32_t take = e;
      if (static_cast<uint32_t>(__builtin_popcount(e)) > left) {  // keep the lowest `left` ties
        take = 0;
        uint32_t rest = e;
        for (uint32_t k = 0; k < left; ++k) {
          const uint32_t low = rest & (~rest + 1u);
          take |= low;
          rest ^= low;
        }
      }
      eq_before += __builtin_popcount(e);
      const uint32_t sel = g | take;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = cand_of(r, h);
        const uint32_t at = base + __builtin_popcount(sel & ((1u << k) - 1u));
        if (((sel >> k) & 1u) && at < lim) orow[at] = W + tile * 32 + k;
      }
      base += __builtin_popcount(sel);
    }
  }

  // ---- window part and -1 padding of the tile's lists, one wave per list ----
  const int rows = min(M, t0 + 32) - t0;
  for (int q = wave; q < rows; q += NW) {
    const int64_t pq = sp + t0 + q;
    const int64_t first = pq - W + 1 > 0 ? pq - W + 1 : 0;
    const int first_slot = static_cast<int>(first % W);
    const int64_t n_win = pq >= 0 ? pq - first + 1 : 0;
    const int pad_from = W + static_cast<int>(total[q]);
    int32_t *dst = a.out + (static_cast<int64_t>(b) * M + t0 + q) * K;
    for (int k = lane; k < K; k += 64) {
      if (k < W) {
        int slot = first_slot + k;
        slot = slot >= W ? slot - W : slot;
        dst[k] = k < n_win ? slot : -1;
      } else if (k >= pad_from) {
        dst[k] = -1;
      }
    }
  }
}

}  // namespace

hipError_t launch_indexer_topk(const IndexerParams &p, hipStream_t stream) {
  if (p.batch == 0 || p.q_len == 0) return hipSuccess;
  constexpr int NW = kIndexerWaves;
  const dim3 grid(static_cast<unsigned>((p.q_len + 31) / 32), static_cast<unsigned>(p.batch));
  const dim3 block(64 * NW);
  switch (p.rank / 16) {
    case 1: hipLaunchKernelGGL((indexer_topk_kernel<1, NW>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((indexer_topk_kernel<2, NW>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((indexer_topk_kernel<4, NW>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((indexer_topk_kernel<8, NW>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sattn
