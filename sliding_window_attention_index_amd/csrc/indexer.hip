// Top-k lists chosen by a synthetic indexer (DeepSeek-V4 CSA/HCA article, §2.3: the indexer,
// fed the low-rank query qr, picks the compressed-region indices of each query; the window
// indices come first).  The article gives neither the scoring nor the weights; here compressed
// row c scores qr[b, t] . kidx[b, c] with a per-row index key, only rows visible at the query's
// position compete, the `topk` highest scores win (ties to the lower row), and the winners are
// listed as cache rows window + c in increasing c after the window part, then -1.
//
// gfx950 mapping: one workgroup per 32 queries of a batch row; its waves split the candidate
// tiles.  A 32-candidate score tile is S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = index
// keys, B = the 32 queries' qr in registers); lane (n, h) holds 16 candidates of query n.  Lane
// n also supplies candidate row c0 + n of the A operand, so every score pass runs wave-wide and
// only stores depend on the lane's query.  In the MFMA layout each 16-byte load of a wave touches
// 32 rows, four per group of four lanes, which costs the vector memory unit four times the cycles
// of a contiguous load; so for rank 64 and 128 each wave stages its next tile in its own LDS slot
// with direct global->LDS DMA in contiguous pieces (swizzled for conflict-free reads) and reads
// the A operand from there.  Scores are recomputed in every pass instead of stored (32 x 8192
// scores would not fit in LDS; the index keys stay in L2).
//
// Fast path, two score passes.  The selection needs only a monotone map of the scores, so the
// first pass bins each score by its float bits >> 18 (sign, exponent and 5 mantissa bits: bins
// 1/32 octave wide for positive scores) inside a window of 256 codes placed per query from the
// root mean square of its first 32 scores (from 2 octaves below it to 6 above; everything lower
// falls in bin 0, everything higher in bin 255), one LDS histogram per query.  A wave-parallel suffix
// scan finds the bin holding the k-th largest score.  The second pass sets one bit per row
// above that bin in an LDS bitmap and appends the rows inside it (a few dozen for smooth score
// distributions) to a per-query LDS bucket; each bucket member is then ranked exactly (score,
// then lower row first) against the others, the winners' bits are set, and one wave per query
// turns its bitmap into the ordered list.
//
// Exact path, taken by the whole workgroup when some query's threshold bin is an edge bin of
// the window, holds more rows than the bucket, or the candidates exceed the bitmap (8192 rows): a radix
// select on order-preserving 32-bit keys (four 8-bit passes over LDS histograms), a counting
// pass and an ordered collection pass (32-bit masks in candidate order, ties to the lower row).
#include <climits>
#include <type_traits>

#include "lds_tile.hpp"
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

constexpr int kHistStride = 257;   // 256 bins, and a spare bin that absorbs invisible candidates
constexpr int kMaxMapTiles = 256;  // bitmap capacity: 256 tiles = 8192 compressed rows
constexpr int kMapStride = 257;    // words of one query's bitmap, one more against bank conflicts
constexpr int kBucketCap = 128;    // rows of a query's threshold bin that the exact ranking takes
constexpr int kCodeShift = 18;        // bin code: float bits >> 18 (5 mantissa bits, 1/32 octave)
constexpr int kWindowBelow = 64;      // the window starts 64 codes (2 octaves) below the estimate
constexpr int kMinWindowCode = 32;    // the window's first code is a normal float's (2^-126 and up)
constexpr int kMaxWindowCode = 7936;  // ... and its last code, first + 255, stays a positive float's

// LDS accesses of the score passes that the compiler does not see.  A compiler-visible LDS access
// would be preceded by a wait for every DMA in flight into this wave's slot (it cannot tell the
// addresses apart), which would cancel the prefetch; these are ordered by hand instead: an
// s_waitcnt lgkmcnt(0) (lds_drain) before the barrier that publishes them.
__device__ __forceinline__ void ds_add_u32_raw(uint32_t addr, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v));
}
__device__ __forceinline__ void ds_write_b32_raw(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v));
}
__device__ __forceinline__ uint32_t ds_add_rtn_u32_raw(uint32_t addr, uint32_t v) {
  uint32_t r;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr), "v"(v));
  return r;
}
__device__ __forceinline__ void lds_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// Inclusive prefix sum over the lanes of a wave: lane l gets x[0] + ... + x[l].
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), off, 64));
    if (l >= off) x += y;
  }
  return x;
}

// The bin of the need-th largest entry of a 256-bin histogram (need >= 1, at most the total):
// the largest d whose suffix count reaches need.  One wave, 4 bins a lane.  Returns d (uniform)
// and sets `above` to the count in bins above d and `in_bin` to the count in bin d.
__device__ __forceinline__ uint32_t find_bin(const uint32_t *row, uint32_t need, uint32_t &above_out,
                                             uint32_t &in_bin_out) {
  const int lane = lane_id();
  const uint32_t *hq = row + 4 * lane;  // bins 4 lane .. 4 lane + 3
  const uint32_t c0 = hq[0], c1 = hq[1], c2 = hq[2], c3 = hq[3];
  const uint32_t incl = wave_suffix_sum(c0 + c1 + c2 + c3);
  const uint64_t reach = __ballot(incl >= need);  // lanes 0 .. l*: the suffix never grows with l
  const int ls = reach ? 63 - __builtin_clzll(reach) : 0;
  uint32_t above = incl - (c0 + c1 + c2 + c3);
  uint32_t d = 4 * lane, cd;
  if (above + c3 >= need) { d += 3; cd = c3; }
  else if (above + c3 + c2 >= need) { above += c3; d += 2; cd = c2; }
  else if (above + c3 + c2 + c1 >= need) { above += c3 + c2; d += 1; cd = c1; }
  else { above += c3 + c2 + c1; cd = c0; }
  above_out = __builtin_amdgcn_readlane(above, ls);
  in_bin_out = __builtin_amdgcn_readlane(cd, ls);
  return __builtin_amdgcn_readlane(d, ls);
}

// Histograms (pass 1) and threshold-bin buckets (pass 2 on) never live at the same time.
union HistOrBucket {
  uint32_t hist[32 * kHistStride];
  uint2 bucket[32 * kBucketCap];
};

template <int S, int NW>
__global__ __launch_bounds__(64 * NW) void indexer_topk_kernel(IndexerParams a) {
  constexpr int D = 16 * S;                     // rank
  constexpr bool kDma = D == 64 || D == 128;    // staged through LDS (the swizzled tile layout)
  using Tile = SwizzledTile<kDma ? D : 64>;
  __shared__ __align__(256) uint8_t ring[kDma ? NW * Tile::kBytes : 256];
  __shared__ HistOrBucket hb;
  __shared__ uint32_t gmap[32 * kMapStride];
  __shared__ uint32_t cnt_gt[NW][32], cnt_eq[NW][32];
  __shared__ uint32_t prefix[32], krem[32], total[32], bcount[32];
  __shared__ int32_t ecut[32];
  __shared__ uint32_t exact_path;

  uint32_t *const hist = hb.hist;
  uint2 *const bucket = hb.bucket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * 32;
  const int M = a.q_len, R = a.rank, W = a.window, K = a.window + a.topk;
  const int64_t sp = a.start_pos[b];

  auto visible_rows = [&](int64_t pos) __attribute__((always_inline)) -> int {
    if (a.ratio <= 0 || pos < 0) return 0;
    const int64_t v = (pos + 1) / a.ratio;
    return static_cast<int>(v < a.n_comp ? v : a.n_comp);
  };
  // This lane's query (n): queries past M stand in for the last one (their lists are not written).
  const int t_last = min(M, t0 + 32) - 1;
  const int t = min(t0 + n, t_last);
  const int vis = visible_rows(sp + t);
  const int vis_min = visible_rows(sp + t0);  // rows every query of the tile sees
  const int c_wg = visible_rows(sp + t_last);  // rows the tile's last query sees (the most)
  const int n_tiles = (c_wg + 31) / 32;
  const int tile_lo = n_tiles * wave / NW, tile_hi = n_tiles * (wave + 1) / NW;
  const int full_hi = min(tile_hi, max(tile_lo, vis_min / 32));  // tiles below it need no mask

  // B operand: qr[b, t, 8 (h S + s) .. + 8] (MFMA step s, lane half h: the same rank slice as
  // the A operand).
  const __bf16 *qb = static_cast<const __bf16 *>(a.qr) + static_cast<int64_t>(b) * M * R;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc_ix(qb, static_cast<uint32_t>(M) * R * 2);
  bf16x8 qf[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, static_cast<uint32_t>(t * R + 8 * (h * S + s)) * 2, 0, 0));
  const __bf16 *kb = static_cast<const __bf16 *>(a.kidx) + static_cast<int64_t>(b) * a.n_comp * R;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc_ix(kb, static_cast<uint32_t>(a.n_comp) * R * 2);

  // A operand of tile `tile` read straight from memory: index keys of rows 32 tile + n (rows past
  // n_comp read 0).
  auto load_k = [&](int tile, u32x4 (&kf)[S]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      kf[s] = __builtin_amdgcn_raw_buffer_load_b128(
          krs, static_cast<uint32_t>((tile * 32 + n) * R + 8 * (h * S + s)) * 2, 0, 0);
  };
  auto scores = [&](const u32x4 (&kf)[S]) __attribute__((always_inline)) {
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], st, 0, 0, 0);
    return st;
  };
  // LDS staging (rank 64 and 128): this wave's slot, the DMA sources of its lanes (row, chunk of
  // a tile, in 1 KiB pieces) and the slot address of its A operand (row n, chunk h S + s at
  // kaddr ^ 16 s; the slot base has bits 4..7 clear).
  const uint32_t slot_addr = lds_addr(ring) + wave * Tile::kBytes;
  uint32_t dma_off[kDma ? Tile::kDmaPerTile : 1];
  if constexpr (kDma) {
#pragma unroll
    for (int u = 0; u < Tile::kDmaPerTile; ++u) {
      int row, chunk;
      Tile::dma_source(u, lane, row, chunk);
      dma_off[u] = static_cast<uint32_t>(row * R * 2 + chunk * 16);
    }
  }
  const uint32_t kaddr = slot_addr + Tile::offset(n, h * S);
  // Rows past n_comp read zeros (the descriptor's range check).
  auto issue_tile = [&](int tile) __attribute__((always_inline)) {
    if constexpr (kDma) {
      const uint32_t base = static_cast<uint32_t>(tile) * (32u * R * 2);
#pragma unroll
      for (int u = 0; u < Tile::kDmaPerTile; ++u) dma16(krs, ring + wave * Tile::kBytes + u * 1024, base + dma_off[u]);
    }
  };

  // f(tile, scores) over tiles [lo, hi), the next tile's keys fetched while a tile is scored.
  auto for_tiles = [&](int lo, int hi, auto &&f) __attribute__((always_inline)) {
    if (lo >= hi) return;
    if constexpr (kDma) {
      // One slot: wait for the tile, copy the A operand to registers, refill the slot with the
      // next tile, then score.
      issue_tile(lo);
      for (int tile = lo; tile < hi; ++tile) {
        wait_vmcnt<0>();
        u32x4 kf[S];
#pragma unroll
        for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<0>(kaddr ^ (16u * s));
        lgkm_fence<0>(kf);
        if (tile + 1 < hi) issue_tile(tile + 1);
        f(tile, scores(kf));
      }
    } else {
      // Two register buffers used in turn (no copy waits for the loads in flight).  The loads are
      // unconditional, so that the wait before each score counts only the loads behind it (a load
      // past the last row reads zeros through the buffer descriptor's range check), and a
      // scheduling barrier keeps the compiler from sinking them next to their use.
      u32x4 ka[S], kb2[S];
      load_k(lo, ka);
      for (int tile = lo; tile < hi; tile += 2) {
        load_k(tile + 1, kb2);
        __builtin_amdgcn_sched_barrier(0);
        f(tile, scores(ka));
        if (tile + 1 >= hi) break;
        load_k(tile + 2, ka);
        __builtin_amdgcn_sched_barrier(0);
        f(tile + 1, scores(kb2));
      }
    }
  };

  // ---- set-up: list sizes, cleared state, and each query's bin window ----
  if (threadIdx.x < 32) {
    const int q = threadIdx.x;
    const int v = t0 + q < M ? visible_rows(sp + t0 + q) : 0;
    const uint32_t tot = static_cast<uint32_t>(min(a.topk, v));
    total[q] = tot;
    krem[q] = tot;
    prefix[q] = 0;
    bcount[q] = 0;
  }
  if (threadIdx.x == 0) exact_path = n_tiles > kMaxMapTiles ? 1u : 0u;
  for (int i = threadIdx.x; i < 32 * kHistStride; i += 64 * NW) hist[i] = 0;
  for (int i = threadIdx.x; i < 32 * kMapStride; i += 64 * NW) gmap[i] = 0;
  if (wave == 0 && n_tiles > 0) {
    u32x4 kf[S];
    load_k(0, kf);
    const f32x16 st = scores(kf);
    float s2 = 0.0f;
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (cand_of(r, h) < vis) {
        s2 += st[r] * st[r];
        ++cnt;
      }
    s2 += __uint_as_float(other_half(__float_as_uint(s2)));
    cnt += other_half(cnt);
    if (h == 0) {
      const float rms = cnt > 0 ? sqrtf(s2 / static_cast<float>(cnt)) : 0.0f;
      const int code = static_cast<int>(__float_as_uint(rms) >> kCodeShift);
      ecut[n] = min(max(code - kWindowBelow, kMinWindowCode), kMaxWindowCode);  // the window's first code
    }
  }
  __syncthreads();

  // ---- window part and -1 padding of the tile's lists, one wave per list (their sizes are
  // known now; the stores drain while the scores are computed) ----
  const int rows = t_last - t0 + 1;
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

  // ---- fast path, pass 1: histogram of window bins ----
  if (exact_path == 0) {
    // bin = clamp(code, ec, ec + 255) - ec: bin 0 holds every score of code ec and below (the
    // negative ones included), bin 255 every score of code ec + 255 and above.  The clamp is
    // taken on the score itself, between the smallest float of code ec and the largest of code
    // ec + 255 (both positive normal floats), and the clamped code indexes the row from hbase.
    const int ec = ecut[n];
    const float lo_f = __uint_as_float(static_cast<uint32_t>(ec) << kCodeShift);
    const float hi_f = __uint_as_float((static_cast<uint32_t>(ec + 255) << kCodeShift) | ((1u << kCodeShift) - 1));
    const uint32_t hbase = lds_addr(hist) + static_cast<uint32_t>(n * kHistStride - ec) * 4u;
    auto clamped = [&](float x) __attribute__((always_inline)) {
      return __float_as_uint(__builtin_amdgcn_fmed3f(x, lo_f, hi_f)) >> kCodeShift;
    };
    for_tiles(tile_lo, full_hi, [&](int, const f32x16 &st) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) ds_add_u32_raw(hbase + 4u * clamped(st[r]), 1u);
    });
    for_tiles(full_hi, tile_hi, [&](int tile, const f32x16 &st) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds_add_u32_raw(hbase + 4u * (tile * 32 + cand_of(r, h) < vis ? clamped(st[r]) : static_cast<uint32_t>(ec + 256)),
                       1u);
    });
    lds_drain();
    __syncthreads();
    for (int q = wave; q < 32; q += NW) {
      const uint32_t tot = __builtin_amdgcn_readfirstlane(total[q]);
      const int vq = visible_rows(sp + t0 + q);
      if (tot == 0 || tot >= static_cast<uint32_t>(vq)) continue;  // nothing to choose between
      uint32_t above, in_bin;
      const uint32_t d = find_bin(hist + q * kHistStride, tot, above, in_bin);
      if (lane == 0) {
        krem[q] = tot - above;  // rows still to take from bin d
        prefix[q] = d;
        if (d == 0 || d == 255 || in_bin > kBucketCap) exact_path = 1;
      }
    }
    __syncthreads();
  }

  if (exact_path == 0) {
    // ---- fast path, pass 2: bitmap of the rows above the threshold bin, bucket of the rows in it ----
    // For an interior bin B of this query's window (code eb = ec + B), with scores compared as
    // signed integers of their bits: code > eb <=> bits > gt_bits, code >= eb <=> bits >= ge_bits.
    // Lists that take every visible row use their visibility mask; empty lists choose nothing.
    const uint32_t tot = total[n];
    const bool take_all = tot != 0 && tot >= static_cast<uint32_t>(vis);
    int gt_bits = INT_MAX, ge_bits = INT_MAX;
    if (tot != 0 && !take_all) {
      const int eb = ecut[n] + static_cast<int>(prefix[n]);
      ge_bits = eb << kCodeShift;
      gt_bits = ge_bits | ((1 << kCodeShift) - 1);
    }
    const uint32_t grow = lds_addr(gmap) + static_cast<uint32_t>(n * kMapStride) * 4u;
    const uint32_t bslots = lds_addr(bucket) + static_cast<uint32_t>(n * kBucketCap) * 8u;
    // Bits are set at half 0's candidate positions and moved to this lane's half (4 h) at the end.
    auto mark = [&](int tile, const f32x16 &st, auto full) __attribute__((always_inline)) {
      uint32_t g = 0, nge = 0, vbits = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int x = static_cast<int>(__float_as_uint(st[r]));
        const bool v = decltype(full)::value || tile * 32 + cand_of(r, h) < vis;
        const uint32_t bit = 1u << cand_of(r, 0);
        vbits |= v ? bit : 0u;
        g |= (v && x > gt_bits) ? bit : 0u;
        nge += (v && x >= ge_bits) ? 1u : 0u;
      }
      const uint32_t neq = take_all ? 0u : nge - static_cast<uint32_t>(__builtin_popcount(g));
      g = (take_all ? vbits : g) << (4 * h);
      if (neq != 0) {  // this lane holds rows of its query's threshold bin: reserve, then fill
        uint32_t slot = ds_add_rtn_u32_raw(lds_addr(&bcount[n]), neq);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int x = static_cast<int>(__float_as_uint(st[r]));
          const int c = tile * 32 + cand_of(r, h);
          if ((decltype(full)::value || c < vis) && x >= ge_bits && x <= gt_bits) {
            if (slot < kBucketCap) {
              u32x2 e;
              e[0] = __float_as_uint(st[r]);
              e[1] = static_cast<uint32_t>(c);
              ds_write_b64<0>(bslots + 8u * slot, e);
            }
            ++slot;
          }
        }
      }
      g |= other_half(g);
      if (h == 0) ds_write_b32_raw(grow + 4u * static_cast<uint32_t>(tile), g);
    };
    for_tiles(tile_lo, full_hi,
              [&](int tile, const f32x16 &st) __attribute__((always_inline)) { mark(tile, st, std::true_type{}); });
    for_tiles(full_hi, tile_hi,
              [&](int tile, const f32x16 &st) __attribute__((always_inline)) { mark(tile, st, std::false_type{}); });
    lds_drain();
    __syncthreads();

    // Rank each bucket member against the others (higher score first, then lower row); the
    // first krem of them are chosen.  Bucket members are positive floats with the same top
    // 32 - kCodeShift bits, and rows are below 8192 here, so (low kCodeShift bits of the score,
    // 8191 - row) as one 32-bit key orders them exactly.  Lane l holds members l and l + 64; each member is broadcast to the
    // wave in turn.
    for (int q = wave; q < 32; q += NW) {
      const uint32_t m = min(__builtin_amdgcn_readfirstlane(bcount[q]), static_cast<uint32_t>(kBucketCap));
      if (m == 0) continue;
      const uint32_t take = krem[q];
      const uint2 *bq = bucket + q * kBucketCap;
      static_assert(kCodeShift + 13 <= 32 && kMaxMapTiles * 32 <= 8192, "bucket keys fit 32 bits");
      auto key32 = [](uint2 v) __attribute__((always_inline)) {
        return ((v.x & ((1u << kCodeShift) - 1)) << 13) | (8191u - v.y);
      };
      const uint2 m0 = static_cast<uint32_t>(lane) < m ? bq[lane] : make_uint2(0u, 8191u);  // key 0
      const uint32_t k0 = key32(m0);
      uint32_t r0 = 0;
      if (m <= 64) {
        // 8 members at a time: lanes past m hold key 0, which ranks above no member.
        const uint32_t m8 = (m + 7) & ~7u;
        for (uint32_t f = 0; f < m8; f += 8) {
#pragma unroll
          for (uint32_t u = 0; u < 8; ++u)
            r0 += static_cast<uint32_t>(__builtin_amdgcn_readlane(k0, f + u)) > k0 ? 1u : 0u;
        }
        if (static_cast<uint32_t>(lane) < m && r0 < take)
          atomicOr(&gmap[q * kMapStride + (m0.y >> 5)], 1u << (m0.y & 31));
      } else {
        const uint2 m1 = static_cast<uint32_t>(lane) + 64 < m ? bq[lane + 64] : make_uint2(0u, 8191u);
        const uint32_t k1 = key32(m1);
        uint32_t r1 = 0;
        for (uint32_t f = 0; f < 64; ++f) {
          const uint32_t kf = static_cast<uint32_t>(__builtin_amdgcn_readlane(k0, f));
          r0 += kf > k0 ? 1u : 0u;
          r1 += kf > k1 ? 1u : 0u;
        }
        for (uint32_t f = 64; f < m; ++f) {
          const uint32_t kf = static_cast<uint32_t>(__builtin_amdgcn_readlane(k1, f - 64));
          r0 += kf > k0 ? 1u : 0u;
          r1 += kf > k1 ? 1u : 0u;
        }
        if (static_cast<uint32_t>(lane) < m && r0 < take)
          atomicOr(&gmap[q * kMapStride + (m0.y >> 5)], 1u << (m0.y & 31));
        if (static_cast<uint32_t>(lane) + 64 < m && r1 < take)
          atomicOr(&gmap[q * kMapStride + (m1.y >> 5)], 1u << (m1.y & 31));
      }
    }
    __syncthreads();

    // One wave per list: the bitmap's set bits in increasing row order.
    for (int q = wave; q < 32; q += NW) {
      const uint32_t tq = __builtin_amdgcn_readfirstlane(total[q]);
      if (tq == 0) continue;
      int32_t *orow = a.out + (static_cast<int64_t>(b) * M + t0 + q) * K + W;
      const uint32_t *gq = gmap + q * kMapStride;
      uint32_t base = 0;
      for (int j0 = 0; j0 < n_tiles; j0 += 64) {
        const int j = j0 + lane;
        uint32_t word = j < n_tiles ? gq[j] : 0u;
        const uint32_t c = __builtin_popcount(word);
        const uint32_t incl = wave_prefix_sum(c);
        uint32_t pos = base + incl - c;
        while (word != 0) {
          const int bit = __builtin_ctz(word);
          word &= word - 1;
          if (pos < tq) orow[pos] = W + 32 * j + bit;
          ++pos;
        }
        base += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  } else {
    // ---- exact path ----
    __syncthreads();  // every wave has read exact_path before the state below is reset
    if (threadIdx.x < 32) {
      prefix[threadIdx.x] = 0;
      krem[threadIdx.x] = total[threadIdx.x];
    }
    // Keys of the 16 candidates this lane holds in tile `tile` (invisible ones flagged).
    auto tile_keys = [&](int tile, uint32_t (&key)[16], uint32_t &vmask) __attribute__((always_inline)) {
      u32x4 kf[S];
      load_k(tile, kf);
      const f32x16 st = scores(kf);
      vmask = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        key[r] = score_key(st[r]);
        if (tile * 32 + cand_of(r, h) < vis) vmask |= 1u << r;
      }
    };

    // Radix select: the k-th largest key of each query, 8 bits per pass.
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = threadIdx.x; i < 32 * kHistStride; i += 64 * NW) hist[i] = 0;
      __syncthreads();
      const uint32_t pre = prefix[n];
      const bool want = krem[n] > 0;
      for (int tile = tile_lo; tile < tile_hi; ++tile) {
        uint32_t key[16], vmask;
        tile_keys(tile, key, vmask);
        if (!want) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool match = (vmask >> r) & 1u && (pass == 0 || (key[r] >> (shift + 8)) == pre);
          if (match) atomicAdd(&hist[n * kHistStride + ((key[r] >> shift) & 255u)], 1u);
        }
      }
      __syncthreads();
      for (int q = wave; q < 32; q += NW) {
        const uint32_t need = __builtin_amdgcn_readfirstlane(krem[q]);
        if (need == 0) continue;
        uint32_t above, in_bin;
        const uint32_t d = find_bin(hist + q * kHistStride, need, above, in_bin);
        if (lane == 0) {
          krem[q] = need - above;
          prefix[q] = (prefix[q] << 8) | d;
        }
      }
      __syncthreads();
    }

    // Count the winners above the threshold and the ties at it, per wave.
    const uint32_t T = prefix[n];      // the k-th largest key
    const uint32_t need_eq = krem[n];  // ties at T to take
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

    // Collect the winners in increasing row order.
    int32_t *orow = a.out + (static_cast<int64_t>(b) * M + t0 + n) * K + W;
    const uint32_t lim = t0 + n < M ? total[n] : 0u;  // the counts add up to it; the bound guards the row
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
}

template <int S>
hipError_t launch_rank(const IndexerParams &p, hipStream_t stream) {
  constexpr int NW = S <= 4 ? 16 : 8;  // 128 VGPRs a lane at 16 waves; rank 128 needs more
  const dim3 grid(static_cast<unsigned>((p.q_len + 31) / 32), static_cast<unsigned>(p.batch));
  if (trace_on())
    trace("indexer_topk_kernel<rank=%d, waves=%d> grid=%ux%u block=%d n_comp=%d topk=%d window=%d ratio=%d", 16 * S, NW,
          grid.x, grid.y, 64 * NW, p.n_comp, p.topk, p.window, p.ratio);
  hipLaunchKernelGGL((indexer_topk_kernel<S, NW>), grid, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_topk(const IndexerParams &p, hipStream_t stream) {
  if (p.batch == 0 || p.q_len == 0) return hipSuccess;
  switch (p.rank / 16) {
    case 1: return launch_rank<1>(p, stream);
    case 2: return launch_rank<2>(p, stream);
    case 4: return launch_rank<4>(p, stream);
    case 8: return launch_rank<8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sattn
