// Sliding-window attention over a varlen batch (bf16, MFMA), persistent.
//
// Problem (vLLM PR #49815 report, "关键源码片段"): per sequence of a
// cu_seqlens batch, query i attends keys j of the same sequence inside the
// window, GQA head h reads KV head h / (H / H_kv), and per-head sinks are
// either a bias on the logit of the sequence's key 0 or a null logit in the
// denominator.  The report also notes that the window path is only fast if
// the kernel visits just the key blocks that meet the band; iterating every
// key block and masking afterwards costs O(seq_len^2).
//
// gfx950 mapping:
//   * A tile is (KV head g, QT consecutive queries of one sequence); each of
//     the 4 waves of a workgroup owns 32 rows = 32/G queries x G heads (the G
//     query heads of one KV head share every K/V element, so they fill the
//     MFMA N dimension).  A tile walks the 32-key blocks that meet the band
//     of any of its queries.
//   * Workgroups are persistent: each loops over its share of the non-empty
//     tiles, enumerated on the device from cu_seqlens.  Round k hands a
//     contiguous run of tiles to each XCD and rotates the XCDs from round to
//     round, so neighbouring tiles (which share most of their keys) run
//     together in one XCD's L2 while the XCDs stay evenly loaded.
//   * Everything a tile reads arrives through one stream of direct
//     global->LDS DMA into a 4-slot ring of swizzled tiles: first the tile's
//     128 Q rows (two slots), then its K/V blocks (one slot each: K tile +
//     V tile).  The stream runs three slots ahead across tile boundaries, so
//     the next tile's Q and first keys load while the current tile computes.
//     Each wave waits for its own DMA of a slot, one barrier publishes it,
//     and the DMA that refills the slot freed by the previous step is issued
//     after that barrier.
//   * LDS reads are inline asm that the compiler cannot see, so it never
//     inserts a full vmcnt(0) for them; the wave keeps the exact vmcnt count
//     of its outstanding DMAs and O stores (stores are buffer stores with a
//     fixed instruction count; rows past the sequence fall outside the
//     buffer and are dropped, as are Q/K/V rows past it, which read as zero).
//   * Per block: S^T = K . Q^T (v_mfma_f32_32x32x16_bf16; A = K rows from
//     LDS, B = Q rows held in registers), online softmax in the S^T
//     accumulator layout (one head-row per lane pair), then
//     O^T += V^T . P^T with V^T fetched by ds_read_b64_tr_b16.
#include <algorithm>

#include "lds_tile.hpp"
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kXcds = 8;
constexpr int kRing = 4;

template <int I>
struct Idx {
  static constexpr int value = I;
};

// What the stream needs to know about one tile (wave-uniform; nblk == 0 marks "no tile").
struct TileInfo {
  int g;             // KV head
  int a, L, Lq;      // sequence start, length, computed length (min(L, max_seqlen))
  int q_first, q_last;
  int lo_wg, hi_wg;  // keys any query of the tile can see
  int nblk;          // 32-key blocks
};

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <int D, int G>
__global__ __launch_bounds__(256) void window_fwd_mfma(WindowParams p) {
  using Tile = SwizzledTile<D>;
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int QW = 32 / G;                  // queries per wave
  constexpr int QT = 4 * QW;                  // queries per tile
  constexpr int DPW = Tile::kDmaPerTile / 4;  // DMA instructions per wave per 32-row tile
  constexpr int kSlot = 2 * Tile::kBytes;     // K tile + V tile (or two Q half-tiles)
  constexpr int kDmaPerSlot = 2 * DPW;        // DMA instructions per wave per slot
  constexpr int kStageBytes = 32 * 128;       // O staging per wave: 32 rows x 32 dims of fp32
  constexpr int kStores = 2 * DB + 1;         // O stores + one lse store per wave per tile
  static_assert(DPW >= 1, "tile too small for four waves");
  static_assert(64 % G == 0, "a Q slot must hold whole queries");
  __shared__ __attribute__((aligned(1024))) char ring[kRing * kSlot];
  __shared__ __attribute__((aligned(16))) char stage[4 * kStageBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int H = p.num_heads, Hkv = p.num_kv_heads;
  const int wl = p.window_left, wr = p.window_right;
  const float c = p.scale_log2;  // > 0 on this path

  // ---- tile enumeration: tiles of (head g, sequence s) in order, ceil(Lq_s / QT) per sequence ----
  // One 64-sequence chunk of cu_seqlens is cached in registers (lane = sequence).
  int ch_base = 0, ch_tiles0 = 0, ch_a = 0, ch_len = 0, ch_nt = 0, ch_incl = 0;
  auto load_chunk = [&](int base, int tiles_before) {
    const int s = base + lane;
    const bool ok = s < p.num_seqs;
    ch_a = ok ? p.cu_seqlens[s] : 0;
    ch_len = ok ? p.cu_seqlens[s + 1] - ch_a : 0;
    ch_nt = ok ? (min(ch_len, p.max_seqlen) + QT - 1) / QT : 0;
    ch_incl = tiles_before + wave_incl_scan(ch_nt);
    ch_base = base;
    ch_tiles0 = tiles_before;
  };
  int per_head = 0;
  for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
    load_chunk(s0, per_head);
    per_head = __builtin_amdgcn_readlane(ch_incl, 63);
  }
  if (p.num_seqs > 64) load_chunk(0, 0);
  const int total = per_head * Hkv;
  const int per_xcd = gridDim.x / kXcds;  // workgroups per XCD (the grid is a multiple of 8)
  const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
  auto locate = [&](int k) -> TileInfo {
    TileInfo t = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    const int r = (k * kXcds + xcd) * per_xcd + jx;  // k-th tile of this workgroup
    if (r >= total) return t;
    t.g = r / per_head;
    const int rr = r - t.g * per_head;
    if (rr < ch_tiles0) load_chunk(0, 0);  // a new head starts over
    uint64_t m;
    while (!(m = __ballot(ch_incl > rr))) load_chunk(ch_base + 64, __builtin_amdgcn_readlane(ch_incl, 63));
    const int l0 = __builtin_ctzll(m);
    const int tile = rr - (__builtin_amdgcn_readlane(ch_incl, l0) - __builtin_amdgcn_readlane(ch_nt, l0));
    t.a = __builtin_amdgcn_readlane(ch_a, l0);
    t.L = __builtin_amdgcn_readlane(ch_len, l0);
    t.Lq = min(t.L, p.max_seqlen);
    t.q_first = tile * QT;
    t.q_last = min(t.Lq, t.q_first + QT) - 1;
    t.lo_wg = wl < 0 ? 0 : max(0, t.q_first - wl);
    t.hi_wg = wr < 0 ? t.L - 1 : min(t.L - 1, t.q_last + wr);
    t.nblk = (t.hi_wg - t.lo_wg + kBlockKeys) / kBlockKeys;
    return t;
  };
  // Sinks of heads 0..63 in lane registers (read with a lane shuffle per tile).
  const float sink_lane = (p.sink_mode != kSinkNone && lane < H) ? p.sinks[lane] : 0.0f;

  // ---- per-lane DMA sources inside a 32-row tile ----
  const uint32_t kv_tok = static_cast<uint32_t>(Hkv) * D * 2;  // bytes between tokens of k / v
  const uint32_t q_tok = static_cast<uint32_t>(H) * D * 2;     // bytes between tokens of q / o
  uint32_t kv_src[DPW], q_src[2][DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    int row, chunk;
    Tile::dma_source(wave * DPW + u, lane, row, chunk);
    kv_src[u] = static_cast<uint32_t>(row) * kv_tok + chunk * 16;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int R = t * 32 + row;  // row of a Q slot: query R / G, head R % G
      q_src[t][u] = static_cast<uint32_t>(R / G) * q_tok + (R % G) * D * 2 + chunk * 16;
    }
  }

  // ---- the stream: per tile two Q slots, then nblk K/V slots ----
  // The issue cursor runs three slots ahead and every tile has at least three slots, so the tile
  // being computed is either the issue cursor's tile or the one before it.
  TileInfo it = locate(0);  // tile issue_k
  TileInfo pt = it;         // tile issue_k - 1
  if (it.nblk == 0) return;  // workgroup-uniform: nothing to do
  int issue_k = 0, issue_pos = 0;  // next slot to issue: position issue_pos of tile issue_k
  int issued = 0;                   // slots issued so far
  auto issue_next = [&](int slot) {
    if (it.nblk == 0) return;  // the schedule is exhausted
    char *dst = ring + slot * kSlot;
    if (issue_pos < 2) {
      const __bf16 *qb = static_cast<const __bf16 *>(p.q) + (static_cast<int64_t>(it.a) * H + it.g * G) * D;
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qb, static_cast<uint32_t>(it.Lq - 1) * q_tok + G * D * 2);
      const uint32_t base = static_cast<uint32_t>(it.q_first + issue_pos * (64 / G)) * q_tok;
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        dma16(qrs, dst + (wave * DPW + u) * 1024, base + q_src[0][u]);
        dma16(qrs, dst + Tile::kBytes + (wave * DPW + u) * 1024, base + q_src[1][u]);
      }
    } else {
      const int64_t kv0 = (static_cast<int64_t>(it.a) * Hkv + it.g) * D;
      const uint32_t bytes = static_cast<uint32_t>(it.L - 1) * kv_tok + D * 2;
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const __bf16 *>(p.k) + kv0, bytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const __bf16 *>(p.v) + kv0, bytes);
      const uint32_t row0 = static_cast<uint32_t>(it.lo_wg + (issue_pos - 2) * kBlockKeys) * kv_tok;
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        dma16(krs, dst + (wave * DPW + u) * 1024, row0 + kv_src[u]);
        dma16(vrs, dst + Tile::kBytes + (wave * DPW + u) * 1024, row0 + kv_src[u]);
      }
    }
    ++issued;
    if (++issue_pos == 2 + it.nblk) {
      ++issue_k;
      issue_pos = 0;
      pt = it;
      it = locate(issue_k);
    }
  };

  // ---- per-lane LDS read offsets: rows (K for the A operand, Q for B) and V^T quads ----
  const uint32_t ring_addr = lds_addr(ring);
  uint32_t koff[S];
#pragma unroll
  for (int s = 0; s < S; ++s) koff[s] = ring_addr + Tile::offset(n, h * S + s);
  const int g16 = lane >> 4, i16 = lane & 15;
  uint32_t voff[2][DB][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 16 * tt + 4 * h + (i16 >> 2) + 8 * e;
        const int chunk = 4 * db + 2 * (g16 & 1) + ((i16 & 3) >> 1);
        voff[tt][db][e] = ring_addr + Tile::kBytes + Tile::offset(row, chunk) + (i16 & 1) * 8;
      }

  // ---- compute-side state of the current tile ----
  int comp_k = 0, comp_pos = 0;
  int since_store = 1 << 20;  // steps since this wave last issued its O stores
  bf16x8 qf[S];
  f32x16 acc[DB];
  RowSoftmax rs;
  int wq0 = 0, wq1 = 0, lo_w = 0, hi_w = -1, my_q = 0;
  bool wave_active = false;
  float sink_raw = 0.0f;

  auto begin_tile = [&](TileInfo t) {
    wq0 = t.q_first + wave * QW;
    wave_active = wq0 < t.Lq;
    wq1 = min(t.Lq, wq0 + QW) - 1;
    lo_w = wl < 0 ? 0 : max(0, wq0 - wl);
    hi_w = wr < 0 ? t.L - 1 : min(t.L - 1, wq1 + wr);
    my_q = wq0 + n / G;
    const int head = t.g * G + n % G;
    float sink = 0.0f;
    if (p.sink_mode != kSinkNone) sink = H <= 64 ? __shfl(sink_lane, head, 64) : p.sinks[head];
    sink_raw = sink * kLog2e / c;  // the running max is kept in raw logit units
    // An opaque zero: a plain f32x16{} is loop invariant, and the compiler keeps it in 16 AGPRs
    // across the whole persistent loop, which costs the kernel its second wave per SIMD.
    float z = 0.0f;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = z;
    rs.m = p.sink_mode == kSinkNull ? sink_raw : kNegInf;
    rs.l = (p.sink_mode == kSinkNull && h == 0) ? 1.0f : 0.0f;  // the lane pair of a row splits l
  };

  auto load_q = [&](auto I, int half) {
    constexpr int off = decltype(I)::value * kSlot;
    u32x4 r[S];
    if (half) {
#pragma unroll
      for (int s = 0; s < S; ++s) r[s] = ds_read_b128<off + Tile::kBytes>(koff[s]);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) r[s] = ds_read_b128<off>(koff[s]);
    }
    lgkm_fence<0>(r);
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = __builtin_bit_cast(bf16x8, r[s]);
  };

  auto compute_block = [&](auto I, TileInfo t, int blk) {
    constexpr int off = decltype(I)::value * kSlot;
    const int kb0 = t.lo_wg + blk * kBlockKeys;
    u32x4 kf[S];
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<off>(koff[s]);
    lgkm_fence<0>(kf);
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], st, 0, 0, 0);
    // V^T quads: read while the QK products and the softmax run (the K rows are dead by then).
    u32x2 vr[4 * DB];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 2; ++e) vr[(tt * DB + db) * 2 + e] = ds_read_tr_b16<off>(voff[tt][db][e]);
    // Element r of lane (n, h) is key kb0 + 8*(r/4) + 4h + r%4 for this lane's row.
    if (p.sink_mode == kSinkKey0 && kb0 == 0 && h == 0) st[0] += sink_raw;
    const int kb1 = kb0 + kBlockKeys - 1;
    const bool interior = (wl < 0 || kb0 >= wq1 - wl) && (wr < 0 || kb1 <= wq0 + wr) && kb1 <= t.hi_wg;
    if (!interior) {
      const int lo_q = wl < 0 ? 0 : my_q - wl;
      const int hi_q = min(t.hi_wg, wr < 0 ? t.L - 1 : my_q + wr);
      mask_block(st, range_bits(lo_q - kb0, hi_q - kb0), h);
    }
    float alpha;
    if (softmax_need_rescale(rs, block_max(st), c, alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    bf16x8 pb[2];
    softmax_probs(st, rs, c, pb);
    lgkm_fence<0>(vr);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 ra = vr[(tt * DB + db) * 2], rb = vr[(tt * DB + db) * 2 + 1];
        const u32x4 av = {ra[0], ra[1], rb[0], rb[1]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[tt], acc[db], 0, 0, 0);
      }
  };

  // O and lse of the tile, always kStores buffer stores per wave (rows past the sequence fall
  // outside the buffer and are dropped, as is the lse of the upper half-wave).  The O^T
  // accumulator gives a lane 4-dim pieces of one row; stored as they are, every instruction
  // would scatter 8-byte pieces over 32 rows.  Instead each 32-dim block of the accumulator goes
  // through a wave-private LDS area as scaled fp32 (16-byte chunk c of row r at c ^ (r & 7):
  // conflict free both ways), is read back as 8 consecutive dims per lane, rounded and stored as
  // 16 bytes per lane, 64 contiguous bytes per row.
  auto store_tile = [&](TileInfo t) {
    const float l_tot = halves_sum(rs.l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t row0 = static_cast<int64_t>(t.a) * H + t.g * G;  // first (token, head) row of the tile's group
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(static_cast<__bf16 *>(p.o) + row0 * D, static_cast<uint32_t>(t.Lq - 1) * q_tok + G * D * 2);
    const uint32_t sbase = lds_addr(stage) + wave * kStageBytes;
    // write side: lane (n, h) holds dims 32 db + 8 j + 4 h .. +3 of row n = fp32 chunk 2 j + h
    const uint32_t wr0 = sbase + n * 128;
    // read side: lane l takes row 16 i + l / 4, fp32 chunks 2 (l % 4) and 2 (l % 4) + 1
    const int rl = lane >> 2, q4 = lane & 3;
    const uint32_t rd0 = sbase + rl * 128 + (((2 * q4) ^ (rl & 7)) << 4);
    const uint32_t rd1 = sbase + rl * 128 + (((2 * q4 + 1) ^ (rl & 7)) << 4);
    // Wave row r = 16 i + rl is query wq0 + r / G, head t.g * G + r % G; as G divides 16 or 16
    // divides G, its byte offset splits into a lane part (row rl) and a uniform part (16 i).
    const uint32_t vlane = static_cast<uint32_t>(rl / G) * q_tok + (rl % G) * D * 2 + q4 * 16;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // scaled here, where the lane still owns row n (after the transposition it does not)
        const u32x4 w = {__float_as_uint(acc[db][4 * j] * inv), __float_as_uint(acc[db][4 * j + 1] * inv),
                         __float_as_uint(acc[db][4 * j + 2] * inv), __float_as_uint(acc[db][4 * j + 3] * inv)};
        ds_write_b128<0>(wr0 + (((2 * j + h) ^ (n & 7)) << 4), w);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 x[2];
        x[0] = ds_read_b128<0>(rd0 + i * 2048);
        x[1] = ds_read_b128<0>(rd1 + i * 2048);
        lgkm_fence<0>(x);
        const bf16x8 v = {static_cast<__bf16>(__uint_as_float(x[0][0])), static_cast<__bf16>(__uint_as_float(x[0][1])),
                          static_cast<__bf16>(__uint_as_float(x[0][2])), static_cast<__bf16>(__uint_as_float(x[0][3])),
                          static_cast<__bf16>(__uint_as_float(x[1][0])), static_cast<__bf16>(__uint_as_float(x[1][1])),
                          static_cast<__bf16>(__uint_as_float(x[1][2])), static_cast<__bf16>(__uint_as_float(x[1][3]))};
        const uint32_t uni = static_cast<uint32_t>(wq0 + (16 * i) / G) * q_tok + ((16 * i) % G) * D * 2 + db * 64;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ors, vlane,
                                               __builtin_amdgcn_readfirstlane(uni), 0);
      }
    }
    const __amdgpu_buffer_rsrc_t lrs =
        make_rsrc(p.lse ? p.lse + row0 : nullptr, p.lse ? (static_cast<uint32_t>(t.Lq - 1) * H + G) * 4 : 0u);
    const float lse_v = l_tot > 0.0f ? (rs.m * c + log2f(l_tot)) * kLn2 : kNegInf;
    const uint32_t loff = h == 0 ? (static_cast<uint32_t>(my_q) * H + n % G) * 4 : 0xffffffffu;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse_v), lrs, loff, 0, 0);
  };

  // Wait until this slot's DMA (issued three steps earlier) has landed.  Vector-memory operations
  // of this wave that are younger than it: the DMA of up to two later slots and, within three steps
  // after a tile ended, that tile's stores.
  auto wait_slot = [&](int younger_slots, bool stores_younger) {
    if (stores_younger) {
      if (younger_slots >= 2) wait_vmcnt<2 * kDmaPerSlot + kStores>();
      else if (younger_slots == 1) wait_vmcnt<kDmaPerSlot + kStores>();
      else wait_vmcnt<kStores>();
    } else {
      if (younger_slots >= 2) wait_vmcnt<2 * kDmaPerSlot>();
      else if (younger_slots == 1) wait_vmcnt<kDmaPerSlot>();
      else wait_vmcnt<0>();
    }
  };

  for (int s0 = 0; s0 < kRing - 1; ++s0) issue_next(s0);

  int step_no = 0;  // stream position being computed
  bool done = false;
  auto step = [&](auto I) {
    constexpr int i = decltype(I)::value;
    if (done) return;
    const TileInfo t = comp_k == issue_k ? it : pt;  // copied before the issue below may move on
    wait_slot(min(2, issued - step_no - 1), since_store < 3);
    __builtin_amdgcn_s_barrier();
    issue_next((i + kRing - 1) % kRing);
    if (comp_pos == 0) {
      begin_tile(t);
      if (wave < 2) load_q(I, wave);
    } else if (comp_pos == 1) {
      if (wave >= 2) load_q(I, wave - 2);
    } else {
      const int blk = comp_pos - 2;
      const int kb0 = t.lo_wg + blk * kBlockKeys;
      if (wave_active && kb0 <= hi_w && kb0 + kBlockKeys - 1 >= lo_w) compute_block(I, t, blk);
    }
    ++since_store;
    if (++comp_pos == 2 + t.nblk) {
      store_tile(t);
      since_store = 0;
      comp_pos = 0;
      ++comp_k;
      done = (comp_k == issue_k ? it : pt).nblk == 0;
    }
    ++step_no;
  };
  while (!done) {
    step(Idx<0>{});
    step(Idx<1>{});
    step(Idx<2>{});
    step(Idx<3>{});
  }
}

template <int D, int G>
hipError_t launch(const WindowParams &p, hipStream_t stream) {
  constexpr int QT = 4 * (32 / G);
  static const int per_cu = [] {
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, window_fwd_mfma<D, G>, 256, 0) == hipSuccess ? n : 1;
  }();
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // Upper bound of the non-empty tiles (cu_seqlens stays on the device).
  const int64_t tiles = static_cast<int64_t>((p.max_seqlen + QT - 1) / QT) * p.num_seqs * p.num_kv_heads;
  int64_t grid = std::min<int64_t>(tiles, static_cast<int64_t>(cus) * std::max(per_cu, 1));
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((window_fwd_mfma<D, G>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const WindowParams &p, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch<D, 1>(p, stream);
    case 2: return launch<D, 2>(p, stream);
    case 4: return launch<D, 4>(p, stream);
    case 8: return launch<D, 8>(p, stream);
    case 16: return launch<D, 16>(p, stream);
    default: return launch<D, 32>(p, stream);
  }
}

}  // namespace

bool window_mfma_supported(const WindowParams &p) {
  const int G = p.group;
  // Buffer offsets are 32-bit: one sequence's q / o / k / v span must stay below 2 GiB.
  const int64_t seq_span = static_cast<int64_t>(p.max_seqlen) * p.num_heads * p.head_dim * 2;
  return p.scale_log2 > 0.0f && (p.head_dim == 64 || p.head_dim == 128) &&
         (G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32) && seq_span < (int64_t(1) << 31);
}

hipError_t launch_window_mfma(const WindowParams &p, hipStream_t stream) {
  return p.head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sattn
