// Sliding-window attention over a varlen batch (bf16, MFMA).
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
//   * One workgroup per tile = (KV head g, QT consecutive queries of one
//     sequence).  Each of its waves (4 at D = 128, 8 at D = 64) owns 32 rows = 32/G queries x G heads
//     (the G query heads of one KV head share every K/V element, so they fill
//     the MFMA N dimension) and keeps their Q operand in registers.  The tile
//     walks the 32-key blocks that meet the band of any of its queries; a
//     wave skips the blocks outside its own band.
//   * Tile ids are dealt out XCD by XCD: the workgroups the dispatcher sends to
//     one XCD (blockIdx % 8) take a contiguous run of tiles, so neighbouring
//     tiles of a sequence, which read mostly the same keys, meet in that XCD's
//     L2.
//   * K and V blocks arrive by direct global->LDS DMA (buffer_load ... lds)
//     into a ring of swizzled slots (K tile + V tile; 3 slots at D = 128, so
//     that three workgroups share a CU, 4 at D = 64) shared by the
//     workgroup's waves; each wave fetches an equal share of every slot.
//     Block j + slots - 1 is requested while block j is computed.  Requests
//     past the last block point outside the buffer (they read no memory and
//     land as zeros in a slot no step reads), so every step waits for the
//     same number of this wave's requests; one barrier per step then
//     publishes the slot and frees the one read in the step before.
//   * LDS reads are inline asm the compiler cannot see, so it never inserts
//     a full vmcnt(0) wait for them; lgkmcnt waits are explicit.
//   * Per block: S^T = K . Q^T (v_mfma_f32_32x32x16_bf16; A = K rows from
//     LDS, B = Q rows held in registers), online softmax in the S^T
//     accumulator layout (one head-row per lane pair), then
//     O^T += V^T . P^T with V^T fetched by ds_read_b64_tr_b16.
//   * The output goes back through LDS (the ring, once every wave is done
//     with it) so that each store instruction writes whole 64-byte row runs.
#include "lds_tile.hpp"
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kXcds = 8;
constexpr uint32_t kNoData = 0x80000000u;  // a buffer offset past every valid range

template <int I>
struct Idx {
  static constexpr int value = I;
};

// Waves per workgroup.  D = 64 (four waves per SIMD) runs workgroups of eight waves, two to a CU, so
// that each staged K/V block serves twice the queries of a four-wave tile (the causal shape, 4
// queries per wave at G = 8, measured 2-3% faster).  D = 128 keeps four waves, three workgroups to a
// CU: six- and eight-wave workgroups (two and one to a CU) measured 33% and 21% slower there.
template <int D, int G>
constexpr int waves_per_wg() {
  return D == 64 ? 8 : 4;
}

template <int D, int G>
__global__ __launch_bounds__((64 * waves_per_wg<D, G>()), (D == 64 ? 4 : (G <= 4 || G == 32) ? 3 : 1)) void window_fwd_mfma(WindowParams p, int tiles_per_seq, int n_tiles) {
  using Tile = SwizzledTile<D>;
  // D = 128 runs three workgroups per CU: a 3-slot ring (48 KB of LDS) and LDS addresses derived
  // by XOR from one base per operand instead of one register per read (168 VGPRs; G = 8 and 16
  // index their rows with a few more registers and stay at two).  D = 64 keeps four slots and
  // precomputed addresses (116 VGPRs, four waves per SIMD).
  constexpr int kRing = D == 128 ? 3 : 4;
  constexpr bool kXorAddr = D == 128;
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int NW = waves_per_wg<D, G>();
  constexpr int QW = 32 / G;                  // queries per wave
  constexpr int QT = NW * QW;                 // queries per tile
  constexpr int kSlot = 2 * Tile::kBytes;     // K tile + V tile
  // The slot's 1 KB DMA instructions (K tile, then V tile) are dealt out evenly over the waves: with
  // at most one wave per K instruction, wave w takes K instructions w h .. w h + h - 1 and the same
  // V instructions (the same source offsets); with twice as many waves, wave w takes instruction w.
  constexpr int kSlotDma = 2 * Tile::kDmaPerTile;
  constexpr int kDmaPerWave = kSlotDma / NW;
  constexpr int kSrcRegs = kDmaPerWave == 1 ? 1 : kDmaPerWave / 2;  // distinct source offsets
  static_assert(kSlotDma % NW == 0 && (kDmaPerWave == 1 || kDmaPerWave % 2 == 0), "DMA plan");
  constexpr int kStageBytes = 32 * 128;       // O staging per wave: 32 rows x 32 dims of fp32
  static_assert(kSlotDma >= NW, "every wave takes part in the stream");
  static_assert(NW * kStageBytes <= kRing * kSlot, "staging lives in the ring");
  __shared__ __attribute__((aligned(1024))) char ring[kRing * kSlot];

  // ---- which tile: XCD x takes tiles [x * per_xcd, (x + 1) * per_xcd) in dispatch order ----
  const int per_xcd = gridDim.x / kXcds;
  const int t = static_cast<int>(blockIdx.x % kXcds) * per_xcd + static_cast<int>(blockIdx.x / kXcds);
  if (t >= n_tiles) return;
  const int tq = t % tiles_per_seq;
  const int sg = t / tiles_per_seq;
  const int seq = sg % p.num_seqs;
  const int g = sg / p.num_seqs;
  const int a = p.cu_seqlens[seq];
  const int L = p.cu_seqlens[seq + 1] - a;
  const int Lq = min(L, p.max_seqlen);
  const int q_first = tq * QT;
  if (q_first >= Lq) return;  // workgroup-uniform
  const int q_last = min(Lq, q_first + QT) - 1;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int H = p.num_heads, Hkv = p.num_kv_heads;
  const int wl = p.window_left, wr = p.window_right;
  const float c = p.scale_log2;  // > 0 on this path

  // Keys of the tile and of this wave's queries.
  const int lo_wg = wl < 0 ? 0 : max(0, q_first - wl);
  const int hi_wg = wr < 0 ? L - 1 : min(L - 1, q_last + wr);
  const int nblk = (hi_wg - lo_wg + kBlockKeys) / kBlockKeys;
  const int wq0 = q_first + wave * QW;
  const bool wave_active = wq0 < Lq;
  const int wq1 = min(Lq, wq0 + QW) - 1;
  const int lo_w = wl < 0 ? 0 : max(0, wq0 - wl);
  const int hi_w = wr < 0 ? L - 1 : min(L - 1, wq1 + wr);
  const int my_q = wq0 + n / G;  // this lane's query (row n = query wq0 + n / G, head g G + n % G)
  const int head = g * G + n % G;

  // ---- K / V stream ----
  const uint32_t kv_tok = static_cast<uint32_t>(Hkv) * D * 2;  // bytes between tokens of k / v
  const uint32_t q_tok = static_cast<uint32_t>(H) * D * 2;     // bytes between tokens of q / o
  const int64_t kv0 = (static_cast<int64_t>(a) * Hkv + g) * D;
  const int64_t kv_span = static_cast<int64_t>(L - 1) * kv_tok + D * 2;
  const uint32_t kv_bytes = kv_span > 0x7fffffff ? 0x7fffffffu : static_cast<uint32_t>(kv_span);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const __bf16 *>(p.k) + kv0, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const __bf16 *>(p.v) + kv0, kv_bytes);
  auto dma_index = [&](int u) {  // wave-uniform; request 2k + t: K (t = 0) or V (t = 1) instruction w h + k
    if constexpr (kDmaPerWave == 1) return wave;
    else return (u & 1) * Tile::kDmaPerTile + wave * kSrcRegs + (u >> 1);
  };
  uint32_t kv_src[kSrcRegs];
#pragma unroll
  for (int u = 0; u < kSrcRegs; ++u) {
    int row, chunk;
    Tile::dma_source(dma_index(kDmaPerWave == 1 ? u : 2 * u) % Tile::kDmaPerTile, lane, row, chunk);
    kv_src[u] = static_cast<uint32_t>(row) * kv_tok + chunk * 16;
  }
  auto issue = [&](auto I, int blk) {  // block blk (any index) into ring slot I
    constexpr int off = decltype(I)::value * kSlot;
    const uint32_t row0 = blk < nblk ? static_cast<uint32_t>(lo_wg + blk * kBlockKeys) * kv_tok : kNoData;
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int d = dma_index(u);
      dma16(d < Tile::kDmaPerTile ? krs : vrs, ring + off + d * 1024, row0 + kv_src[kDmaPerWave == 1 ? 0 : u >> 1]);
    }
  };

  // This lane's sink: the G sinks of the KV head's query heads come through scalar loads (one address
  // for the whole wave) and each lane picks its own.  A vector load here would be waited for before
  // the Q rows and the first K/V blocks are requested, a memory round trip more per tile.
  float sink = 0.0f;
  if (p.sink_mode != kSinkNone) {
    const float *sg = p.sinks + g * G;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float sv = sg[i];
      sink = n % G == i ? sv : sink;
    }
  }

  // ---- Q operand in registers: row n, logical chunks h S .. h S + S - 1 (rows past Lq read 0) ----
  bf16x8 qf[S];
  {
    const __bf16 *qb = static_cast<const __bf16 *>(p.q) + (static_cast<int64_t>(a) * H + g * G) * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qb, static_cast<uint32_t>(Lq - 1) * q_tok + G * D * 2);
    const uint32_t qoff = static_cast<uint32_t>(my_q) * q_tok + (n % G) * D * 2 + h * D;
#pragma unroll
    for (int s = 0; s < S; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 16 * s, 0, 0));
  }
  issue(Idx<0>{}, 0);
  issue(Idx<1>{}, 1);
  if constexpr (kRing == 4) issue(Idx<2>{}, 2);

  // ---- per-lane LDS read addresses of the K rows (A operand) and V^T quads.  XOR addressing (D = 128;
  // bits 4..7 of every tile base are clear): row n's logical chunk h S + s at kbase ^ 16 s, V^T quads
  // at vbase ^ (64 db + 32 e) plus rows 8 e + 16 tt.  Otherwise one precomputed register per read
  // (koff, voff). ----
  const uint32_t ring_addr = lds_addr(ring);
  const int g16 = lane >> 4, i16 = lane & 15;
  const uint32_t kbase = ring_addr + Tile::offset(n, h * S);
  const uint32_t vbase = ring_addr + Tile::kBytes +
                         Tile::offset(4 * h + (i16 >> 2), 2 * (g16 & 1) + ((i16 & 3) >> 1)) + (i16 & 1) * 8;
  constexpr int kRow8 = 8 * Tile::kRowBytes;
  uint32_t koff[kXorAddr ? 1 : S];
  uint32_t voff[2][DB][2];
  if constexpr (!kXorAddr) {
#pragma unroll
    for (int s = 0; s < S; ++s) koff[s] = ring_addr + Tile::offset(n, h * S + s);
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
  }

  const float sink_raw = sink * kLog2e / c;  // the running max is kept in raw logit units
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  RowSoftmax rs;
  rs.m = p.sink_mode == kSinkNull ? sink_raw : kNegInf;
  rs.l = (p.sink_mode == kSinkNull && h == 0) ? 1.0f : 0.0f;  // the lane pair of a row splits l

  auto compute_block = [&](auto I, int kb0) {
    constexpr int off = decltype(I)::value * kSlot;
    u32x4 kf[S];
    if constexpr (kXorAddr) {
      uint32_t kb_ = kbase;  // opaque per block: the XORed addresses stay local
      asm volatile("" : "+v"(kb_));
#pragma unroll
      for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<off>(kb_ ^ (16u * s));
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<off>(koff[s]);
    }
    lgkm_fence<0>(kf);
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], st, 0, 0, 0);
    // V^T quads: read while the QK products and the softmax run (the K rows are dead by then).
    u32x2 vr[4 * DB];
    if constexpr (kXorAddr) {
      uint32_t vb = vbase;
      asm volatile("" : "+v"(vb));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        vr[db * 2] = ds_read_tr_b16<off>(vb ^ (64u * db));
        vr[db * 2 + 1] = ds_read_tr_b16<off + kRow8>(vb ^ (64u * db + Tile::kRow8Xor));
        vr[2 * DB + db * 2] = ds_read_tr_b16<off + 2 * kRow8>(vb ^ (64u * db));
        vr[2 * DB + db * 2 + 1] = ds_read_tr_b16<off + 3 * kRow8>(vb ^ (64u * db + Tile::kRow8Xor));
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 2; ++e) vr[(tt * DB + db) * 2 + e] = ds_read_tr_b16<off>(voff[tt][db][e]);
    }
    // Element r of lane (n, h) is key kb0 + 8*(r/4) + 4h + r%4 for this lane's row.
    if (p.sink_mode == kSinkKey0 && kb0 == 0 && h == 0) st[0] += sink_raw;
    const int kb1 = kb0 + kBlockKeys - 1;
    const bool interior = (wl < 0 || kb0 >= wq1 - wl) && (wr < 0 || kb1 <= wq0 + wr) && kb1 <= hi_wg;
    if (!interior) {
      const int lo_q = wl < 0 ? 0 : my_q - wl;
      const int hi_q = min(hi_wg, wr < 0 ? L - 1 : my_q + wr);
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

  // Step j: block j is in slot j % kRing.  This wave's requests younger than block j's are those of
  // blocks j + 1 .. j + kRing - 2 (block j + kRing - 1 is requested after the barrier), so one
  // fixed wait covers every step, the first included.
  auto step = [&](auto I, int j) {
    constexpr int i = decltype(I)::value;
    wait_vmcnt<(kRing - 2) * kDmaPerWave>();
    __builtin_amdgcn_s_barrier();
    issue(Idx<(i + kRing - 1) % kRing>{}, j + kRing - 1);  // the slot block j - 1 was read from
    const int kb0 = lo_wg + j * kBlockKeys;
    if (wave_active && kb0 <= hi_w && kb0 + kBlockKeys - 1 >= lo_w) compute_block(I, kb0);
  };
  for (int j = 0; j < nblk; j += kRing) {
    step(Idx<0>{}, j);
    if (j + 1 >= nblk) break;
    step(Idx<1>{}, j + 1);
    if (j + 2 >= nblk) break;
    step(Idx<2>{}, j + 2);
    if constexpr (kRing == 4) {
      if (j + 3 >= nblk) break;
      step(Idx<3>{}, j + 3);
    }
  }

  // ---- epilogue: o = acc / l and lse, through the ring once every wave is done with it ----
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  const float l_tot = halves_sum(rs.l);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t row0 = static_cast<int64_t>(a) * H + g * G;  // first (token, head) row of the group
  const __amdgpu_buffer_rsrc_t ors =
      make_rsrc(static_cast<__bf16 *>(p.o) + row0 * D, static_cast<uint32_t>(Lq - 1) * q_tok + G * D * 2);
  const uint32_t sbase = ring_addr + wave * kStageBytes;
  // write side: lane (n, h) holds dims 32 db + 8 j + 4 h .. +3 of row n = fp32 chunk 2 j + h;
  // 16-byte chunk c of staged row r sits at c ^ (r & 7) (conflict free both ways)
  const uint32_t wr0 = sbase + n * 128;
  // read side: lane l takes row 16 i + l / 4, fp32 chunks 2 (l % 4) and 2 (l % 4) + 1
  const int rl = lane >> 2, q4 = lane & 3;
  const uint32_t rd0 = sbase + rl * 128 + (((2 * q4) ^ (rl & 7)) << 4);
  const uint32_t rd1 = sbase + rl * 128 + (((2 * q4 + 1) ^ (rl & 7)) << 4);
  // Wave row r = 16 i + rl is query wq0 + r / G, head g G + r % G; as G divides 16 or 16 divides
  // G, its byte offset splits into a lane part (row rl) and a uniform part (16 i).  Rows past the
  // sequence fall outside the buffer and are dropped.
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
      buffer_store_b128_sgpr(__builtin_bit_cast(u32x4, v), ors, vlane, __builtin_amdgcn_readfirstlane(uni));
    }
  }
  if (p.lse && h == 0 && my_q < Lq)
    p.lse[(static_cast<int64_t>(a) + my_q) * H + head] = l_tot > 0.0f ? (rs.m * c + log2f(l_tot)) * kLn2 : kNegInf;
}

template <int D, int G>
hipError_t launch(const WindowParams &p, hipStream_t stream) {
  constexpr int NW = waves_per_wg<D, G>();
  constexpr int QT = NW * (32 / G);
  const int64_t tiles_per_seq = (p.max_seqlen + QT - 1) / QT;
  const int64_t n_tiles = tiles_per_seq * p.num_seqs * p.num_kv_heads;
  if (n_tiles <= 0) return hipSuccess;
  const int64_t per_xcd = (n_tiles + kXcds - 1) / kXcds;
  if (per_xcd * kXcds > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (trace_on())
    trace("window_fwd_mfma<D=%d, G=%d> grid=%lld block=%d tiles=%lld (%lld per sequence, %d queries each) seqs=%d "
          "kv_heads=%d window=(%d, %d) sink_mode=%d", D, G, static_cast<long long>(per_xcd * kXcds), 64 * NW,
          static_cast<long long>(n_tiles), static_cast<long long>(tiles_per_seq), QT, p.num_seqs, p.num_kv_heads,
          p.window_left, p.window_right, p.sink_mode);
  hipLaunchKernelGGL((window_fwd_mfma<D, G>), dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(64 * NW), 0, stream, p,
                     static_cast<int>(tiles_per_seq), static_cast<int>(n_tiles));
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
