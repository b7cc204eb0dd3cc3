// Top-k index-gathered attention over an fp8 K=V cache (bf16 queries and outputs, MFMA).
//
// Problem: as the bf16 indexed kernel (DeepSeek-V4 CSA/HCA article, §4.1-§4.4: one shared cache
// row per token is the key and the value of every head, -1 marks unused list entries), over a
// cache quantised as the article's §5.3 describes for the compressed kv: the dims without rotary
// embedding in fp8, the rotary dims at higher precision.  Layout here (the article fixes none):
// a row of 128 dims holds its first 128 - RD dims as e4m3 codes (OCP fn) times one power-of-two
// fp32 scale per row, and its last RD dims (0 or 64) as bf16.
//
// gfx950 mapping: one wave64 per task (a query, 32 of its heads, one slice of its list), four
// independent waves per workgroup, as in the bf16 kernel.  Per 32-row block the wave DMAs into one
// of NT wave-private LDS slots: the rows' fp8 bytes (16-byte chunks swizzled per row), their
// scales and, when RD = 64, their bf16 rotary dims straight into a swizzled 32 x 64 tile.  The
// codes never go back to LDS as bf16: each operand is converted in registers
// (v_cvt_scalef32_pk_bf16_fp8) right before its MFMA.
//   * K (A operand of S^T = K . Q^T): lane (row n, half h) reads its row's codes and converts
//     them times the row's scale, so the logits are those of the dequantised rows.
//   * V^T (A operand of O^T = V^T . P^T): ds_read_b64_tr_b8 hands each lane 8 codes of one dim
//     from 8 rows; they are converted unscaled and each key's scale moves to its probability
//     instead (sum_j p_j (2^e_j c_jd) = sum_j (p_j 2^e_j) c_jd).
// A power of two times a bf16 or an e4m3 value is exact in bf16 (away from the subnormal range),
// so every product entering an MFMA equals the bf16 kernel's on the dequantised rows, in the
// same MFMA step mapping: the two kernels agree bit for bit.  The fp8 rows halve (RD = 0) or cut
// by a quarter (RD = 64) the bytes gathered per row.
#include "lds_tile.hpp"
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
// List entries staged per wave at a time: a whole prefill list (window plus top-k, up to 1024) with
// the 2-slot ring, so that a task streams its blocks without a restart; 512 with the 4-slot ring,
// whose workgroups would otherwise not fit two to a CU at rd = 0 (decode slices are short anyway).
template <int NT>
constexpr int idx_cap() {
  return NT == 2 ? 1024 : 512;
}
// Staged stand-in for an entry that is not a row: times any of the row sizes used here (4, 64, 128
// bytes, modulo 2^32), plus an in-row offset below 128, it lands at 0xfffe0000 or above, past the
// end of every buffer (all are < 2^31) and far from wrapping.
constexpr uint32_t kBadRow = 0x3ffffc00u;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS read of one dword the compiler does not see (it would otherwise wait for every DMA in
// flight before reading LDS); the result is tied to an lgkmcnt(0) wait.
__device__ __forceinline__ int ds_read_i32(uint32_t addr) {
  int r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr));
  return r;
}

// LDS read of one dword the compiler does not see, without a wait (lgkm_fence orders it).
__device__ __forceinline__ uint32_t ds_read_b32_raw(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// One 4-byte DMA per lane from rsrc + voffset into lds (+4 * lane).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, void *lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds), 4, voffset, 0, 0, 0);
}

// Eight e4m3 codes (two dwords) times a power-of-two scale -> eight bf16 (four dwords).
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true));
  return r;
}

template <int OFF>
__device__ __forceinline__ u32x2 ds_read_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int OFF>
__device__ __forceinline__ uint32_t ds_read_b32_off(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Eight LDS bytes per lane, transposed across lanes: in each group of 16 lanes, lane i receives as
// its byte e (e = 0..7) byte i % 8 of the 8 bytes that lane 2e + i / 8 of the group addresses.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr_b8(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// The block's probabilities as softmax_probs makes them (same exponentials, same sum into l):
// pb = bf16(p) for the bf16 rotary dims (when kPlain), pbs = bf16(p * scale of the key) for the
// fp8 dims.  Accumulator element r of lane (n, h) is key 8 (r / 4) + 4h + r % 4, whose scale is
// ks[r / 4][r % 4].
template <bool kPlain>
__device__ __forceinline__ void softmax_probs_scaled(const f32x16 &st, RowSoftmax &rs, float c, const u32x4 (&ks)[4],
                                                     bf16x8 (&pb)[2], bf16x8 (&pbs)[2]) {
  const float mc = rs.m == kNegInf ? 0.0f : rs.m * c;
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int r = 8 * t + j;
      const float e0 = fast_exp2(fmaf(st[r], c, -mc));
      const float e1 = fast_exp2(fmaf(st[r + 1], c, -mc));
      l0 += e0;
      l1 += e1;
      if constexpr (kPlain) {
        pb[t][j] = static_cast<__bf16>(e0);
        pb[t][j + 1] = static_cast<__bf16>(e1);
      }
      pbs[t][j] = static_cast<__bf16>(e0 * __uint_as_float(ks[r >> 2][r & 3]));
      pbs[t][j + 1] = static_cast<__bf16>(e1 * __uint_as_float(ks[r >> 2][(r & 3) + 1]));
    }
  }
  rs.l += l0 + l1;
}

template <int I>
struct Slot {
  static constexpr int value = I;
};

template <int RD, int NT>
__global__ __launch_bounds__(256) void indexed_fp8_mfma(IndexedParams p) {
  constexpr int D = 128;
  constexpr int S = D / 16;   // MFMA steps over head_dim
  constexpr int DB = D / 32;  // 32-wide blocks of output dims
  using T64 = SwizzledTile<64>;
  constexpr int D8 = D - RD;                        // fp8 bytes per row
  constexpr int DB8 = D8 / 32;                      // output dim blocks read from fp8 codes
  constexpr int kChunks8 = D8 / 16;                 // 16-byte chunks of an fp8 row
  constexpr int kRowsPer256 = 256 / D8;             // fp8 rows per 256 bytes of LDS
  constexpr int kF8Bytes = kBlockKeys * D8;         // a block's fp8 bytes
  constexpr int kRopeBytes = RD ? T64::kBytes : 0;  // a block's rotary tile
  constexpr int kScaleOff = kRopeBytes + kF8Bytes;  // a block's scales (64 lanes x 4 bytes)
  constexpr int kSlotBytes = kScaleOff + 256;
  constexpr int kF8Dma = kF8Bytes / 1024;
  constexpr int kRopeDma = RD ? T64::kDmaPerTile : 0;
  constexpr int kDpb = kF8Dma + kRopeDma + 1;       // DMA instructions per block
  static_assert(RD == 0 || RD == 64, "rotary dims");
  static_assert((NT & (NT - 1)) == 0 && NT >= 2 && NT <= 4, "ring size");
  static_assert(kSlotBytes % 256 == 0, "slot bases keep bits 4..7 clear");
  static_assert(kSlotBytes >= 32 * 128, "the epilogue stages 32 rows of 128 bytes in a slot");
  __shared__ __attribute__((aligned(1024))) char ring[4][NT * kSlotBytes];
  constexpr int kIdxCap = idx_cap<NT>();
  __shared__ __attribute__((aligned(16))) int32_t lists[4][kIdxCap];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5;   // half of the wave: which 8 dims of each MFMA step / which key quads
  const int n = lane & 31;   // key row (A operand) / head (B operand and outputs)
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

  // B operand of S^T: q[bt, head0 + n, 16s + 8h .. +8], the bf16 kernel's MFMA steps: steps
  // 0 .. D8 / 16 - 1 cover the fp8 dims, the rest the rotary dims.
  bf16x8 qf[S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + (bt * H + head0 + n) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 16);
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
  // This batch row's cache parts and this query's list through bounds-checked buffer resources.
  const __amdgpu_buffer_rsrc_t f8rs = make_rsrc(static_cast<const uint8_t *>(p.kv) + b * static_cast<int64_t>(N) * D8,
                                                static_cast<uint32_t>(N) * D8);
  const __amdgpu_buffer_rsrc_t scrs = make_rsrc(p.kv_scale + b * static_cast<int64_t>(N), static_cast<uint32_t>(N) * 4u);
  const __amdgpu_buffer_rsrc_t rprs =
      make_rsrc(RD ? static_cast<const __bf16 *>(p.kv_rope) + b * static_cast<int64_t>(N) * RD : p.kv,
                RD ? static_cast<uint32_t>(N) * RD * 2u : 0u);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.idx + bt * K, static_cast<uint32_t>(K) * 4u);
  char *const wring = ring[wave];
  const uint32_t ring_addr = lds_addr(wring);
  int32_t *list = lists[wave];
  const uint32_t list_addr = lds_addr(list);

  // Slot layout: [rotary tile (RD = 64)][fp8 rows][scales].  Row r of a block (list entry r) keeps
  // its fp8 16-byte chunk q at chunk q ^ ((r / kRowsPer256) % kChunks8) of its D8 bytes: 16
  // consecutive rows reading one logical chunk, and the 8 rows x 2 chunks of a transposed read,
  // then fall in distinct banks.  DMA instruction u of the fp8 bytes fills LDS bytes 1024 u ..;
  // lane l fetches the chunk that belongs at byte 1024 u + 16 l.
  auto f8_swz = [](int r) { return (r / kRowsPer256) & (kChunks8 - 1); };
  constexpr int kReads = kF8Dma + kRopeDma + 1;
  auto issue_block = [&](int j) {
    char *slot = wring + (j & (NT - 1)) * kSlotBytes;
    const uint32_t lbase = list_addr + static_cast<uint32_t>(j * kBlockKeys) * 4u;
    uint32_t xs[kReads];
#pragma unroll
    for (int u = 0; u < kF8Dma; ++u) xs[u] = ds_read_b32_raw(lbase + ((1024 * u + 16 * lane) / D8) * 4);
#pragma unroll
    for (int u = 0; u < kRopeDma; ++u) {
      int row, chunk;
      T64::dma_source(u, lane, row, chunk);
      xs[kF8Dma + u] = ds_read_b32_raw(lbase + row * 4);
    }
    xs[kReads - 1] = ds_read_b32_raw(lbase + (lane & (kBlockKeys - 1)) * 4);
    lgkm_fence<0>(xs);
#pragma unroll
    for (int u = 0; u < kF8Dma; ++u) {
      const int pos = 1024 * u + 16 * lane;
      const int row = pos / D8;
      const int chunk = ((pos % D8) / 16) ^ f8_swz(row);
      dma16(f8rs, slot + kRopeBytes + u * 1024, xs[u] * D8 + chunk * 16);
    }
#pragma unroll
    for (int u = 0; u < kRopeDma; ++u) {
      int row, chunk;
      T64::dma_source(u, lane, row, chunk);
      const uint32_t x = xs[kF8Dma + u];
      dma16(rprs, slot + u * 1024, x * (RD * 2) + chunk * 16);
    }
    {
      const uint32_t x = xs[kReads - 1];
      dma4(scrs, slot + kScaleOff, lane < kBlockKeys ? x * 4u : 0xfffff000u);
    }
  };

  // Per-lane LDS offsets inside a slot (the XORed terms stay inside one row).
  //  K, fp8 step s: bytes 16 s + 8 h .. + 7 of row n at (k8 ^ 16 s).  K, rotary step s (RD = 64):
  //  logical chunk 2 (s - D8 / 16) + h of row n of the tile at (kr ^ 32 (s - D8 / 16)).
  const uint32_t k8 = kRopeBytes + n * D8 + 16 * f8_swz(n) + 8 * h;
  const uint32_t kr = T64::offset(n, h);
  //  V^T, fp8 dims 32 db + (lane & 31): lane (group g16, index i16) reads 8 bytes of row
  //  8 (i16 / 8) + 4h + (i16 / 2) % 4 (+ 16 tt), dims 32 db + 16 (g16 % 2) + 8 (i16 % 2) ..: after
  //  the transposed read, lane (n, h) holds the codes of dim 32 db + n for keys 4h .. 4h + 3 and
  //  8 + 4h .. 8 + 4h + 3 (+ 16 tt), the key order of the probabilities' B operand.
  uint32_t v8;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int row = 8 * (i16 >> 3) + 4 * h + ((i16 >> 1) & 3);
    v8 = kRopeBytes + row * D8 + 16 * ((g16 & 1) ^ f8_swz(row)) + 8 * (i16 & 1);
  }
  //  V^T, rotary dims (RD = 64): the quads of the bf16 kernel's D = 64 tile.
  uint32_t voff;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int c2 = 2 * (g16 & 1) + ((i16 & 3) >> 1);
    voff = T64::offset(4 * h + (i16 >> 2), c2) + (i16 & 1) * 8;
  }
  constexpr int kRow8 = 8 * T64::kRowBytes;
  constexpr int kRows16 = 16 * D8;  // 16 fp8 rows (the same swizzle)

  // Every LDS operand address of a block, computed once for slot 0 (the XORed chunk addresses in
  // registers); the slot is the reads' immediate offset (the block loop runs over compile-time
  // slots).
  constexpr int kS8 = D8 / 16;  // MFMA steps over fp8 dims
  constexpr int kSR = S - kS8 > 0 ? S - kS8 : 1;
  uint32_t a_k8[kS8], a_kr[kSR], a_v8[DB8], a_vr[2][2];
#pragma unroll
  for (int s = 0; s < kS8; ++s) a_k8[s] = (ring_addr + k8) ^ (16u * s);
#pragma unroll
  for (int s = 0; s < kSR; ++s) a_kr[s] = (ring_addr + kr) ^ (32u * s);
  const uint32_t a_ks = ring_addr + kScaleOff + 4 * n, a_ps = ring_addr + kScaleOff + 16 * h;
#pragma unroll
  for (int db = 0; db < DB8; ++db) a_v8[db] = (ring_addr + v8) ^ (32u * db);
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2) {
    a_vr[d2][0] = (ring_addr + voff) ^ (64u * d2);
    a_vr[d2][1] = (ring_addr + voff) ^ (64u * d2 + T64::kRow8Xor);
  }

  auto compute = [&](auto I, int j) {
    constexpr int so = decltype(I)::value * kSlotBytes;  // the slot's byte offset
    // K operand and the scales: this lane's row (K) and its keys' (probabilities).
    u32x2 k8r[kS8];
    u32x4 krr[kSR];
#pragma unroll
    for (int s = 0; s < kS8; ++s) k8r[s] = ds_read_b64<so>(a_k8[s]);
    if constexpr (RD) {
#pragma unroll
      for (int s = 0; s < S - kS8; ++s) krr[s] = ds_read_b128<so>(a_kr[s]);
    }
    int ksb[1];
    ksb[0] = static_cast<int>(ds_read_b32_off<so>(a_ks));
    u32x4 ks[4];
    ks[0] = ds_read_b128<so>(a_ps);
    ks[1] = ds_read_b128<so + 32>(a_ps);
    ks[2] = ds_read_b128<so + 64>(a_ps);
    ks[3] = ds_read_b128<so + 96>(a_ps);
    uint32_t xr[1];
    xr[0] = ds_read_b32_raw(list_addr + (j * kBlockKeys + n) * 4);
    lgkm_fence<0>(k8r);
    if constexpr (RD) lgkm_fence<0>(krr);
    lgkm_fence<0>(ksb);
    lgkm_fence<0>(ks);
    lgkm_fence<0>(xr);
    const uint32_t vmask = static_cast<uint32_t>(__ballot(xr[0] != kBadRow));  // tile row n's entry is a row
    if (vmask == 0u) return;
    const uint32_t zmask = key0 ? static_cast<uint32_t>(__ballot(xr[0] == 0u)) : 0u;  // ... and it is row 0
    const float kscale = __int_as_float(ksb[0]);
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const u32x4 kf = s < kS8 ? fp8x8_to_bf16(k8r[s][0], k8r[s][1], kscale) : krr[s < kS8 ? 0 : s - kS8];
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[s], st, 0, 0, 0);
    }
    // V^T operands.
    u32x2 v8r[2 * DB8];
#pragma unroll
    for (int db = 0; db < DB8; ++db) {
      v8r[db] = ds_read_tr_b8<so>(a_v8[db]);
      v8r[DB8 + db] = ds_read_tr_b8<so + kRows16>(a_v8[db]);
    }
    constexpr int kV16 = RD ? 8 : 1;
    u32x2 vr[kV16];
    if constexpr (RD) {
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        vr[d2 * 2] = ds_read_tr_b16<so>(a_vr[d2][0]);
        vr[d2 * 2 + 1] = ds_read_tr_b16<so + kRow8>(a_vr[d2][1]);
        vr[4 + d2 * 2] = ds_read_tr_b16<so + 2 * kRow8>(a_vr[d2][0]);
        vr[4 + d2 * 2 + 1] = ds_read_tr_b16<so + 3 * kRow8>(a_vr[d2][1]);
      }
    }
    // Accumulator element r of lane (n, h) is key 8*(r/4) + 4h + r%4 of head n.
    if (zmask) bias_block(st, zmask, h, sink_raw);
    if (vmask != 0xffffffffu) mask_block(st, vmask, h);
    float alpha;
    if (softmax_need_rescale(rs, block_max(st), c, alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    bf16x8 pb[2], pbs[2];
    softmax_probs_scaled<RD != 0>(st, rs, c, ks, pb, pbs);
    lgkm_fence<0>(v8r);
    if constexpr (RD) lgkm_fence<0>(vr);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db < DB8) {
          const u32x2 w = v8r[tt * DB8 + db];
          const u32x4 av = fp8x8_to_bf16(w[0], w[1], 1.0f);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pbs[tt], acc[db], 0, 0, 0);
        } else {
          const int d2 = db - DB8;
          const u32x2 ra = vr[(tt * 2 + d2) * 2], rb = vr[(tt * 2 + d2) * 2 + 1];
          const u32x4 av = {ra[0], ra[1], rb[0], rb[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[tt], acc[db], 0, 0, 0);
        }
      }
  };

  for (int c0 = kb; c0 < ke; c0 += kIdxCap) {
    const int cend = min(ke, c0 + kIdxCap);
    const int nblk = (cend - c0 + kBlockKeys - 1) / kBlockKeys;
    asm volatile("" ::: "memory");  // the previous chunk's list reads (inline asm) stay before these stores
    // Stage the chunk's entries (kBadRow for -1, out-of-range entries and past the chunk's end).
    // Every DMA of the previous chunk has been waited for, so nothing reads or fills LDS meanwhile.
    {
      constexpr int kLoads = kIdxCap / 256;
      u32x4 v[kLoads];
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        v[i] = (256 * i < nblk * kBlockKeys)
                   ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   lrs, static_cast<uint32_t>(c0 + 256 * i + 4 * lane) * 4u, 0, 0))
                   : u32x4{};
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int j = 256 * i + 4 * lane;
        if (j < nblk * kBlockKeys) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int x = static_cast<int>(v[i][e]);
            w[e] = c0 + j + e < cend && x >= 0 && x < N ? static_cast<uint32_t>(x) : kBadRow;
          }
          *reinterpret_cast<u32x4 *>(list + j) = w;
        }
      }
    }
    wave_lds_sync();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NT; ++j)
      if (j < nblk) issue_block(j);
    auto step = [&](auto I, int j) {  // block j, in ring slot I = j % NT
      // This wave's DMAs younger than block j's: those of the next min(NT - 1, nblk - 1 - j) blocks.
      const int younger = min(NT - 1, nblk - 1 - j);
      if (younger == 3) wait_vmcnt<3 * kDpb>();
      else if (younger == 2) wait_vmcnt<2 * kDpb>();
      else if (younger == 1) wait_vmcnt<kDpb>();
      else wait_vmcnt<0>();
      compute(I, j);
      if (j + NT < nblk) issue_block(j + NT);  // the slot's reads are done (lgkm fences above)
    };
    for (int j = 0; j < nblk; j += NT) {
      step(Slot<0>{}, j);
      if (j + 1 >= nblk) break;
      step(Slot<1>{}, j + 1);
      if constexpr (NT == 4) {
        if (j + 2 >= nblk) break;
        step(Slot<2>{}, j + 2);
        if (j + 3 >= nblk) break;
        step(Slot<3>{}, j + 3);
      }
    }
  }

  // Epilogue: o = acc / l, lse = ln(2) * (m + log2 l).  Lane (n, h) holds dims 32db + 8j + 4h + {0..3}
  // of head n.  Each 32-dim block goes through the wave's first ring slot as scaled fp32 (16-byte
  // chunk q of row r at q ^ (r & 7)) and comes back as 8 consecutive dims per lane.
  const float l_tot = halves_sum(rs.l);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (rs.m * c + log2f(l_tot)) * kLn2 : kNegInf;
  const int64_t row0 = partial ? (static_cast<int64_t>(part) * BM + bt) * H + head0 : bt * H + head0;
  const int rl = lane >> 2, q4 = lane & 3;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 w = {__float_as_uint(acc[db][4 * j] * inv), __float_as_uint(acc[db][4 * j + 1] * inv),
                       __float_as_uint(acc[db][4 * j + 2] * inv), __float_as_uint(acc[db][4 * j + 3] * inv)};
      ds_write_b128<0>(ring_addr + n * 128 + (((2 * j + h) ^ (n & 7)) << 4), w);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + rl;  // head head0 + r
      u32x4 x[2];
      x[0] = ds_read_b128<0>(ring_addr + r * 128 + (((2 * q4) ^ (r & 7)) << 4));
      x[1] = ds_read_b128<0>(ring_addr + r * 128 + (((2 * q4 + 1) ^ (r & 7)) << 4));
      lgkm_fence<0>(x);
      const int64_t e0 = (row0 + r) * D + 32 * db + 8 * q4;
      if (partial) {
        *reinterpret_cast<u32x4 *>(p.part_o + e0) = x[0];
        *reinterpret_cast<u32x4 *>(p.part_o + e0 + 4) = x[1];
      } else {
        const bf16x8 v = {static_cast<__bf16>(__uint_as_float(x[0][0])), static_cast<__bf16>(__uint_as_float(x[0][1])),
                          static_cast<__bf16>(__uint_as_float(x[0][2])), static_cast<__bf16>(__uint_as_float(x[0][3])),
                          static_cast<__bf16>(__uint_as_float(x[1][0])), static_cast<__bf16>(__uint_as_float(x[1][1])),
                          static_cast<__bf16>(__uint_as_float(x[1][2])), static_cast<__bf16>(__uint_as_float(x[1][3]))};
        *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(p.o) + e0) = v;
      }
    }
  }
  if (h == 0) {
    if (partial) p.part_lse[row0 + n] = lse_v;
    else if (p.lse) p.lse[row0 + n] = lse_v;
  }
}

template <int RD, int NT>
hipError_t launch(const IndexedParams &p, hipStream_t stream) {
  const int n_hg = p.num_heads / 32;
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * n_hg * p.num_parts;
  const int64_t blocks = (tasks + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (trace_on())
    trace("indexed_fp8_mfma<rope_dims=%d, NT=%d> grid=%lld block=256 (rows=%lld x head groups=%d x slices=%d of %d "
          "entries) kv_len=%d topk=%d sink_mode=%d", RD, NT, static_cast<long long>(blocks),
          static_cast<long long>(p.batch) * p.q_len, p.num_heads / 32, p.num_parts, p.part_len, p.kv_len, p.topk,
          p.sink_mode);
  hipLaunchKernelGGL((indexed_fp8_mfma<RD, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool indexed_fp8_supported(const IndexedParams &p) {
  // One batch row's cache parts and list are addressed with 32-bit buffer offsets.
  const int64_t row_bytes = (p.head_dim - p.rope_dims) + 2 * p.rope_dims;
  return p.scale_log2 > 0.0f && p.head_dim == 128 && (p.rope_dims == 0 || p.rope_dims == 64) &&
         p.num_heads % 32 == 0 && static_cast<int64_t>(p.kv_len) * row_bytes < (int64_t(1) << 31) - 4096 &&
         static_cast<int64_t>(p.topk) * 4 < (int64_t(1) << 31);
}

hipError_t launch_indexed_fp8(const IndexedParams &p, hipStream_t stream) {
  // Few tasks (decode-like): one workgroup per CU anyway, so each wave keeps four blocks in flight.
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * (p.num_heads / 32) * p.num_parts;
  const bool deep = tasks < 4096;
  if (p.rope_dims == 64) return deep ? launch<64, 4>(p, stream) : launch<64, 2>(p, stream);
  return deep ? launch<0, 4>(p, stream) : launch<0, 2>(p, stream);
}

}  // namespace sattn
