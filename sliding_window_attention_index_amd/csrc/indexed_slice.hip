// Top-k index-gathered attention for few queries with long lists (the decode shape): one workgroup
// per (query, list slice) gathers the slice's cache rows once for every head of the query.
//
// Problem (DeepSeek-V4 CSA/HCA article, §4.1-§4.4): all query heads share one cache row per token,
// which is both the key and the value; the article gathers listed rows into shared memory so that
// the two products become dense GEMMs over the heads, then adds the per-head null-logit sink to the
// denominator.  Long lists are cut into contiguous slices whose partial softmax statistics are
// merged afterwards (nano-vllm XAttention offload note, technical details: per-chunk statistics
// combined into global ones), here by the merge kernel on the same stream.
//
// gfx950 mapping (workgroup = 4 waves; H = 32 NHG heads, NHG in {1, 2}):
//   * The slice is staged in passes of up to 256 list entries: each wave reads 64 entries (one per
//     lane), turns them into row byte offsets (an out-of-range stand-in for -1 and out-of-range
//     entries) and DMAs two 32-row tiles into LDS with buffer_load ... lds; every row of the pass
//     is fetched once for all heads.  Each wave's second tile is requested once the first four
//     tiles have landed, so that a workgroup computes its first half while the second streams in.
//   * Wave (hg, kg) owns head group hg (32 heads, their q in registers as the B operand) and every
//     KS-th tile of the pass (KS = 4 / NHG key groups): S^T = K . Q^T and O^T += V^T . P^T with
//     v_mfma_f32_32x32x16_bf16 and the online softmax of softmax_block.hpp.
//   * The key groups of a head group are combined through LDS (each wave writes its accumulator and
//     (m, l), then finalises a quarter of the query's heads, with stores that cover whole rows).
//   * Single slice: o and lse are written.  Several slices: the slice's fp32 partial (o_c, lse_c)
//     goes to the workspace for the merge kernel.
#include "lds_tile.hpp"
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kPassTiles = 8;                          // 32-entry tiles staged per pass
constexpr int kPass = kPassTiles * kBlockKeys;         // list entries per pass
constexpr uint32_t kBadRow = 0xfffff000u;              // staged offset of an entry that is not a row

__device__ __forceinline__ int ds_read_i32(uint32_t addr) {
  int r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr));
  return r;
}
// The same without the wait: the caller ties the result to an lgkmcnt wait (lgkm_fence).
__device__ __forceinline__ int ds_read_i32_nowait(uint32_t addr) {
  int r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ void ds_write_u32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v));
}
// 16-byte store written through to device scope (sc1): the partials are read by the next kernel, not
// by this one, and on the decode shape sending them on at once measured faster than leaving 16.8 MB
// dirty in the L2 caches until the end of the launch (16.8 vs 18.4 us).
__device__ __forceinline__ void store_b128_through(float *p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// Barrier after this wave's own LDS writes have completed (the DMA-filled tiles are covered by the
// caller's vmcnt wait).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int NHG>
__global__ __launch_bounds__(256, 2) void indexed_slice_mfma(IndexedParams p) {
  using Tile = SwizzledTile<D>;
  constexpr int S = D / 16;                 // MFMA steps over head_dim
  constexpr int DB = D / 32;                // 32-wide blocks of output dims
  constexpr int kDpb = Tile::kDmaPerTile;   // DMA instructions per tile
  constexpr int KS = 4 / NHG;               // waves sharing a head group
  constexpr int HPW = 8 * NHG;              // heads finalised per wave (a quarter of the query's)
  constexpr int C = D / 4;                  // 16-byte fp32 chunks of a head row
  constexpr int HPI = 64 / C;               // head rows per wave-wide step of the finalisation
  constexpr int CPL = HPW / HPI;            // steps (heads) per lane
  constexpr int kRowF = D * 4;              // bytes of one staged fp32 head row
  constexpr int kStage = 32 * kRowF;        // one wave's staged accumulator (32 heads)
  static_assert(NHG == 1 || NHG == 2, "head groups");
  static_assert(4 * kStage <= kPassTiles * Tile::kBytes, "staged accumulators fit in the tile area");
  static_assert(CPL >= 1, "steps");
  __shared__ __attribute__((aligned(1024))) char tiles[kPassTiles * Tile::kBytes];
  __shared__ __attribute__((aligned(16))) uint32_t tmask[2][kPassTiles];  // valid rows; rows that are cache row 0
  __shared__ __attribute__((aligned(16))) float stat[4][2][32];           // per wave: m (raw units), l per head

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int hg = wave / KS, kg = wave % KS;
  const int H = p.num_heads, N = p.kv_len, K = p.topk;
  const int64_t BM = static_cast<int64_t>(p.batch) * p.q_len;
  // Slice `part` of query bt; all slices of a query share blockIdx.x % 8 (one XCD).
  const int64_t bt = static_cast<int64_t>(blockIdx.x) % BM;
  const int part = static_cast<int>(static_cast<int64_t>(blockIdx.x) / BM);
  const int64_t b = bt / p.q_len;
  const int head0 = hg * 32;
  const bool partial = p.num_parts > 1;
  const bool key0 = p.sink_mode == kSinkKey0;
  const bool null_sink = p.sink_mode == kSinkNull;
  const float c = p.scale_log2;  // > 0 on this path

  // B operand of S^T: q[bt, head0 + n, h*D/2 + 8s .. +8].
  bf16x8 qf[S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + (bt * H + head0 + n) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 8);
  }
  const float sink_raw = p.sinks ? p.sinks[head0 + n] * kLog2e / c : 0.0f;  // raw logit units

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  RowSoftmax rs;  // the null sink is seeded once per head (key group 0) when there is one slice
  const bool seed = null_sink && !partial && kg == 0;
  rs.m = seed ? sink_raw : kNegInf;
  rs.l = (seed && h == 0) ? 1.0f : 0.0f;

  const int kb = part * p.part_len;
  const int ke = min(K, kb + p.part_len);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const __bf16 *>(p.kv) + b * static_cast<int64_t>(N) * D,
                                               static_cast<uint32_t>(N) * D * 2u);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.idx + bt * K, static_cast<uint32_t>(K) * 4u);
  const uint32_t ring_addr = lds_addr(tiles);
  const uint32_t mask_addr = lds_addr(&tmask[0][0]);

  // LDS operand addresses (bits 4..7 of every tile base are clear): K rows: row n, logical chunk
  // h*S + s at kbase ^ 16 s; V^T quads at vbase ^ (64 db + 32 e) plus rows 8 e + 16 tt.
  const uint32_t kbase = ring_addr + Tile::offset(n, h * S);
  uint32_t vbase;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int c2 = 2 * (g16 & 1) + ((i16 & 3) >> 1);
    vbase = ring_addr + Tile::offset(4 * h + (i16 >> 2), c2) + (i16 & 1) * 8;
  }
  constexpr int kRow8 = 8 * Tile::kRowBytes;

  // Tile t of the current pass: row r holds list entry r of the tile's 32 (bit r of its masks).
  auto compute = [&](int t) {
    const uint32_t vmask = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(ds_read_i32(mask_addr + 4 * t)));
    if (vmask == 0u) return;
    const uint32_t zmask =
        key0 ? static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(ds_read_i32(mask_addr + 4 * (kPassTiles + t)))) : 0u;
    uint32_t kb_ = kbase + t * Tile::kBytes;
    asm volatile("" : "+v"(kb_));
    u32x4 kf[S];
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<0>(kb_ ^ (16u * s));
    lgkm_fence<0>(kf);
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], st, 0, 0, 0);
    uint32_t vb = vbase + t * Tile::kBytes;
    asm volatile("" : "+v"(vb));
    u32x2 vr[4 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      vr[db * 2] = ds_read_tr_b16<0>(vb ^ (64u * db));
      vr[db * 2 + 1] = ds_read_tr_b16<kRow8>(vb ^ (64u * db + Tile::kRow8Xor));
      vr[2 * DB + db * 2] = ds_read_tr_b16<2 * kRow8>(vb ^ (64u * db));
      vr[2 * DB + db * 2 + 1] = ds_read_tr_b16<3 * kRow8>(vb ^ (64u * db + Tile::kRow8Xor));
    }
    if (zmask) bias_block(st, zmask, h, sink_raw);
    if (vmask != 0xffffffffu) mask_block(st, vmask, h);
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

  for (int c0 = kb; c0 < ke; c0 += kPass) {
    const int cend = min(ke, c0 + kPass);
    const int nblk = (cend - c0 + kBlockKeys - 1) / kBlockKeys;
    if (c0 != kb) lds_barrier();  // every wave is done with the previous pass's tiles
    // This lane's list entry: entry n of tile wave + 4h.
    const int j = c0 + kBlockKeys * (wave + 4 * h) + n;
    const int x = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lrs, static_cast<uint32_t>(j) * 4u, 0, 0));
    const bool valid = j < cend && x >= 0 && x < N;
    const uint32_t off = valid ? static_cast<uint32_t>(x) * Tile::kRowBytes : kBadRow;
    const uint64_t vbits = __ballot(valid);
    const uint64_t zbits = __ballot(valid && x == 0);
    if (lane == 0) {
      ds_write_u32(mask_addr + 4 * wave, static_cast<uint32_t>(vbits));
      ds_write_u32(mask_addr + 4 * (wave + 4), static_cast<uint32_t>(vbits >> 32));
      ds_write_u32(mask_addr + 4 * (kPassTiles + wave), static_cast<uint32_t>(zbits));
      ds_write_u32(mask_addr + 4 * (kPassTiles + wave + 4), static_cast<uint32_t>(zbits >> 32));
    }
    // Row offsets of every DMA of this wave's two tiles (lane l of DMA u fetches tile row
    // u * (1024 / row bytes) + l / (row bytes / 16)), gathered before the first DMA is issued.
    uint32_t src[2][kDpb];
#pragma unroll
    for (int tw = 0; tw < 2; ++tw)
#pragma unroll
      for (int u = 0; u < kDpb; ++u) {
        int row, chunk;
        Tile::dma_source(u, lane, row, chunk);
        src[tw][u] = static_cast<uint32_t>(__shfl(static_cast<int>(off), 32 * tw + row, 64)) | static_cast<uint32_t>(chunk * 16);
      }
    // Tiles 0..3 (each wave's first), then tiles 4..7, requested once the first four have landed:
    // every workgroup then finds its first half complete early and computes it while the second
    // half streams in (all requests at once would make every workgroup's tiles land together, at
    // the end of the whole gather).
    const bool has0 = wave < nblk, has1 = wave + 4 < nblk;
    if (has0) {
#pragma unroll
      for (int u = 0; u < kDpb; ++u) dma16(krs, tiles + wave * Tile::kBytes + u * 1024, src[0][u]);
    }
    wait_vmcnt<0>();
    lds_barrier();
    if (has1) {
#pragma unroll
      for (int u = 0; u < kDpb; ++u) dma16(krs, tiles + (wave + 4) * Tile::kBytes + u * 1024, src[1][u]);
    }
    const int first = min(nblk, 4);
    for (int t = kg; t < first; t += KS) compute(t);
    if (nblk > 4) {
      wait_vmcnt<0>();
      lds_barrier();
      for (int t = 4 + kg; t < nblk; t += KS) compute(t);
    }
  }

  // ---- combine the key groups of each head group through LDS (the tile area is free once every
  // wave is past its last tile), then each wave finalises heads [HPW wave, HPW wave + HPW) ----
  lds_barrier();
  {
    const float l_tot = halves_sum(rs.l);
    // Lane (n, h) holds dims 32 db + 8 j + 4 h .. +3 of head n: fp32 chunk 8 db + 2 j + h of the head
    // row, stored at chunk ^ (n & 7).
    const uint32_t wrow = ring_addr + wave * kStage + n * kRowF;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x4 w = {__float_as_uint(acc[db][4 * jj]), __float_as_uint(acc[db][4 * jj + 1]),
                         __float_as_uint(acc[db][4 * jj + 2]), __float_as_uint(acc[db][4 * jj + 3])};
        ds_write_b128<0>(wrow + (((8 * db + 2 * jj + h) ^ (n & 7)) << 4), w);
      }
    if (h == 0) {
      ds_write_u32(lds_addr(&stat[wave][0][n]), __float_as_uint(rs.m));
      ds_write_u32(lds_addr(&stat[wave][1][n]), __float_as_uint(l_tot));
    }
  }
  lds_barrier();

  // Finalised heads: in step q (0 .. CPL - 1) lane l takes head fh = HPW wave + HPI q + l / C (head
  // lh = fh % 32 of group fg), fp32 chunk l % C of its row (dims 4 (l % C) .. +3), so that every
  // store of the wave covers one contiguous stretch of rows.  The key groups' (m, l) of the wave's
  // heads are combined once, by lanes 0 .. HPW - 1 (one head each), and the weights are passed to
  // the lanes of each step by shuffles.
  const int ch = lane % C;
  const int fg = (HPW * wave) / 32;
  const int lh0 = (HPW * wave) % 32;
  float wk[KS], Lh;
  {
    const int j = min(lane, HPW - 1);
    float m_k[KS], l_k[KS];
    u32x2 st2[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
      st2[k] = u32x2{static_cast<uint32_t>(ds_read_i32_nowait(lds_addr(&stat[fg * KS + k][0][lh0 + j]))),
                     static_cast<uint32_t>(ds_read_i32_nowait(lds_addr(&stat[fg * KS + k][1][lh0 + j])))};
    lgkm_fence<0>(st2);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      m_k[k] = __uint_as_float(st2[k][0]);
      l_k[k] = __uint_as_float(st2[k][1]);
    }
    float M = m_k[0];
#pragma unroll
    for (int k = 1; k < KS; ++k) M = fmaxf(M, m_k[k]);
    Lh = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      wk[k] = m_k[k] == kNegInf ? 0.0f : fast_exp2((m_k[k] - M) * c);
      Lh = fmaf(wk[k], l_k[k], Lh);
    }
    const float inv = Lh > 0.0f ? 1.0f / Lh : 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) wk[k] *= inv;  // weight of key group k in the normalised output
    // natural-log lse of this slice (of the whole list with one slice); -inf when nothing counted
    Lh = Lh > 0.0f ? (M * c + log2f(Lh)) * kLn2 : kNegInf;
  }
  f32x4 o4[CPL];
  float lse[CPL];
  {
    u32x4 v[CPL * KS];
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int lh = lh0 + HPI * q + lane / C;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        v[q * KS + k] = ds_read_b128<0>(ring_addr + (fg * KS + k) * kStage + lh * kRowF + ((ch ^ (lh & 7)) << 4));
    }
    lgkm_fence<0>(v);
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int src = HPI * q + lane / C;
      f32x4 a4 = f32x4{};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float a = __shfl(wk[k], src, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = fmaf(a, __uint_as_float(v[q * KS + k][e]), a4[e]);
      }
      o4[q] = a4;
      lse[q] = __shfl(Lh, src, 64);
    }
  }
  const int64_t rh0 = bt * H + HPW * wave;  // first (query, head) row of this wave's heads
  const int64_t lrow = HPI * 0 + lane / C;  // row of this lane within each step

  auto store_out = [&](const f32x4 (&v)[CPL], const float (&lse_v)[CPL]) {
    __bf16 *ob = static_cast<__bf16 *>(p.o) + (rh0 + lrow) * D + 4 * ch;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const bf16x4 w = {static_cast<__bf16>(v[q][0]), static_cast<__bf16>(v[q][1]), static_cast<__bf16>(v[q][2]),
                        static_cast<__bf16>(v[q][3])};
      *reinterpret_cast<bf16x4 *>(ob + static_cast<int64_t>(HPI * q) * D) = w;
    }
    if (p.lse && ch == 0) {
#pragma unroll
      for (int q = 0; q < CPL; ++q) p.lse[rh0 + lrow + HPI * q] = lse_v[q];
    }
  };

  if (!partial) {
    store_out(o4, lse);
    return;
  }

  // ---- this slice's partial (part_o [S, B*M, H, D], part_lse [S, B*M, H]) ----
  const int64_t RH = BM * H;
  float *po = p.part_o + (static_cast<int64_t>(part) * RH + rh0 + lrow) * D + 4 * ch;
#pragma unroll
  for (int q = 0; q < CPL; ++q) store_b128_through(po + static_cast<int64_t>(HPI * q) * D, o4[q]);
  if (ch == 0) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) p.part_lse[part * RH + rh0 + lrow + HPI * q] = lse[q];
  }
}

template <int D, int NHG>
hipError_t launch(const IndexedParams &p, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(p.batch) * p.q_len * p.num_parts;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (trace_on())
    trace("indexed_slice_mfma<D=%d, head groups=%d> grid=%lld block=256 (rows=%lld x slices=%d of %d entries) "
          "kv_len=%d topk=%d sink_mode=%d", D, NHG, static_cast<long long>(blocks),
          static_cast<long long>(p.batch) * p.q_len, p.num_parts, p.part_len, p.kv_len, p.topk, p.sink_mode);
  hipLaunchKernelGGL((indexed_slice_mfma<D, NHG>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const IndexedParams &p, hipStream_t stream) {
  switch (p.num_heads) {
    case 32: return launch<D, 1>(p, stream);
    default: return launch<D, 2>(p, stream);
  }
}

}  // namespace

bool indexed_slice_supported(const IndexedParams &p) {
  const int64_t cache_bytes = static_cast<int64_t>(p.kv_len) * p.head_dim * 2;
  return p.scale_log2 > 0.0f && (p.head_dim == 64 || p.head_dim == 128) &&
         (p.num_heads == 32 || p.num_heads == 64) && cache_bytes < (int64_t(1) << 31) - 4096 &&
         static_cast<int64_t>(p.topk) * 4 < (int64_t(1) << 31);
}

hipError_t launch_indexed_slice(const IndexedParams &p, hipStream_t stream) {
  return p.head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sattn
