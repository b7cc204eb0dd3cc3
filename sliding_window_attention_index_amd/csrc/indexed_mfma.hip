// Top-k index-gathered attention over a single shared K=V head (bf16, MFMA).
//
// Problem (DeepSeek-V4 CSA/HCA article, §4.1-§4.4): every query has a list of
// absolute cache rows (-1 = unused); all query heads share one cache row per
// token, which is both the key and the value.  The article's kernel gathers
// a chunk of listed rows into shared memory so that both products become
// dense GEMMs, then runs the online softmax over chunks and adds the
// per-head null-logit sink to the denominator at the end.
//
// gfx950 mapping (one wave64 per task = one query, 32 of its heads, one slice
// of its list; the four waves of a workgroup are independent):
//   * The slice's list entries are staged in a wave-private LDS area; the
//     wave then streams its 32-row blocks into a private ring of NT swizzled
//     LDS tiles with buffer_load ... lds (each instruction fetches four whole
//     rows; a row that is not listed is read out of bounds and lands as
//     zeros).  NT blocks are in flight at once and no register holds a row
//     in transit; the wave waits for its own DMAs only (vmcnt), no barrier.
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: A = 16-byte reads of the
//     tile rows (keys), B = the 32 heads' q in registers; the accumulator
//     holds 16 keys of one head per lane and the other 16 in lane ^ 32.
//   * O^T += V^T . P^T: the same tile read with ds_read_b64_tr_b16 (the cache
//     row is the value too), P^T = the S^T accumulator rounded to bf16.
//   * Online softmax with a lazy rescale (only when the running maximum grows
//     by more than 2^8); the output goes through LDS so that it is written as
//     whole rows (the 32 heads of a query are one contiguous stretch).
//
// Block-mass instantiation (kMass): the same gather and S^T product, then
// instead of the softmax and PV each logit becomes exp2(s * c - lse * log2 e)
// against a given log-sum-exp and the lane sums are written per block of
// `block_keys` list entries (nano-vllm XAttention offload note, technical
// details: the third stage normalises with the merged global statistics and
// sums per block).  No V read, no accumulator, no epilogue.
#include "lds_tile.hpp"
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"
#include "softmax_block.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kIdxCap = 1024;  // list entries staged per wave at a time
constexpr uint32_t kBadRow = 0xfffff000u;  // staged offset of an entry that is not a row: past every buffer

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
// The same without the wait: the caller ties the result to an lgkmcnt wait (lgkm_fence).
__device__ __forceinline__ int ds_read_i32_nowait(uint32_t addr) {
  int r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

template <int I>
struct Slot {
  static constexpr int value = I;
};

template <int D, int NT, bool kMass>
__global__ __launch_bounds__(256) void indexed_fwd_mfma(IndexedParams p) {
  using Tile = SwizzledTile<D>;
  constexpr int S = D / 16;                  // MFMA steps over head_dim
  constexpr int DB = D / 32;                 // 32-wide blocks of output dims
  constexpr int kDpb = Tile::kDmaPerTile;    // DMA instructions per 32-row block
  static_assert((NT & (NT - 1)) == 0 && NT >= 2 && NT <= 4, "ring size");
  __shared__ __attribute__((aligned(1024))) char tiles[4][NT * Tile::kBytes];
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
  const bool null_sink = !kMass && !partial && p.sink_mode == kSinkNull;

  // B operand of S^T: q[bt, head0 + n, 16s + 8h .. +8] (logical chunk 2s + h of the row).  MFMA
  // step s sums dims 16s .. 16s + 15; the fp8-cache kernel uses the same steps, so that both sum
  // a row's products in one order.
  bf16x8 qf[S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + (bt * H + head0 + n) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 16);
  }
  const float c = p.scale_log2;  // > 0 on this path
  const float sink_raw = p.sinks ? p.sinks[head0 + n] * kLog2e / c : 0.0f;  // raw logit units

  f32x16 acc[kMass ? 1 : DB];  // unused by the block-mass instantiation
  if constexpr (!kMass) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  }
  // Block mass: -lse in base 2 (an lse of -inf makes every valid entry +inf, as exp(s - lse)
  // does; a finite stand-in keeps the masked -inf logits at exp2(-inf) = 0), and this lane's
  // share of the current block's sum.
  float neg_lse2 = 0.0f, bin_sum = 0.0f;
  if constexpr (kMass) {
    const float l = p.lse_in[bt * H + head0 + n];
    neg_lse2 = l == kNegInf ? 3.0e38f : -l * kLog2e;
  }
  RowSoftmax rs;
  rs.m = null_sink ? sink_raw : kNegInf;
  rs.l = (null_sink && h == 0) ? 1.0f : 0.0f;  // the pair of lanes sharing a head splits l

  const int kb = part * p.part_len;
  const int ke = min(K, kb + p.part_len);
  // This batch row's cache and this query's list through bounds-checked buffer resources.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const __bf16 *>(p.kv) + b * static_cast<int64_t>(N) * D,
                                               static_cast<uint32_t>(N) * D * 2u);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.idx + bt * K, static_cast<uint32_t>(K) * 4u);
  char *ring = tiles[wave];
  const uint32_t ring_addr = lds_addr(ring);
  int32_t *list = lists[wave];
  const uint32_t list_addr = lds_addr(list);

  // DMA instruction u of a block fills the tile's bytes [1024 u, 1024 (u + 1)), i.e. tile rows
  // u R .. u R + R - 1 (R = 1024 / row bytes); lane l serves row u R + g, g = l / (row bytes / 16),
  // and fetches its swizzled chunk (Tile::dma_source).  Tile row u R + g holds list entry g U + u
  // of the block (U = DMA instructions per block): any assignment of entries to rows gives the same
  // attention, and this one gives each lane U consecutive entries, read with 16-byte LDS loads.
  constexpr int kR = 1024 / Tile::kRowBytes;  // rows per DMA instruction
  constexpr int kU = kDpb;                    // DMA instructions per block (kR * kU == 32)
  static_assert(kR * kU == kBlockKeys && kU % 4 == 0, "block geometry");
  const int dg = lane / (Tile::kRowBytes / 16);
  auto entry_of_row = [](int r) { return (r % kR) * kU + r / kR; };
  auto issue_block = [&](int j) {  // block j of the staged chunk into ring slot j % NT
    char *dst = ring + (j & (NT - 1)) * Tile::kBytes;
    u32x4 e4[kU / 4];
#pragma unroll
    for (int v = 0; v < kU / 4; ++v) e4[v] = ds_read_b128<0>(list_addr + (j * kBlockKeys + dg * kU + 4 * v) * 4);
    lgkm_fence<0>(e4);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      int row, chunk;
      Tile::dma_source(u, lane, row, chunk);  // row == u * kR + dg
      dma16(krs, dst + u * 1024, e4[u / 4][u % 4] | static_cast<uint32_t>(chunk * 16));  // kBadRow stays out of range
    }
  };

  // LDS operand addresses (bits 4..7 of every tile base are clear, see the window kernel):
  // K rows: row n, logical chunk 2s + h at kbase ^ 32 s; V^T quads at vbase ^ (64 db + 32 e) plus
  // rows 8 e + 16 tt.
  const uint32_t kbase = ring_addr + Tile::offset(n, h);
  uint32_t vbase;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int c2 = 2 * (g16 & 1) + ((i16 & 3) >> 1);
    vbase = ring_addr + Tile::offset(4 * h + (i16 >> 2), c2) + (i16 & 1) * 8;
  }
  constexpr int kRow8 = 8 * Tile::kRowBytes;
  // Every LDS operand address of a block, computed once: the XORed chunk addresses of slot 0 in
  // registers (this kernel has registers to spare at two waves per SIMD), the slot as the reads'
  // immediate offset (the block loop runs over compile-time slots).
  uint32_t kaddr[kMass ? 1 : S], vaddr[DB][2];
#pragma unroll
  for (int s = 0; s < (kMass ? 1 : S); ++s) kaddr[s] = kbase ^ (32u * s);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    vaddr[db][0] = vbase ^ (64u * db);
    vaddr[db][1] = vbase ^ (64u * db + Tile::kRow8Xor);
  }

  // Block j from ring slot I (attention: a compile-time slot, the reads' immediate offset) or
  // `slot` (block mass, which keeps one address register and XORs at every block: there the
  // unrolled slot loop measured slower).  The attention instantiation reads tile row n's list entry
  // with the K operand (one LDS round trip for both) and skips the block once it is known to hold
  // no row; the block-mass instantiation gets the masks from its caller.
  auto compute = [&](auto I, int slot, int j, uint32_t vmask, uint32_t zmask) {
    constexpr int off = decltype(I)::value * Tile::kBytes;
    u32x4 kf[S];
    if constexpr (kMass) {
      uint32_t kb_ = kbase + slot * Tile::kBytes;  // opaque per block: the XORed addresses stay local
      asm volatile("" : "+v"(kb_));
#pragma unroll
      for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<0>(kb_ ^ (32u * s));
      lgkm_fence<0>(kf);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) kf[s] = ds_read_b128<off>(kaddr[s]);
      uint32_t xr[1];
      xr[0] = static_cast<uint32_t>(ds_read_i32_nowait(list_addr + (j * kBlockKeys + entry_of_row(n)) * 4));
      lgkm_fence<0>(kf);
      lgkm_fence<0>(xr);
      vmask = static_cast<uint32_t>(__ballot(xr[0] != kBadRow));  // tile row n's entry is a row
      if (vmask == 0u) return;
      zmask = key0 ? static_cast<uint32_t>(__ballot(xr[0] == 0u)) : 0u;  // ... and it is row 0
    }
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], st, 0, 0, 0);
    if constexpr (kMass) {
      if (zmask) bias_block(st, zmask, h, sink_raw);
      if (vmask != 0xffffffffu) mask_block(st, vmask, h);
      float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        e0 += fast_exp2(fmaf(st[r], c, neg_lse2));
        e1 += fast_exp2(fmaf(st[r + 1], c, neg_lse2));
      }
      bin_sum += e0 + e1;
    } else {
      u32x2 vr[4 * DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        vr[db * 2] = ds_read_tr_b16<off>(vaddr[db][0]);
        vr[db * 2 + 1] = ds_read_tr_b16<off + kRow8>(vaddr[db][1]);
        vr[2 * DB + db * 2] = ds_read_tr_b16<off + 2 * kRow8>(vaddr[db][0]);
        vr[2 * DB + db * 2 + 1] = ds_read_tr_b16<off + 3 * kRow8>(vaddr[db][1]);
      }
      // Accumulator element r of lane (n, h) is key 8*(r/4) + 4h + r%4 of head n.
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
    }
  };

  // Block mass: blocks of block_keys entries are whole runs of 32-entry tiles (block_keys % 32 == 0
  // and every slice starts on a block boundary); `bin_left` tiles of the current block remain.
  // Finished blocks' masses wait in registers (up to kMassBuf) and are written together, so that a
  // task's masses reach memory in whole lines rather than one 4-byte store per block.
  constexpr int kMassBuf = 16;
  const int tiles_per_bin = kMass ? p.block_keys / kBlockKeys : 1;
  int bin = kMass ? kb / p.block_keys : 0;  // first block not yet written
  int bin_left = tiles_per_bin;
  float mbuf[kMass ? kMassBuf : 1];
  int nbuf = 0;
  auto flush_masses = [&]() {
    if (h == 0) {
      float *dst = p.mass + (bt * H + head0 + n) * p.n_bins + bin;
#pragma unroll
      for (int k = 0; k < kMassBuf; ++k)
        if (k < nbuf) dst[k] = mbuf[k];
    }
    bin += nbuf;
    nbuf = 0;
  };
  for (int c0 = kb; c0 < ke; c0 += kIdxCap) {
    const int cend = min(ke, c0 + kIdxCap);
    const int nblk = (cend - c0 + kBlockKeys - 1) / kBlockKeys;
    asm volatile("" ::: "memory");  // the previous chunk's list reads (inline asm) stay before these stores
    // Stage the chunk's entries as byte offsets of their rows (kBadRow for -1, out-of-range
    // entries and past the chunk's end).  Every DMA of the previous chunk has been waited for, so
    // nothing reads or fills LDS meanwhile.
    {
      // 16 bytes per lane per load, every load issued before any is used.
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
            w[e] = c0 + j + e < cend && x >= 0 && x < N ? static_cast<uint32_t>(x) * Tile::kRowBytes : kBadRow;
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
      if constexpr (kMass) {
        const uint32_t x = static_cast<uint32_t>(ds_read_i32(list_addr + (j * kBlockKeys + entry_of_row(n)) * 4));
        const uint32_t vmask = static_cast<uint32_t>(__ballot(x != kBadRow));  // tile row n's entry is a row
        const uint32_t zmask = key0 ? static_cast<uint32_t>(__ballot(x == 0u)) : 0u;  // ... and it is row 0
        if (vmask != 0u) compute(I, j & (NT - 1), j, vmask, zmask);
      } else {
        compute(I, j & (NT - 1), j, 0u, 0u);
      }
      if constexpr (kMass) {
        if (--bin_left == 0 || (j == nblk - 1 && cend == ke)) {  // the block ends with this tile
          const float tot = halves_sum(bin_sum);
#pragma unroll
          for (int k = 0; k < kMassBuf; ++k) mbuf[k] = k == nbuf ? tot : mbuf[k];
          if (++nbuf == kMassBuf) flush_masses();
          bin_sum = 0.0f;
          bin_left = tiles_per_bin;
        }
      }
      if (j + NT < nblk) issue_block(j + NT);  // the slot's reads are done (lgkm fences in compute)
    };
    if constexpr (kMass) {
      for (int j = 0; j < nblk; ++j) step(Slot<0>{}, j);
    } else {
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
  }

  if constexpr (kMass) flush_masses();
  if constexpr (!kMass) {
    // Epilogue: o = acc / l, lse = ln(2) * (m + log2 l).  Lane (n, h) holds dims 32db + 8j + 4h + {0..3}
    // of head n.  Each 32-dim block goes through the wave's first tile as scaled fp32 (16-byte chunk
    // q of row r at q ^ (r & 7)) and comes back as 8 consecutive dims per lane.
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
}

template <int D, int NT, bool kMass>
hipError_t launch(const IndexedParams &p, hipStream_t stream) {
  const int n_hg = p.num_heads / 32;
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * n_hg * p.num_parts;
  const int64_t blocks = (tasks + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (trace_on())
    trace("indexed_fwd_mfma<D=%d, NT=%d, mass=%d> grid=%lld block=256 tasks=%lld (rows=%lld x head groups=%d x "
          "slices=%d of %d entries) kv_len=%d topk=%d sink_mode=%d", D, NT, kMass ? 1 : 0, static_cast<long long>(blocks),
          static_cast<long long>(tasks), static_cast<long long>(p.batch) * p.q_len, n_hg, p.num_parts, p.part_len,
          p.kv_len, p.topk, p.sink_mode);
  hipLaunchKernelGGL((indexed_fwd_mfma<D, NT, kMass>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
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
  // Few tasks (decode-like): one workgroup per CU anyway, so each wave keeps four blocks in flight.
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * (p.num_heads / 32) * p.num_parts;
  const bool deep = tasks < 4096;
  if (p.head_dim == 128) return deep ? launch<128, 4, false>(p, stream) : launch<128, 2, false>(p, stream);
  return deep ? launch<64, 4, false>(p, stream) : launch<64, 2, false>(p, stream);
}

bool block_mass_mfma_supported(const IndexedParams &p) {
  return indexed_mfma_supported(p) && p.block_keys % kBlockKeys == 0;
}

hipError_t launch_block_mass_mfma(const IndexedParams &p, hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(p.batch) * p.q_len * (p.num_heads / 32) * p.num_parts;
  const bool deep = tasks < 4096;
  if (p.head_dim == 128) return deep ? launch<128, 4, true>(p, stream) : launch<128, 2, true>(p, stream);
  return deep ? launch<64, 4, true>(p, stream) : launch<64, 2, true>(p, stream);
}

}  // namespace sattn
