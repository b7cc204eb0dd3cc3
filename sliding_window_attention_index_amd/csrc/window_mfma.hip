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
//   * A workgroup owns one KV head and a tile of QT consecutive queries of one
//     sequence; each of its 4 waves owns 32 rows = 32/G queries x G heads (the
//     G query heads of one KV head share every K/V element, so they fill the
//     MFMA N dimension).
//   * The workgroup walks 32-key blocks from the first to the last key any of
//     its queries can see; K and V blocks are loaded cooperatively into
//     double-buffered LDS tiles (one barrier per block).  A wave skips blocks
//     outside its own band and applies element masks only on blocks that are
//     not entirely inside the window of all its queries.
//   * Per block: S^T = K . Q^T (v_mfma_f32_32x32x16_bf16, A from LDS with
//     16-byte reads, B = Q held in registers), online softmax in the S^T
//     accumulator layout (one head-row per lane pair, v_permlane32_swap for
//     the max), then O^T += V^T . P^T with V^T fetched by ds_read_b64_tr_b16.
//   * Tiles are mapped to workgroup ids so that neighbouring query tiles of
//     one (sequence, KV head), which share most of their keys, land on the
//     same XCD (workgroups are dealt round-robin over the 8 XCDs).
#include "sattn_device.hpp"
#include "sattn_kernels.hpp"

namespace sattn {
namespace {

constexpr int kBlockKeys = 32;
constexpr int kPad = 16;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

template <int D, int G>
__global__ __launch_bounds__(256) void window_fwd_mfma(WindowParams p, int tiles_per_seq, int total_tiles) {
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int LDSS = D + kPad;
  constexpr int QW = 32 / G;       // queries per wave
  constexpr int QT = 4 * QW;       // queries per workgroup
  constexpr int CH = kBlockKeys * D / 8 / 256;  // 16-byte chunks per thread per K (or V) block
  static_assert(CH >= 1, "tile too small for the block");
  __shared__ __attribute__((aligned(16))) __bf16 ktile[2][kBlockKeys * LDSS];
  __shared__ __attribute__((aligned(16))) __bf16 vtile[2][kBlockKeys * LDSS];

  // XCD-aware tile id: consecutive logical tiles share an XCD.
  const int per_xcd = gridDim.x / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total_tiles) return;
  const int seq = logical / tiles_per_seq;
  const int tile = logical % tiles_per_seq;
  const int g = blockIdx.y;
  const int a = p.cu_seqlens[seq];
  const int L = p.cu_seqlens[seq + 1] - a;
  const int Lq = min(L, p.max_seqlen);  // queries past max_seqlen are not computed; keys still are
  const int q_first = tile * QT;
  if (q_first >= Lq) return;  // whole workgroup
  const int wl = p.window_left, wr = p.window_right;
  const int q_last = min(Lq, q_first + QT) - 1;
  const int lo_wg = wl < 0 ? 0 : max(0, q_first - wl);
  const int hi_wg = wr < 0 ? L - 1 : min(L - 1, q_last + wr);
  const int nblk = (hi_wg - lo_wg + kBlockKeys) / kBlockKeys;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int h = lane >> 5, n = lane & 31;
  const int H = p.num_heads, Hkv = p.num_kv_heads;

  // Rows of this wave: row n = query (wq0 + n / G), head g*G + n % G.
  const int wq0 = q_first + wave * QW;
  const bool wave_active = wq0 < Lq;
  const int wq1 = min(Lq, wq0 + QW) - 1;
  const int lo_w = wl < 0 ? 0 : max(0, wq0 - wl);
  const int hi_w = wr < 0 ? L - 1 : min(L - 1, wq1 + wr);
  const int my_q = wq0 + n / G;
  const int my_head = g * G + n % G;
  const bool row_real = my_q < Lq;
  const bool key0 = p.sink_mode == kSinkKey0;
  const bool null_sink = p.sink_mode == kSinkNull;
  const float sink2 = p.sink_mode != kSinkNone ? p.sinks[my_head] * kLog2e : 0.0f;

  bf16x8 qf[S];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) +
                         (static_cast<int64_t>(a + my_q) * H + my_head) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = row_real ? *reinterpret_cast<const bf16x8 *>(qrow + s * 8) : bf16x8{};
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = null_sink ? sink2 : kNegInf;
  float l_part = (null_sink && h == 0) ? 1.0f : 0.0f;

  // Cooperative K/V block loads: chunk c -> key row c / (D/8), 8 dims at (c % (D/8)) * 8.
  const __bf16 *kg = static_cast<const __bf16 *>(p.k) + (static_cast<int64_t>(a) * Hkv + g) * D;
  const __bf16 *vg = static_cast<const __bf16 *>(p.v) + (static_cast<int64_t>(a) * Hkv + g) * D;
  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;
  u32x4 kreg[CH], vreg[CH];
  auto load_block = [&](int blk) {
    const int kb0 = lo_wg + blk * kBlockKeys;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = tid + 256 * u;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int j = kb0 + row;
      if (j <= hi_wg) {
        kreg[u] = *reinterpret_cast<const u32x4 *>(kg + j * tok_stride + col);
        vreg[u] = *reinterpret_cast<const u32x4 *>(vg + j * tok_stride + col);
      } else {
        kreg[u] = u32x4{};
        vreg[u] = u32x4{};
      }
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = tid + 256 * u;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&ktile[buf][row * LDSS + col]) = kreg[u];
      *reinterpret_cast<u32x4 *>(&vtile[buf][row * LDSS + col]) = vreg[u];
    }
  };

  load_block(0);
  const int g16 = lane >> 4, i16 = lane & 15;
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    store_block(buf);
    __syncthreads();
    if (blk + 1 < nblk) load_block(blk + 1);
    const int kb0 = lo_wg + blk * kBlockKeys;
    if (!wave_active || kb0 > hi_w || kb0 + kBlockKeys - 1 < lo_w) continue;

    const __bf16 *kt = ktile[buf];
    const __bf16 *vt = vtile[buf];
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kt + n * LDSS + h * (D / 2) + s * 8);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
    }
    // Element r of lane (n, h) is key kb0 + 8*(r/4) + 4h + r%4 for this lane's row.
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = st[r] * p.scale_log2;
    if (key0 && kb0 == 0 && h == 0) t[0] += sink2;
    const int kb1 = kb0 + kBlockKeys - 1;
    const bool interior = (wl < 0 || kb0 >= wq1 - wl) && (wr < 0 || kb1 <= wq0 + wr) && kb1 <= hi_wg;
    if (!interior) {
      const int lo_q = wl < 0 ? 0 : my_q - wl;
      const int hi_q = wr < 0 ? L - 1 : min(L - 1, my_q + wr);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kb0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (j < lo_q || j > hi_q || j > hi_wg) t[r] = kNegInf;
      }
    }
    float bm = t[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bm = fmaxf(bm, t[r]);
    const float m_new = fmaxf(m_run, halves_max(bm));
    if (__ballot(m_new > m_run + kRescaleThreshold)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
    }
    const float mref = m_run == kNegInf ? 0.0f : m_run;
    bf16x8 pb[2];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(t[r] - mref);
      ps += e;
      pb[r >> 3][r & 7] = static_cast<__bf16>(e);
    }
    l_part += ps;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int ka = 16 * tt + 4 * h + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * (g16 & 1) + (i16 & 3) * 4;
        const bf16x4 ra = lds_read_tr(vt + ka * LDSS + col);
        const bf16x4 rb = lds_read_tr(vt + (ka + 8) * LDSS + col);
        const bf16x8 av = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[tt], acc[db], 0, 0, 0);
      }
    }
  }

  if (!row_real) return;
  const float l_tot = halves_sum(l_part);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t orow = static_cast<int64_t>(a + my_q) * H + my_head;
  __bf16 *dst = static_cast<__bf16 *>(p.o) + orow * D + 4 * h;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x4 v = {static_cast<__bf16>(acc[db][4 * i] * inv), static_cast<__bf16>(acc[db][4 * i + 1] * inv),
                        static_cast<__bf16>(acc[db][4 * i + 2] * inv), static_cast<__bf16>(acc[db][4 * i + 3] * inv)};
      *reinterpret_cast<bf16x4 *>(dst + 32 * db + 8 * i) = v;
    }
  if (p.lse && h == 0) p.lse[orow] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
}

template <int D, int G>
hipError_t launch(const WindowParams &p, hipStream_t stream) {
  constexpr int QT = 4 * (32 / G);
  const int tiles_per_seq = (p.max_seqlen + QT - 1) / QT;
  const int64_t total = static_cast<int64_t>(tiles_per_seq) * p.num_seqs;
  const int64_t grid_x = (total + kXcds - 1) / kXcds * kXcds;
  if (grid_x > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((window_fwd_mfma<D, G>), dim3(static_cast<unsigned>(grid_x), p.num_kv_heads), dim3(256), 0,
                     stream, p, tiles_per_seq, static_cast<int>(total));
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
  return (p.head_dim == 64 || p.head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32);
}

hipError_t launch_window_mfma(const WindowParams &p, hipStream_t stream) {
  return p.head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sattn
