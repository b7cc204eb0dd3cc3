// C ABI of libsattn: host-side validation and kernel dispatch.
//
// Every argument is checked here before anything is enqueued; an invalid call
// returns a status and touches neither the device nor the stream.  All
// launches go to the caller's stream and nothing synchronises (the nano-vllm
// offload note's lesson: kernels that run on a stream other than the one the
// producer's event was waited on read unfinished data).
#include "sattn.h"

#include <cstdint>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sattn_kernels.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(sattn_dtype t) { return t == SATTN_BF16 || t == SATTN_F32; }
bool valid_sink(sattn_sink_mode m) {
  return m == SATTN_SINK_NONE || m == SATTN_SINK_KEY0_BIAS || m == SATTN_SINK_NULL_LOGIT;
}

sattn_status head_dim_status(int32_t d) {
  if (d <= 0) return SATTN_ERR_SHAPE;
  if (d % 8 != 0 || d > 256) return SATTN_ERR_UNSUPPORTED;
  return SATTN_OK;
}

sattn_status launch_status(hipError_t e) { return e == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH; }

// Split-K workspace layout: part_o [S, R, H, D] fp32, then part_lse [S, R, H] fp32,
// each starting on a 256-byte boundary.
size_t part_o_bytes(int64_t parts, int64_t rows, int64_t heads, int64_t dim) {
  return round_up(static_cast<size_t>(parts * rows * heads * dim) * sizeof(float), 256);
}
size_t part_lse_bytes(int64_t parts, int64_t rows, int64_t heads) {
  return round_up(static_cast<size_t>(parts * rows * heads) * sizeof(float), 256);
}

}  // namespace

namespace sattn {

bool trace_on() {
  static const bool on = [] {
    const char *e = getenv("SATTN_TRACE");
    return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
  }();
  return on;
}

void trace(const char *fmt, ...) {
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[sattn] %s\n", line);
}

}  // namespace sattn

extern "C" {

int sattn_abi_version(void) { return SATTN_ABI_VERSION; }

const char *sattn_status_string(sattn_status s) {
  switch (s) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case SATTN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case SATTN_ERR_DTYPE: return "unknown dtype";
    case SATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case SATTN_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case SATTN_ERR_WORKSPACE: return "split-K workspace missing, misaligned or too small";
    case SATTN_ERR_LAUNCH: return "kernel launch failed";
    case SATTN_ERR_ARG: return "invalid enum value or option";
    case SATTN_ERR_SCRATCH_LIMIT: return "split-K partials larger than the library's fixed scratch";
  }
  return "unknown status";
}

size_t sattn_indexed_workspace_size(int32_t batch, int32_t q_len, int32_t num_heads, int32_t head_dim,
                                    int32_t num_splits) {
  if (num_splits <= 1 || batch <= 0 || q_len <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
  const int64_t rows = static_cast<int64_t>(batch) * q_len;
  return part_o_bytes(num_splits, rows, num_heads, head_dim) + part_lse_bytes(num_splits, rows, num_heads);
}

sattn_status sattn_window_fwd(const sattn_window_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_dtype(a->dtype)) return SATTN_ERR_DTYPE;
  if (!valid_sink(a->sink_mode)) return SATTN_ERR_ARG;
  if (a->num_seqs < 0 || a->total_tokens < 0 || a->max_seqlen < 0 || a->num_heads <= 0 ||
      a->num_kv_heads <= 0 || a->num_heads % a->num_kv_heads != 0)
    return SATTN_ERR_SHAPE;
  if (sattn_status s = head_dim_status(a->head_dim)) return s;
  if (!isfinite(a->softmax_scale)) return SATTN_ERR_ARG;
  if (a->total_tokens == 0 || a->num_seqs == 0) return SATTN_OK;
  if (a->max_seqlen == 0) return SATTN_ERR_SHAPE;
  if (!a->q || !a->k || !a->v || !a->o || !a->cu_seqlens) return SATTN_ERR_NULL_PTR;
  if (a->sink_mode != SATTN_SINK_NONE && !a->sinks) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) ||
      !aligned4(a->cu_seqlens) || (a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return SATTN_ERR_ALIGNMENT;

  sattn::WindowParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = a->cu_seqlens;
  p.num_seqs = a->num_seqs;
  p.max_seqlen = a->max_seqlen;
  p.num_heads = a->num_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.group = a->num_heads / a->num_kv_heads;
  p.window_left = a->window_left;
  p.window_right = a->window_right;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.sinks = a->sink_mode != SATTN_SINK_NONE ? a->sinks : nullptr;
  p.sink_mode = a->sink_mode;
  if (a->dtype == SATTN_BF16 && sattn::window_mfma_supported(p))
    return launch_status(sattn::launch_window_mfma(p, stream));
  return launch_status(sattn::launch_window_valu(p, a->dtype == SATTN_F32 ? sattn::kF32 : sattn::kBF16, stream));
}

sattn_status sattn_build_topk_idxs(const sattn_build_idx_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (a->batch < 0 || a->q_len < 0 || a->window < 1 || a->n_comp < 0) return SATTN_ERR_SHAPE;
  if (a->ratio < 0 || (a->ratio == 0 && a->n_comp > 0)) return SATTN_ERR_ARG;
  if (static_cast<int64_t>(a->window) + a->n_comp > INT32_MAX) return SATTN_ERR_SHAPE;
  if (a->batch == 0 || a->q_len == 0) return SATTN_OK;
  if (!a->out || !a->start_pos) return SATTN_ERR_NULL_PTR;
  if (!aligned4(a->out) || !aligned4(a->start_pos)) return SATTN_ERR_ALIGNMENT;
  sattn::BuildIdxParams p;
  p.out = a->out;
  p.start_pos = a->start_pos;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.window = a->window;
  p.ratio = a->ratio;
  p.n_comp = a->n_comp;
  return launch_status(sattn::launch_build_topk_idxs(p, stream));
}

sattn_status sattn_merge_lse(const sattn_merge_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_dtype(a->out_dtype)) return SATTN_ERR_DTYPE;
  if (a->sink_mode != SATTN_SINK_NONE && a->sink_mode != SATTN_SINK_NULL_LOGIT) return SATTN_ERR_ARG;
  if (a->num_parts < 0 || a->rows < 0 || a->num_heads <= 0) return SATTN_ERR_SHAPE;
  if (sattn_status s = head_dim_status(a->head_dim)) return s;
  if (a->rows == 0) return SATTN_OK;
  if (!a->o || (a->num_parts > 0 && (!a->part_o || !a->part_lse))) return SATTN_ERR_NULL_PTR;
  if (a->sink_mode == SATTN_SINK_NULL_LOGIT && !a->sinks) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->o) || (a->part_o && !aligned4(a->part_o)) || (a->part_lse && !aligned4(a->part_lse)) ||
      (a->lse && !aligned4(a->lse)))
    return SATTN_ERR_ALIGNMENT;
  sattn::MergeParams p;
  p.part_o = a->part_o;
  p.part_lse = a->part_lse;
  p.num_parts = a->num_parts;
  p.rows = a->rows;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.sinks = a->sinks;
  p.sink_mode = a->sink_mode;
  p.out_type = a->out_dtype == SATTN_F32 ? sattn::kF32 : sattn::kBF16;
  p.o = a->o;
  p.lse = a->lse;
  return launch_status(sattn::launch_merge(p, stream));
}

}  // extern "C"

namespace sattn {

// sattn_indexed_fwd with the split-K workspace given separately (the caller's buffer, or the
// library's fixed scratch for sattn_indexed_fwd_noalloc); a->workspace and a->workspace_bytes are
// not read here.
sattn_status indexed_fwd_with_workspace(const sattn_indexed_args *a, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_dtype(a->dtype)) return SATTN_ERR_DTYPE;
  if (!valid_sink(a->sink_mode)) return SATTN_ERR_ARG;
  if (a->batch < 0 || a->q_len < 0 || a->num_heads <= 0 || a->kv_len < 0 || a->topk < 0)
    return SATTN_ERR_SHAPE;
  if (sattn_status s = head_dim_status(a->head_dim)) return s;
  if (!isfinite(a->softmax_scale)) return SATTN_ERR_ARG;
  if (a->num_splits < 1 || a->num_splits > (a->topk > 0 ? a->topk : 1)) return SATTN_ERR_ARG;
  const int64_t rows = static_cast<int64_t>(a->batch) * a->q_len;
  if (rows == 0) return SATTN_OK;
  if (rows > INT32_MAX) return SATTN_ERR_UNSUPPORTED;
  if (!a->q || !a->o || (a->topk > 0 && !a->topk_idxs) || (a->kv_len > 0 && !a->kv)) return SATTN_ERR_NULL_PTR;
  if (a->sink_mode != SATTN_SINK_NONE && !a->sinks) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->q) || !aligned16(a->o) || (a->kv && !aligned16(a->kv)) ||
      (a->topk_idxs && !aligned4(a->topk_idxs)) || (a->lse && !aligned4(a->lse)) ||
      (a->sinks && !aligned4(a->sinks)))
    return SATTN_ERR_ALIGNMENT;

  sattn::IndexedParams p = {};
  p.q = a->q;
  p.kv = a->kv;
  p.idx = a->topk_idxs;
  p.o = a->o;
  p.lse = a->lse;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.kv_len = a->kv_len;
  p.topk = a->topk;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.sinks = a->sink_mode != SATTN_SINK_NONE ? a->sinks : nullptr;
  p.sink_mode = a->sink_mode;
  p.num_parts = 1;
  p.part_len = a->topk;
  p.part_o = nullptr;
  p.part_lse = nullptr;

  int parts = 1;
  if (a->num_splits > 1) {
    const size_t need = sattn_indexed_workspace_size(a->batch, a->q_len, a->num_heads, a->head_dim, a->num_splits);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need)
      return SATTN_ERR_WORKSPACE;
    p.part_len = (a->topk + a->num_splits - 1) / a->num_splits;
    parts = (a->topk + p.part_len - 1) / p.part_len;  // slices that hold at least one entry
  }
  const int elem = a->dtype == SATTN_F32 ? sattn::kF32 : sattn::kBF16;
  const bool mfma = a->dtype == SATTN_BF16;
  // Few queries with long lists (the decode shape): one workgroup per (query, slice) gathers each
  // listed row once for all heads.
  const bool by_slice = mfma && sattn::indexed_slice_supported(p) && rows * parts < 4096;
  if (parts == 1) {
    p.part_len = a->topk > 0 ? a->topk : 1;
    if (by_slice) return launch_status(sattn::launch_indexed_slice(p, stream));
    if (mfma && sattn::indexed_mfma_supported(p)) return launch_status(sattn::launch_indexed_mfma(p, stream));
    return launch_status(sattn::launch_indexed_valu(p, elem, stream));
  }
  char *ws = static_cast<char *>(workspace);
  p.num_parts = parts;
  p.part_o = reinterpret_cast<float *>(ws);
  p.part_lse = reinterpret_cast<float *>(ws + part_o_bytes(a->num_splits, rows, a->num_heads, a->head_dim));
  hipError_t e = by_slice ? sattn::launch_indexed_slice(p, stream)
                 : (mfma && sattn::indexed_mfma_supported(p)) ? sattn::launch_indexed_mfma(p, stream)
                                                             : sattn::launch_indexed_valu(p, elem, stream);
  if (e != hipSuccess) return SATTN_ERR_LAUNCH;
  sattn::MergeParams m;
  m.part_o = p.part_o;
  m.part_lse = p.part_lse;
  m.num_parts = parts;
  m.rows = static_cast<int>(rows);
  m.num_heads = a->num_heads;
  m.head_dim = a->head_dim;
  m.sinks = p.sinks;
  m.sink_mode = a->sink_mode == SATTN_SINK_NULL_LOGIT ? SATTN_SINK_NULL_LOGIT : SATTN_SINK_NONE;
  m.out_type = elem;
  m.o = a->o;
  m.lse = a->lse;
  return launch_status(sattn::launch_merge(m, stream));
}

}  // namespace sattn

extern "C" {

sattn_status sattn_indexed_fwd(const sattn_indexed_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  return sattn::indexed_fwd_with_workspace(a, a->workspace, a->workspace_bytes, stream);
}

sattn_status sattn_block_mass(const sattn_block_mass_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_dtype(a->dtype)) return SATTN_ERR_DTYPE;
  if (!valid_sink(a->sink_mode)) return SATTN_ERR_ARG;
  if (a->batch < 0 || a->q_len < 0 || a->num_heads <= 0 || a->kv_len < 0 || a->topk < 0 || a->block_keys < 1)
    return SATTN_ERR_SHAPE;
  if (sattn_status s = head_dim_status(a->head_dim)) return s;
  if (!isfinite(a->softmax_scale)) return SATTN_ERR_ARG;
  const int64_t rows = static_cast<int64_t>(a->batch) * a->q_len;
  if (rows == 0 || a->topk == 0) return SATTN_OK;  // no block to write
  if (rows > INT32_MAX) return SATTN_ERR_UNSUPPORTED;
  if (!a->q || !a->topk_idxs || !a->lse || !a->mass || (a->kv_len > 0 && !a->kv)) return SATTN_ERR_NULL_PTR;
  if (a->sink_mode == SATTN_SINK_KEY0_BIAS && !a->sinks) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->q) || (a->kv && !aligned16(a->kv)) || !aligned4(a->topk_idxs) || !aligned4(a->lse) ||
      !aligned4(a->mass) || (a->sinks && !aligned4(a->sinks)))
    return SATTN_ERR_ALIGNMENT;

  sattn::IndexedParams p = {};
  p.q = a->q;
  p.kv = a->kv;
  p.idx = a->topk_idxs;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.kv_len = a->kv_len;
  p.topk = a->topk;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  // Only the key-0 bias touches a block; a null sink belongs to none.
  p.sinks = a->sink_mode == SATTN_SINK_KEY0_BIAS ? a->sinks : nullptr;
  p.sink_mode = a->sink_mode == SATTN_SINK_KEY0_BIAS ? SATTN_SINK_KEY0_BIAS : SATTN_SINK_NONE;
  p.lse_in = a->lse;
  p.mass = a->mass;
  p.block_keys = a->block_keys;
  p.n_bins = static_cast<int>((static_cast<int64_t>(a->topk) + a->block_keys - 1) / a->block_keys);
  p.num_parts = 1;
  p.part_len = a->topk;
  if (a->dtype == SATTN_BF16 && sattn::block_mass_mfma_supported(p)) {
    // Blocks need no merge, so a list is cut into slices of whole blocks whenever that brings the
    // wave count near 4096 (a few per SIMD): decode-like shapes have few queries and long lists.
    const int64_t tasks = rows * (a->num_heads / 32);
    int64_t per = (4096 + tasks - 1) / tasks;  // slices wanted per list
    if (per > p.n_bins) per = p.n_bins;
    if (per > 1) {
      const int64_t bins_per_part = (p.n_bins + per - 1) / per;
      p.part_len = static_cast<int>(bins_per_part * a->block_keys);
      p.num_parts = static_cast<int>((p.n_bins + bins_per_part - 1) / bins_per_part);
    }
    return launch_status(sattn::launch_block_mass_mfma(p, stream));
  }
  return launch_status(sattn::launch_block_mass_valu(p, a->dtype == SATTN_F32 ? sattn::kF32 : sattn::kBF16, stream));
}

sattn_status sattn_compress_pool(const sattn_compress_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_dtype(a->dtype)) return SATTN_ERR_DTYPE;
  if (a->overlap != 0 && a->overlap != 1) return SATTN_ERR_ARG;
  if (a->batch < 0 || a->seq_len < 0 || a->ratio < 1) return SATTN_ERR_SHAPE;
  if (a->head_dim <= 0) return SATTN_ERR_SHAPE;
  if (a->head_dim % 8 != 0) return SATTN_ERR_UNSUPPORTED;
  const int64_t n_out = a->seq_len / a->ratio;
  if (a->out_batch_stride < n_out) return SATTN_ERR_SHAPE;
  if (a->batch == 0 || n_out == 0) return SATTN_OK;
  if (!a->kv || !a->score || !a->ape || !a->out) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->kv) || !aligned16(a->score) || !aligned16(a->ape) || !aligned16(a->out))
    return SATTN_ERR_ALIGNMENT;
  if (static_cast<int64_t>(a->batch) * n_out * (a->head_dim / 8) > (int64_t(1) << 40)) return SATTN_ERR_UNSUPPORTED;
  sattn::CompressParams p;
  p.kv = a->kv;
  p.score = a->score;
  p.ape = a->ape;
  p.out = a->out;
  p.out_batch_stride = a->out_batch_stride;
  p.batch = a->batch;
  p.seq_len = a->seq_len;
  p.head_dim = a->head_dim;
  p.ratio = a->ratio;
  p.overlap = a->overlap;
  return launch_status(sattn::launch_compress_pool(p, a->dtype == SATTN_F32 ? sattn::kF32 : sattn::kBF16, stream));
}

sattn_status sattn_indexer_topk(const sattn_indexer_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (a->batch < 0 || a->q_len < 0 || a->window < 1 || a->n_comp < 0 || a->topk < 0) return SATTN_ERR_SHAPE;
  if (a->ratio < 0 || (a->ratio == 0 && a->n_comp > 0)) return SATTN_ERR_ARG;
  if (a->batch > 65535) return SATTN_ERR_UNSUPPORTED;  // one grid row per batch row
  if (a->rank != 16 && a->rank != 32 && a->rank != 64 && a->rank != 128) return SATTN_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(a->window) + a->topk > INT32_MAX) return SATTN_ERR_SHAPE;
  // 32-bit buffer offsets over one batch row's qr and index keys
  if (static_cast<int64_t>(a->q_len) * a->rank * 2 >= (int64_t(1) << 31) ||
      static_cast<int64_t>(a->n_comp) * a->rank * 2 >= (int64_t(1) << 31))
    return SATTN_ERR_UNSUPPORTED;
  if (a->batch == 0 || a->q_len == 0) return SATTN_OK;
  if (!a->out || !a->qr || !a->start_pos || (a->n_comp > 0 && !a->kidx)) return SATTN_ERR_NULL_PTR;
  if (!aligned4(a->out) || !aligned4(a->start_pos) || !aligned16(a->qr) || (a->kidx && !aligned16(a->kidx)))
    return SATTN_ERR_ALIGNMENT;
  sattn::IndexerParams p;
  p.out = a->out;
  p.qr = a->qr;
  p.kidx = a->kidx;
  p.start_pos = a->start_pos;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.rank = a->rank;
  p.window = a->window;
  p.ratio = a->ratio;
  p.n_comp = a->n_comp;
  p.topk = a->topk;
  return launch_status(sattn::launch_indexer_topk(p, stream));
}

sattn_status sattn_indexed_fp8_fwd(const sattn_indexed_fp8_args *a, hipStream_t stream) {
  if (!a) return SATTN_ERR_NULL_PTR;
  if (!valid_sink(a->sink_mode)) return SATTN_ERR_ARG;
  if (a->batch < 0 || a->q_len < 0 || a->num_heads <= 0 || a->kv_len < 0 || a->topk < 0 || a->head_dim <= 0 ||
      a->rope_dims < 0 || a->rope_dims > a->head_dim)
    return SATTN_ERR_SHAPE;
  if (!isfinite(a->softmax_scale)) return SATTN_ERR_ARG;
  if (a->num_splits < 1 || a->num_splits > (a->topk > 0 ? a->topk : 1)) return SATTN_ERR_ARG;
  const int64_t rows = static_cast<int64_t>(a->batch) * a->q_len;
  if (rows == 0) return SATTN_OK;
  if (rows > INT32_MAX) return SATTN_ERR_UNSUPPORTED;
  if (!a->q || !a->o || (a->topk > 0 && !a->topk_idxs)) return SATTN_ERR_NULL_PTR;
  if (a->kv_len > 0 && (!a->kv_fp8 || !a->kv_scale || (a->rope_dims > 0 && !a->kv_rope))) return SATTN_ERR_NULL_PTR;
  if (a->sink_mode != SATTN_SINK_NONE && !a->sinks) return SATTN_ERR_NULL_PTR;
  if (!aligned16(a->q) || !aligned16(a->o) || (a->kv_fp8 && !aligned16(a->kv_fp8)) ||
      (a->kv_rope && !aligned16(a->kv_rope)) || (a->kv_scale && !aligned4(a->kv_scale)) ||
      (a->topk_idxs && !aligned4(a->topk_idxs)) || (a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return SATTN_ERR_ALIGNMENT;

  sattn::IndexedParams p = {};
  p.q = a->q;
  p.kv = a->kv_fp8;
  p.kv_scale = a->kv_scale;
  p.kv_rope = a->kv_rope;
  p.rope_dims = a->rope_dims;
  p.idx = a->topk_idxs;
  p.o = a->o;
  p.lse = a->lse;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.kv_len = a->kv_len;
  p.topk = a->topk;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.sinks = a->sink_mode != SATTN_SINK_NONE ? a->sinks : nullptr;
  p.sink_mode = a->sink_mode;
  p.num_parts = 1;
  p.part_len = a->topk > 0 ? a->topk : 1;
  if (!sattn::indexed_fp8_supported(p)) return SATTN_ERR_UNSUPPORTED;

  if (a->num_splits == 1) return launch_status(sattn::launch_indexed_fp8(p, stream));
  const size_t need = sattn_indexed_workspace_size(a->batch, a->q_len, a->num_heads, a->head_dim, a->num_splits);
  if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255u) || a->workspace_bytes < need)
    return SATTN_ERR_WORKSPACE;
  p.part_len = (a->topk + a->num_splits - 1) / a->num_splits;
  const int parts = (a->topk + p.part_len - 1) / p.part_len;  // slices that hold at least one entry
  if (parts == 1) {
    p.part_len = a->topk;
    return launch_status(sattn::launch_indexed_fp8(p, stream));
  }
  char *ws = static_cast<char *>(a->workspace);
  p.num_parts = parts;
  p.part_o = reinterpret_cast<float *>(ws);
  p.part_lse = reinterpret_cast<float *>(ws + part_o_bytes(a->num_splits, rows, a->num_heads, a->head_dim));
  if (sattn::launch_indexed_fp8(p, stream) != hipSuccess) return SATTN_ERR_LAUNCH;
  sattn::MergeParams m;
  m.part_o = p.part_o;
  m.part_lse = p.part_lse;
  m.num_parts = parts;
  m.rows = static_cast<int>(rows);
  m.num_heads = a->num_heads;
  m.head_dim = a->head_dim;
  m.sinks = p.sinks;
  m.sink_mode = a->sink_mode == SATTN_SINK_NULL_LOGIT ? SATTN_SINK_NULL_LOGIT : SATTN_SINK_NONE;
  m.out_type = sattn::kBF16;
  m.o = a->o;
  m.lse = a->lse;
  return launch_status(sattn::launch_merge(m, stream));
}

}  // extern "C"
