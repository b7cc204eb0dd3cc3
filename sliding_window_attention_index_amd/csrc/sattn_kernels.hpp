// Internal launch interface between the C ABI layer (sattn_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sattn {

enum ElemType : int { kBF16 = 0, kF32 = 1 };

// Window path: varlen batch, GQA, key set = band around each query.
struct WindowParams {
  const void *q, *k, *v;
  void *o;
  float *lse;                 // may be null
  const int32_t *cu_seqlens;  // [num_seqs + 1]
  int num_seqs, max_seqlen;
  int num_heads, num_kv_heads, head_dim, group;  // group = num_heads / num_kv_heads
  int window_left, window_right;                 // < 0: unbounded
  float scale_log2;                              // softmax_scale * log2(e)
  const float *sinks;                            // [num_heads] or null
  int sink_mode;
};

// Device-side top-k list construction.
struct BuildIdxParams {
  int32_t *out;              // [batch, q_len, window + n_comp]
  const int32_t *start_pos;  // [batch]
  int batch, q_len, window, ratio, n_comp;
};

// Indexed path: one shared K=V head per batch row, top-k lists.
struct IndexedParams {
  const void *q;        // [B, M, H, D]
  const void *kv;       // [B, N, D]
  const int32_t *idx;   // [B, M, K]
  void *o;              // [B, M, H, D] (single pass)
  float *lse;           // [B, M, H] or null
  int batch, q_len, num_heads, head_dim, kv_len, topk;
  float scale_log2;
  const float *sinks;
  int sink_mode;
  int num_parts;        // slices of the list; 1 = single pass
  int part_len;         // entries per slice (ceil(topk / num_parts))
  float *part_o;        // [num_parts, B*M, H, D] when num_parts > 1
  float *part_lse;      // [num_parts, B*M, H]
  // Block-mass launches (o, lse and part_* unused; part_len is a multiple of block_keys):
  const float *lse_in;  // [B*M, H] natural log, the normaliser
  float *mass;          // [B*M, H, n_bins]
  int block_keys, n_bins;
  // fp8 cache launches (kv = e4m3 codes [B, N, D - rope_dims]):
  const float *kv_scale;  // [B, N] one power-of-two scale per row
  const void *kv_rope;    // [B, N, rope_dims] bf16, or null when rope_dims == 0
  int rope_dims;
};

// Synthetic indexer: top-k compressed rows per query, after the window part of the list.
struct IndexerParams {
  int32_t *out;              // [batch, q_len, window + topk]
  const void *qr;            // [batch, q_len, rank] bf16
  const void *kidx;          // [batch, n_comp, rank] bf16
  const int32_t *start_pos;  // [batch]
  int batch, q_len, rank, window, ratio, n_comp, topk;
};

// Compressor pooling (one compressed row per complete window of `ratio` tokens).
struct CompressParams {
  const void *kv, *score;  // [batch, seq_len, coff * head_dim]
  const void *ape;         // [ratio, coff * head_dim]
  void *out;               // row w of batch b at out + (b * out_batch_stride + w) * head_dim
  int64_t out_batch_stride;
  int batch, seq_len, head_dim, ratio, overlap;
};

struct MergeParams {
  const float *part_o, *part_lse;
  int num_parts, rows, num_heads, head_dim;
  const float *sinks;
  int sink_mode;        // none or null
  int out_type;         // ElemType
  void *o;
  float *lse;
};

// Host-side launch trace: with SATTN_TRACE=1 in the environment (read once), every launcher prints
// one line per kernel launch to stderr (kernel variant, grid, and the sizes that chose them) before
// launching.  Off by default; nothing else changes.
bool trace_on();
void trace(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

// Launchers return hipSuccess or the launch error; they never synchronise.
hipError_t launch_window_valu(const WindowParams &p, int elem_type, hipStream_t stream);
hipError_t launch_indexed_valu(const IndexedParams &p, int elem_type, hipStream_t stream);
hipError_t launch_merge(const MergeParams &p, hipStream_t stream);

// MFMA (bf16) kernels.  `supported` tells whether a shape has an MFMA variant.
bool window_mfma_supported(const WindowParams &p);
hipError_t launch_window_mfma(const WindowParams &p, hipStream_t stream);
bool indexed_mfma_supported(const IndexedParams &p);
hipError_t launch_indexed_mfma(const IndexedParams &p, hipStream_t stream);
// One workgroup per (query, list slice) for all heads of the query (few queries, long lists); split
// launches write partials for launch_merge.
bool indexed_slice_supported(const IndexedParams &p);
hipError_t launch_indexed_slice(const IndexedParams &p, hipStream_t stream);
bool indexed_fp8_supported(const IndexedParams &p);
hipError_t launch_indexed_fp8(const IndexedParams &p, hipStream_t stream);

hipError_t launch_build_topk_idxs(const BuildIdxParams &p, hipStream_t stream);
hipError_t launch_compress_pool(const CompressParams &p, int elem_type, hipStream_t stream);
hipError_t launch_indexer_topk(const IndexerParams &p, hipStream_t stream);

// Per-block attention mass of the lists (IndexedParams block-mass fields).
hipError_t launch_block_mass_valu(const IndexedParams &p, int elem_type, hipStream_t stream);
bool block_mass_mfma_supported(const IndexedParams &p);
hipError_t launch_block_mass_mfma(const IndexedParams &p, hipStream_t stream);

}  // namespace sattn

#include "sattn.h"

namespace sattn {
// The C ABI's indexed call with the split-K workspace given separately (sattn_api.cpp).
sattn_status indexed_fwd_with_workspace(const sattn_indexed_args *a, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);
}  // namespace sattn
