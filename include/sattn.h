/*
 * sattn.h -- C ABI of libsattn: index-gathered attention forward with online
 * softmax for AMD Instinct MI355X (gfx950).
 *
 * For every query token there is a set of keys.  The library computes
 *     o = softmax(scale * q . k^T + sink term) . v
 * over that set only, and optionally the natural-log log-sum-exp of the
 * logits.  The key set is either
 *   - a sliding window inside one sequence of a varlen batch (vLLM PR #49815
 *     report, "关键源码片段": `context_attention_fwd` takes q, k, v, o,
 *     per-sequence start/length from cu_seqlens, the softmax scale, a q-side
 *     and a k-side window width and per-head sinks; its test reference builds
 *     GQA with repeat_interleave and masks |i - j| > window), or
 *   - an explicit top-k list of rows of a single-head cache whose row is read
 *     as both key and value (DeepSeek-V4 CSA/HCA article, §3.3 cache layout
 *     and §4.2 gather: `topk_idxs[b, m, k]` holds absolute cache rows, -1
 *     marks an unused slot).
 *
 * Sink semantics (vLLM report, `_fwd_kernel` sink branch; DeepSeek-V4 article
 * §4.4):
 *   SATTN_SINK_KEY0_BIAS  sinks[h] is added to the logit of key 0 (the first
 *                         token of the sequence on the window path, cache row 0
 *                         on the indexed path) when that key is in the set;
 *   SATTN_SINK_NULL_LOGIT sinks[h] is a logit with no value: exp(sinks[h])
 *                         enters the softmax denominator only.
 * Sinks are in natural-logit units and are not multiplied by the scale.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing, keeps no pointer after returning and holds no mutable
 *     global state, so it may be called from several host threads.  The one
 *     exception is sattn_indexed_fwd_noalloc, whose split-K partials live in a
 *     fixed device array per GPU (see its declaration).
 *   - Every kernel is enqueued on `stream` (the split-K merge included);
 *     nothing runs on the default stream unless `stream` is it, and nothing
 *     synchronises.  A caller that produces inputs on another stream must make
 *     `stream` wait on it (an event), as the nano-vllm offload note's stream
 *     fix shows.
 *   - Arguments are validated on the host before any launch; on error a status
 *     is returned and nothing is enqueued.  A launch failure returns
 *     SATTN_ERR_LAUNCH.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Tensors are dense, row-major (last dimension contiguous); q/k/v/o/kv
 *     must be 16-byte aligned and head_dim a multiple of 8.
 *   - Output rows whose key set is empty get o = 0 and lse = -inf (with a null
 *     sink: lse = sinks[h]).
 *
 * Tracing: with SATTN_TRACE set to a value other than "" or "0" when the
 * library first looks at it, every kernel launch prints one line to stderr,
 * "[sattn] <kernel variant> grid=... block=... (<the sizes that chose it>)",
 * before the launch is enqueued.
 */
#ifndef SATTN_H
#define SATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SATTN_ABI_VERSION 7

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_NULL_PTR = 1,    /* a required pointer is NULL                        */
  SATTN_ERR_SHAPE = 2,       /* a size is negative/zero or inconsistent           */
  SATTN_ERR_DTYPE = 3,       /* unknown dtype                                     */
  SATTN_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. head_dim > 256)   */
  SATTN_ERR_ALIGNMENT = 5,   /* a tensor pointer is not 16-byte aligned           */
  SATTN_ERR_WORKSPACE = 6,   /* split-K workspace missing or too small            */
  SATTN_ERR_LAUNCH = 7,      /* the HIP runtime rejected a kernel launch          */
  SATTN_ERR_ARG = 8,         /* bad enum value or option                          */
  SATTN_ERR_SCRATCH_LIMIT = 9 /* split-K partials exceed the fixed scratch of
                                 sattn_indexed_fwd_noalloc                          */
} sattn_status;

typedef enum { SATTN_BF16 = 0, SATTN_F32 = 1 } sattn_dtype;

typedef enum {
  SATTN_SINK_NONE = 0,
  SATTN_SINK_KEY0_BIAS = 1,
  SATTN_SINK_NULL_LOGIT = 2
} sattn_sink_mode;

/*
 * Sliding-window attention over a varlen batch.
 *
 *   q   [total_tokens, num_heads,    head_dim]  dtype
 *   k,v [total_tokens, num_kv_heads, head_dim]  dtype
 *   o   [total_tokens, num_heads,    head_dim]  dtype (written)
 *   lse [total_tokens, num_heads] fp32, natural log (written; may be NULL)
 *   cu_seqlens  device int32 [num_seqs + 1]: cu[0] = 0, non-decreasing,
 *               cu[num_seqs] = total_tokens; sequence s owns tokens
 *               [cu[s], cu[s+1]).  Zero-length sequences are allowed.
 *   max_seqlen  an upper bound of every sequence length (sizes the grid);
 *               tokens past max_seqlen in a longer sequence are NOT computed,
 *               as with the page's max_input_len.
 *   Query head h reads KV head h / (num_heads / num_kv_heads).
 *   Query i of a sequence attends key j of the same sequence iff
 *       (window_left  < 0 or j >= i - window_left) and
 *       (window_right < 0 or j <= i + window_right).
 *   A symmetric window of width w is (w, w); causal is (w - 1, 0) for a
 *   w-token window including the query itself, or (-1, 0) for full causal.
 *   sinks: device fp32 [num_heads]; required unless sink_mode is NONE.
 */
typedef struct {
  sattn_dtype dtype;
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t max_seqlen;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window_left;
  int32_t window_right;
  float softmax_scale;
  const float *sinks;
  sattn_sink_mode sink_mode;
} sattn_window_args;

/*
 * Top-k index-gathered attention over a single-head cache shared by all
 * query heads (each cache row is both key and value).
 *
 *   q         [batch, q_len, num_heads, head_dim]  dtype
 *   kv        [batch, kv_len, head_dim]            dtype
 *   topk_idxs [batch, q_len, topk] int32: absolute rows of kv[b]; any value
 *             outside [0, kv_len) (the documented one is -1) is not a key.
 *             Valid entries of one list must be distinct (a repeated row
 *             would be counted twice).  List order does not matter.
 *   o         [batch, q_len, num_heads, head_dim]  dtype (written)
 *   lse       [batch, q_len, num_heads] fp32 natural log (written; may be NULL)
 *   num_splits 1: one pass.  S > 1: the list is cut into S contiguous slices
 *             of ceil(topk / S) entries (slices that would hold no entry are
 *             not created); each slice's normalised partial output and
 *             log-sum-exp go to `workspace`, then a second kernel on the same
 *             stream merges them (sattn_merge_lse) into o / lse.  A null sink
 *             enters once, in the merge; a key-0 bias applies in the slice that
 *             holds row 0.  1 <= S <= topk is required.
 *   workspace  device buffer of at least
 *             sattn_indexed_workspace_size(batch, q_len, num_heads, head_dim, S)
 *             bytes, 256-byte aligned (may be NULL when S == 1).  Layout:
 *             part_o [S, batch*q_len, num_heads, head_dim] fp32, then part_lse
 *             [S, batch*q_len, num_heads] fp32, each from a 256-byte boundary;
 *             after the call the slices' partials are there.  Calls that overlap
 *             and share one workspace race.
 */
typedef struct {
  sattn_dtype dtype;
  const void *q;
  const void *kv;
  const int32_t *topk_idxs;
  void *o;
  float *lse;
  int32_t batch;
  int32_t q_len;
  int32_t num_heads;
  int32_t head_dim;
  int32_t kv_len;
  int32_t topk;
  float softmax_scale;
  const float *sinks;
  sattn_sink_mode sink_mode;
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
} sattn_indexed_args;

/*
 * Merge of per-chunk partial results (the nano-vllm offload note's
 * three-stage KV chunking: partial softmax statistics per chunk, merged into
 * global ones).
 *
 *   part_o   [num_parts, rows, num_heads, head_dim] fp32: each part's output
 *            normalised by its own denominator
 *   part_lse [num_parts, rows, num_heads] fp32: each part's log-sum-exp;
 *            -inf marks a part with no key (its part_o is ignored)
 *   sink_mode NONE or NULL_LOGIT (the null sink is added to the merged
 *            denominator once); KEY0_BIAS is rejected (it belongs to a part).
 *   o        [rows, num_heads, head_dim] out_dtype (written)
 *   lse      [rows, num_heads] fp32 natural log (written; may be NULL)
 *   o_m = sum_c exp(lse_c - M) o_c / W,  W = sum_c exp(lse_c - M) [+ exp(sink - M)],
 *   lse = M + log W,  M = max(lse_c, sink).
 */
typedef struct {
  const float *part_o;
  const float *part_lse;
  int32_t num_parts;
  int32_t rows;
  int32_t num_heads;
  int32_t head_dim;
  const float *sinks;
  sattn_sink_mode sink_mode;
  sattn_dtype out_dtype;
  void *o;
  float *lse;
} sattn_merge_args;

/*
 * Top-k lists of the indexed path built on the device (DeepSeek-V4 CSA/HCA
 * article: §2.3, a query's list is its sliding-window indices followed by its
 * compressed-region indices; §3.3, the cache of a batch row is
 * [window + n_comp, d] with position p's row in ring slot p % window and
 * compressed row c at window + c, compressed token c existing once position
 * (c + 1) * ratio - 1 has been seen).
 *
 *   out       [batch, q_len, window + n_comp] int32 (written), the idx argument
 *             of sattn_indexed_fwd with topk = window + n_comp
 *   start_pos [batch] int32 device array: query t of batch row b sits at
 *             absolute position start_pos[b] + t (a negative position sees
 *             nothing)
 *   window    ring size (>= 1)
 *   ratio     tokens per compressed row; 0 = no compressed region (n_comp
 *             must then be 0)
 *   n_comp    compressed rows held by the cache (>= 0)
 *
 * Entry k < window of a query at position p is the ring slot of position
 * max(0, p - window + 1) + k when that position is <= p, else -1; entry
 * window + c is row window + c when (c + 1) * ratio - 1 <= p, else -1.  So a
 * list holds its valid rows first in each part, in increasing position, then
 * -1 padding; all valid rows are distinct.
 */
typedef struct {
  int32_t *out;
  const int32_t *start_pos;
  int32_t batch;
  int32_t q_len;
  int32_t window;
  int32_t ratio;
  int32_t n_comp;
} sattn_build_idx_args;

sattn_status sattn_build_topk_idxs(const sattn_build_idx_args *args, hipStream_t stream);

/*
 * Attention mass of each block of list entries, normalised by a given
 * log-sum-exp (nano-vllm XAttention offload note, technical details: the
 * third stage of the chunked estimate normalises with the global softmax
 * statistics that the first two stages produced per chunk and merged, and
 * sums per block).  Here the statistics are those of the indexed path, e.g.
 * the lse that sattn_indexed_fwd (one pass, or split-K and merged) returns.
 *
 *   q, kv, topk_idxs, softmax_scale, sinks, sink_mode: as sattn_indexed_args
 *   lse        [batch, q_len, num_heads] fp32 natural log: the normaliser
 *   block_keys entries per block (>= 1); block c of a list is entries
 *              [c * block_keys, (c + 1) * block_keys)
 *   mass       [batch, q_len, num_heads, ceil(topk / block_keys)] fp32
 *              (written, every element)
 *
 *   mass[b, t, h, c] = sum over valid entries k of block c (0 <= idx < kv_len)
 *                      of exp(softmax_scale * q[b, t, h] . kv[b, idx] + bias - lse[b, t, h]),
 *   bias = sinks[h] for cache row 0 under KEY0_BIAS, else 0.  A null sink
 *   belongs to no block: with the lse of the same list, the masses of a row
 *   plus exp(sinks[h] - lse) sum to 1 (without a null sink they sum to 1).
 *   A block with no valid entry gets 0; lse = -inf with a valid entry gives
 *   +inf.  The fast path is bf16 with head_dim 64 or 128, num_heads a
 *   multiple of 32, block_keys a multiple of 32 and softmax_scale > 0; other
 *   shapes (fp32 among them) take a generic kernel.
 */
typedef struct {
  sattn_dtype dtype;
  const void *q;
  const void *kv;
  const int32_t *topk_idxs;
  const float *lse;
  float *mass;
  int32_t batch;
  int32_t q_len;
  int32_t num_heads;
  int32_t head_dim;
  int32_t kv_len;
  int32_t topk;
  int32_t block_keys;
  float softmax_scale;
  const float *sinks;
  sattn_sink_mode sink_mode;
} sattn_block_mass_args;

sattn_status sattn_block_mass(const sattn_block_mass_args *args, hipStream_t stream);

/*
 * Gated pooling of the compressor (DeepSeek-V4 CSA/HCA article, §5.1: a compressed row is the
 * sum over a window of kv_i * softmax(score_i), with the learned absolute position term ape
 * added to the scores; with overlap, kv and score carry 2 * head_dim features per token and the
 * overlap transform lets window i see the previous window's tokens through their first
 * head_dim features and its own tokens through their last head_dim features).
 *
 *   kv, score  [batch, seq_len, coff * head_dim] dtype (coff = 2 if overlap, else 1): the
 *              projected kv and gate scores of every token
 *   ape        [ratio, coff * head_dim] dtype
 *   out        compressed row w of batch b at out + (b * out_batch_stride + w) * head_dim,
 *              w < seq_len / ratio (written); out_batch_stride >= seq_len / ratio rows, so out
 *              may point at the compressed region of a [batch, window + n_comp, head_dim]
 *              cache (out = cache + window * head_dim, stride window + n_comp)
 *
 *   Window w holds tokens [w * ratio, (w + 1) * ratio); a trailing partial window is not
 *   compressed.  For every feature f < head_dim:
 *     entries = {(kv[t][lo + f], score[t][lo + f] + ape[t - w * ratio][lo + f]) : t in window w}
 *               with lo = head_dim if overlap else 0,
 *             plus, with overlap and w > 0, {(kv[t][f], score[t][f] + ape[t - (w-1) * ratio][f]) :
 *               t in window w - 1};
 *     out[w][f] = sum over entries of kv * exp(s) / sum of exp(s).
 *   Computed in fp32; out rounded to dtype.  head_dim must be a multiple of 8 and the tensors
 *   16-byte aligned.
 */
typedef struct {
  sattn_dtype dtype;
  const void *kv;
  const void *score;
  const void *ape;
  void *out;
  int64_t out_batch_stride;
  int32_t batch;
  int32_t seq_len;
  int32_t head_dim;
  int32_t ratio;
  int32_t overlap;
} sattn_compress_args;

sattn_status sattn_compress_pool(const sattn_compress_args *args, hipStream_t stream);

/*
 * Top-k lists chosen by a synthetic indexer (DeepSeek-V4 CSA/HCA article, §2.3: the indexer,
 * fed the low-rank query qr, picks each query's compressed-region indices; the window indices
 * come first and the two parts are concatenated).  The article fixes neither the scoring nor
 * the weights; here:
 *
 *   out       [batch, q_len, window + topk] int32 (written), the idx argument of
 *             sattn_indexed_fwd with topk' = window + topk
 *   qr        [batch, q_len, rank] bf16: low-rank query of each token
 *   kidx      [batch, n_comp, rank] bf16: index key of each compressed row
 *   start_pos [batch] int32 device array: query t of batch row b is at position start_pos[b] + t
 *   window, ratio, n_comp: as sattn_build_idx_args (the window part of a list is identical)
 *   rank      16, 32, 64 or 128
 *
 * Errors: SHAPE for negative sizes or window < 1; ARG for ratio < 0, or ratio 0 with n_comp > 0;
 * UNSUPPORTED for another rank, batch > 65535, or q_len * rank or n_comp * rank at or above 2^30;
 * NULL_PTR / ALIGNMENT for a missing or misaligned pointer (qr and kidx 16-byte, out and
 * start_pos 4-byte; kidx may be null when n_comp is 0).  batch or q_len 0 is a no-op.  The call
 * is asynchronous on `stream` and allocates nothing.
 *
 * Entries [0, window) are the window part of sattn_build_topk_idxs.  The candidates are the
 * compressed rows c the query sees ((c + 1) * ratio - 1 <= position, c < n_comp); each scores
 * qr[b, t] . kidx[b, c] (fp32 accumulation of bf16 products); the min(topk, candidates) highest
 * scores win, ties going to the lower c; entries window .. are the winners as rows window + c in
 * increasing c, then -1.
 */
typedef struct {
  int32_t *out;
  const void *qr;
  const void *kidx;
  const int32_t *start_pos;
  int32_t batch;
  int32_t q_len;
  int32_t rank;
  int32_t window;
  int32_t ratio;
  int32_t n_comp;
  int32_t topk;
} sattn_indexer_args;

sattn_status sattn_indexer_topk(const sattn_indexer_args *args, hipStream_t stream);

/*
 * Top-k index-gathered attention (as sattn_indexed_fwd) over an fp8 cache (DeepSeek-V4 CSA/HCA
 * article, §5.3: the compressed kv is quantised with the dims that carry no rotary embedding in
 * fp8 and the rotary dims at higher precision; §4.1-§4.4: the gathered attention).  The article
 * fixes no layout; the one taken here:
 *
 *   q, topk_idxs, o, lse, softmax_scale, sinks, sink_mode, num_splits, workspace: as
 *             sattn_indexed_args with dtype bf16 (the workspace size is the same)
 *   kv_fp8    [batch, kv_len, head_dim - rope_dims] uint8: e4m3 codes (OCP "fn": bias 7, no
 *             infinities; S.1111.111 is NaN) of the first head_dim - rope_dims dims of each row
 *   kv_scale  [batch, kv_len] fp32: one scale per row, a positive power of two (the keys take
 *             only its exponent, the values its whole value: other scales are not supported and
 *             give unspecified results); row value = e4m3(code) * scale
 *   kv_rope   [batch, kv_len, rope_dims] bf16: the last rope_dims dims of each row (NULL when
 *             rope_dims is 0)
 *   head_dim  128; rope_dims 0 or 64; num_heads a multiple of 32; softmax_scale > 0
 *
 * Errors as sattn_indexed_fwd; other head_dim / rope_dims / num_heads values or scale <= 0 give
 * UNSUPPORTED.  kv_fp8, kv_rope and q 16-byte aligned; kv_scale 4-byte aligned.
 */
typedef struct {
  const void *q;
  const uint8_t *kv_fp8;
  const float *kv_scale;
  const void *kv_rope;
  const int32_t *topk_idxs;
  void *o;
  float *lse;
  int32_t batch;
  int32_t q_len;
  int32_t num_heads;
  int32_t head_dim;
  int32_t rope_dims;
  int32_t kv_len;
  int32_t topk;
  float softmax_scale;
  const float *sinks;
  sattn_sink_mode sink_mode;
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
} sattn_indexed_fp8_args;

sattn_status sattn_indexed_fp8_fwd(const sattn_indexed_fp8_args *args, hipStream_t stream);

sattn_status sattn_window_fwd(const sattn_window_args *args, hipStream_t stream);
sattn_status sattn_indexed_fwd(const sattn_indexed_args *args, hipStream_t stream);
sattn_status sattn_merge_lse(const sattn_merge_args *args, hipStream_t stream);

/*
 * sattn_indexed_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results; `workspace` and `workspace_bytes` are ignored and the split-K partials (num_splits > 1)
 * go to a fixed scratch array of SATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it has run on until the process ends.  The call allocates nothing.
 *   - Calls whose partials need more than the scratch
 *     (sattn_indexed_workspace_size(...) > SATTN_NOALLOC_SCRATCH_BYTES) return
 *     SATTN_ERR_SCRATCH_LIMIT before anything is enqueued.
 *   - The scratch of the current device (hipGetDevice) is used; `stream` must belong to it
 *     (a stream of another device returns SATTN_ERR_UNSUPPORTED before anything is enqueued).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 *     different streams, or from several host threads without ordering) race and give wrong
 *     results.  Calls ordered on one stream do not.
 *   - With num_splits == 1 no scratch is touched.
 */
#define SATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
sattn_status sattn_indexed_fwd_noalloc(const sattn_indexed_args *args, hipStream_t stream);

/* Bytes of split-K workspace sattn_indexed_fwd needs (0 when num_splits <= 1). */
size_t sattn_indexed_workspace_size(int32_t batch, int32_t q_len, int32_t num_heads,
                                    int32_t head_dim, int32_t num_splits);

/* Static, NUL-terminated description of a status code. */
const char *sattn_status_string(sattn_status status);

/* SATTN_ABI_VERSION of the loaded library. */
int sattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */
