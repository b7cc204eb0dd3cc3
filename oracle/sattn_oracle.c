/*
 * sattn_oracle.c -- plain CPU reference for index-gathered attention forward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library it checks.
 *
 * What it computes (sources are the two pages that define the problem):
 *   - vLLM PR #49815 report, "关键源码片段" / test file: the dense fp32 window
 *     reference `_reference` -- per sequence of a cu_seqlens batch, GQA head h
 *     reads KV head h / (H / H_kv) (repeat_interleave), scores q.k * scale,
 *     the per-head sink added to the score of the sequence's key 0, keys with
 *     |i - j| > window excluded, softmax over keys, weighted sum of v.
 *   - same report, `_fwd_kernel` sink branch: the "null logit" sink semantics,
 *     where the sink is one more term of the softmax denominator and never of
 *     the numerator (the state starts at m = sink, l = 1).
 *   - DeepSeek-V4 CSA/HCA article, §4.2 (gather) and §4.4 (attention sink):
 *     each query's key set is its top-k index list into a single-head cache
 *     whose row serves as both key and value; -1 marks an unused slot; the
 *     per-head sink enters only the denominator.
 *   - nano-vllm "XAttention Offload Stream Synchronization Fix", technical
 *     details, three-stage KV chunking: per-chunk partial softmax statistics
 *     merged into global ones.
 *
 * Everything is evaluated in double precision, straight from the definition:
 * logits for the key set, softmax with the maximum subtracted (an exact
 * identity), weighted sum.  There is no blocking, no online rescaling and no
 * reordering beyond that.  Inputs are fp32 (bf16 inputs arrive upcast exactly).
 *
 * Readings where the pages leave a point open:
 *   - the window is inclusive: key j is attended by query i of the same
 *     sequence iff i - wl <= j <= i + wr (wl or wr < 0: unbounded on that side);
 *   - "key 0" is sequence-local position 0 on the window path and cache row 0
 *     on the indexed path, and the bias applies only when that key is in the set;
 *   - an empty key set gives o = 0 and lse = -inf (with a null sink: lse = sink);
 *   - lse is the natural-log log-sum-exp of the logits, null sink included;
 *   - indices outside [0, N) are not keys; duplicate valid indices are rejected.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { SINK_NONE = 0, SINK_KEY0 = 1, SINK_NULL = 2 };

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARGS = -1,
  ORACLE_ERR_DUPLICATE = -2,
  ORACLE_ERR_NOMEM = -3
};

/*
 * Softmax attention of one query row over an explicit key set.
 *   logit_j = scale * <q, k_j> + bias_j              (bias_j: key-0 sink, else 0)
 *   den     = sum_j exp(logit_j) [+ exp(sink) for a null sink]
 *   o       = sum_j exp(logit_j) * v_j / den
 *   lse     = log(den)
 * The common maximum is subtracted before exponentiating; it cancels exactly.
 */
static void attend_set(const float *q, int D, double scale, int nkeys,
                       const float *const *krows, const float *const *vrows,
                       const double *bias, int null_sink, double sink,
                       double *logit, double *o, double *lse) {
  double m = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += (double)q[d] * (double)krows[j][d];
    logit[j] = scale * dot + (bias ? bias[j] : 0.0);
    if (logit[j] > m) m = logit[j];
  }
  if (null_sink && sink > m) m = sink;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (m == -INFINITY) { /* no key and no (finite) sink */
    *lse = -INFINITY;
    return;
  }
  double den = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    double e = exp(logit[j] - m);
    den += e;
    for (int d = 0; d < D; ++d) o[d] += e * (double)vrows[j][d];
  }
  if (null_sink) den += exp(sink - m);
  for (int d = 0; d < D; ++d) o[d] /= den;
  *lse = m + log(den);
}

static int seq_of_token(const int32_t *cu, int num_seqs, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) { /* last sequence whose start is <= t */
    int mid = (lo + hi + 1) / 2;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/*
 * Window path.  q [T,H,D], k/v [T,Hkv,D] (fp32), cu_seqlens [num_seqs+1].
 * rows: token indices to evaluate (NULL = all T tokens, in order); o is
 * [num_rows,H,D] and lse [num_rows,H] in double.
 */
int oracle_window(const float *q, const float *k, const float *v, const int32_t *cu_seqlens,
                  int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                  int window_left, int window_right, double scale,
                  const float *sinks, int sink_mode,
                  const int64_t *rows, int64_t num_rows, double *o, double *lse, int nthreads) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_heads % num_kv_heads != 0 || (sink_mode != SINK_NONE && !sinks))
    return ORACLE_ERR_ARGS;
  const int64_t T = num_seqs > 0 ? cu_seqlens[num_seqs] : 0;
  const int64_t nr = rows ? num_rows : T;
  const int H = num_heads, Hkv = num_kv_heads, D = head_dim, G = H / Hkv;
  int32_t maxlen = 0;
  for (int s = 0; s < num_seqs; ++s) {
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return ORACLE_ERR_ARGS;
    if (cu_seqlens[s + 1] - cu_seqlens[s] > maxlen) maxlen = cu_seqlens[s + 1] - cu_seqlens[s];
  }
  for (int64_t r = 0; r < nr; ++r)
    if (rows && (rows[r] < 0 || rows[r] >= T)) return ORACLE_ERR_ARGS;
  int err = ORACLE_OK;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    const float **kr = malloc(sizeof(*kr) * (size_t)(maxlen + 1));
    const float **vr = malloc(sizeof(*vr) * (size_t)(maxlen + 1));
    double *bias = malloc(sizeof(double) * (size_t)(maxlen + 1));
    double *logit = malloc(sizeof(double) * (size_t)(maxlen + 1));
    if (!kr || !vr || !bias || !logit) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = ORACLE_ERR_NOMEM;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
      for (int64_t r = 0; r < nr; ++r) {
        const int64_t t = rows ? rows[r] : r;
        const int s = seq_of_token(cu_seqlens, num_seqs, t);
        const int64_t a = cu_seqlens[s];
        const int64_t L = cu_seqlens[s + 1] - a;
        const int64_t i = t - a;
        int64_t lo = window_left < 0 ? 0 : i - window_left;
        int64_t hi = window_right < 0 ? L - 1 : i + window_right;
        if (lo < 0) lo = 0;
        if (hi > L - 1) hi = L - 1;
        for (int h = 0; h < H; ++h) {
          const int g = h / G;
          int n = 0;
          for (int64_t j = lo; j <= hi; ++j, ++n) {
            kr[n] = k + ((a + j) * Hkv + g) * (int64_t)D;
            vr[n] = v + ((a + j) * Hkv + g) * (int64_t)D;
            bias[n] = (sink_mode == SINK_KEY0 && j == 0) ? (double)sinks[h] : 0.0;
          }
          attend_set(q + (t * H + h) * (int64_t)D, D, scale, n, kr, vr, bias,
                     sink_mode == SINK_NULL, sink_mode == SINK_NULL ? (double)sinks[h] : 0.0,
                     logit, o + (r * H + h) * (int64_t)D, lse + r * H + h);
        }
      }
    }
    free(kr); free(vr); free(bias); free(logit);
  }
  return err;
}

static int cmp_i32(const void *x, const void *y) {
  int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
  return (a > b) - (a < b);
}

/*
 * Indexed path.  q [B,M,H,D], kv [B,N,D] (each row is key and value),
 * topk_idxs [B,M,K] int32 (-1 = unused).  rows: flat query indices b*M+t
 * (NULL = all B*M).  o [num_rows,H,D], lse [num_rows,H] in double.
 */
int oracle_indexed(const float *q, const float *kv, const int32_t *topk_idxs,
                   int batch, int q_len, int num_heads, int head_dim, int kv_len, int topk,
                   double scale, const float *sinks, int sink_mode,
                   const int64_t *rows, int64_t num_rows, double *o, double *lse, int nthreads) {
  if (batch < 0 || q_len < 0 || num_heads <= 0 || head_dim <= 0 || kv_len < 0 || topk < 0 ||
      (sink_mode != SINK_NONE && !sinks))
    return ORACLE_ERR_ARGS;
  const int64_t BM = (int64_t)batch * q_len;
  const int64_t nr = rows ? num_rows : BM;
  const int H = num_heads, D = head_dim, N = kv_len, K = topk;
  for (int64_t r = 0; r < nr; ++r)
    if (rows && (rows[r] < 0 || rows[r] >= BM)) return ORACLE_ERR_ARGS;
  int err = ORACLE_OK;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    const float **kr = malloc(sizeof(*kr) * (size_t)(K + 1));
    double *bias = malloc(sizeof(double) * (size_t)(K + 1));
    double *logit = malloc(sizeof(double) * (size_t)(K + 1));
    int32_t *sorted = malloc(sizeof(int32_t) * (size_t)(K + 1));
    if (!kr || !bias || !logit || !sorted) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = ORACLE_ERR_NOMEM;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < nr; ++r) {
        const int64_t bt = rows ? rows[r] : r;
        const int64_t b = bt / (q_len > 0 ? q_len : 1);
        const int32_t *list = topk_idxs + bt * K;
        int n = 0;
        for (int j = 0; j < K; ++j) {
          const int32_t x = list[j];
          if (x < 0 || x >= N) continue; /* -1 padding (and anything outside the cache) */
          kr[n] = kv + (b * N + x) * (int64_t)D;
          sorted[n] = x;
          ++n;
        }
        qsort(sorted, (size_t)n, sizeof(int32_t), cmp_i32);
        int dup = 0;
        for (int j = 1; j < n; ++j) dup |= sorted[j] == sorted[j - 1];
        if (dup) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
          err = ORACLE_ERR_DUPLICATE;
          continue;
        }
        for (int h = 0; h < H; ++h) {
          int nn = 0;
          for (int j = 0; j < K; ++j) {
            const int32_t x = list[j];
            if (x < 0 || x >= N) continue;
            bias[nn++] = (sink_mode == SINK_KEY0 && x == 0) ? (double)sinks[h] : 0.0;
          }
          attend_set(q + (bt * H + h) * (int64_t)D, D, scale, n, kr, kr, bias,
                     sink_mode == SINK_NULL, sink_mode == SINK_NULL ? (double)sinks[h] : 0.0,
                     logit, o + (r * H + h) * (int64_t)D, lse + r * H + h);
        }
      }
    }
    free(kr); free(bias); free(logit); free(sorted);
  }
  return err;
}

/*
 * Merge of per-chunk partial results (three-stage KV chunking: each chunk
 * carries its own softmax statistics; the merged statistics are their
 * log-sum-exp).  part_o [S,R,H,D] is each chunk's own normalised output and
 * part_lse [S,R,H] its log-sum-exp (-inf: the chunk had no key).  A null sink
 * enters the merged denominator once.
 *   M   = max(max_c lse_c, sink)
 *   W   = sum_c exp(lse_c - M) [+ exp(sink - M)]
 *   o   = sum_c exp(lse_c - M) * o_c / W,   lse = M + log W
 */
int oracle_merge(const float *part_o, const float *part_lse, int num_parts, int64_t rows,
                 int num_heads, int head_dim, const float *sinks, int sink_mode,
                 double *o, double *lse) {
  if (num_parts < 0 || rows < 0 || num_heads <= 0 || head_dim <= 0 ||
      sink_mode == SINK_KEY0 || (sink_mode == SINK_NULL && !sinks))
    return ORACLE_ERR_ARGS;
  const int H = num_heads, D = head_dim;
  for (int64_t r = 0; r < rows; ++r) {
    for (int h = 0; h < H; ++h) {
      const int64_t rh = r * H + h;
      double M = -INFINITY;
      for (int c = 0; c < num_parts; ++c) {
        double x = part_lse[c * rows * H + rh];
        if (x > M) M = x;
      }
      const int null_sink = sink_mode == SINK_NULL;
      if (null_sink && (double)sinks[h] > M) M = sinks[h];
      double *out = o + rh * D;
      for (int d = 0; d < D; ++d) out[d] = 0.0;
      if (M == -INFINITY) {
        lse[rh] = -INFINITY;
        continue;
      }
      double W = 0.0;
      for (int c = 0; c < num_parts; ++c) {
        double w = exp((double)part_lse[c * rows * H + rh] - M);
        if (w == 0.0) continue; /* an empty chunk carries no output */
        W += w;
        const float *oc = part_o + (c * rows * H + rh) * D;
        for (int d = 0; d < D; ++d) out[d] += w * (double)oc[d];
      }
      if (null_sink) W += exp((double)sinks[h] - M);
      for (int d = 0; d < D; ++d) out[d] /= W;
      lse[rh] = M + log(W);
    }
  }
  return ORACLE_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
