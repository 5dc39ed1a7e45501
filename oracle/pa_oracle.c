/*
 * Paged grouped-query attention: the fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library: it is written from the
 * pages' definitions and nothing else.
 *
 * Pages cited (by short name):
 *   [IBM-PA]  "一行 Triton 代码同时跑赢 NVIDIA 和 AMD：IBM Research 把大模型推理的
 *             「硬件鸿沟」填平了" (papers.ananclaw.com, summary of arXiv 2511.11581)
 *   [GUIDE]   "从兆字节到兆瓦：基于CUDA与Triton的高性能LLM与扩散内核全指南"
 *             (zhxwu.com GPU programming guide)
 *
 * What it computes (one output row per query token and query head):
 *   - Result: scaled dot-product attention, softmax of the scaled scores
 *     Q K^T / sqrt(d_k) applied to V ([GUIDE] section "拆解多头注意力（MHA）",
 *     the SDPA formula).  The scale is an argument; the workloads pass
 *     1/sqrt(128) rounded to fp32.
 *   - Causal rule: a future token's score is minus infinity ([GUIDE] section
 *     "Triton实现Flash Attention", causal-mask item).  Query token i of a chunk
 *     of q_s new tokens at the end of a context of L_s tokens sits at absolute
 *     position L_s - q_s + i; tokens after that position are its future.
 *   - Paged KV cache read through a block table, prefix cache, and query
 *     heads grouped onto a shared KV head ([IBM-PA] the model-feature list in
 *     section "同一个模型,为什么"换张卡"就这么难?" and the Q-Block step of the
 *     five-step list).  Query head h reads KV head h / G, G = Hq / Hkv.
 *   - Split partials and their log-sum-exp merge (the parallel tiled softmax
 *     step of [IBM-PA]'s five-step list).  The merge is the algebra of the
 *     online-softmax statistics m and l ([GUIDE] section "Flash Attention革命",
 *     online-softmax item): split k yields its normalised output O_k and
 *     lse_k = m_k + ln l_k; with M = max_k lse_k and w_k = exp(lse_k - M),
 *     O = sum_k w_k O_k / sum_k w_k and LSE = M + ln sum_k w_k.
 *
 *   - Paged KV append, the write that precedes attention: the q_s new tokens
 *     of a sequence are the last q_s positions of its L_s-token context
 *     (same reading as the causal rule), so new token i lands at position
 *     L_s - q_s + i, in the page the block table names for that position,
 *     at slot position mod P ([IBM-PA] model-feature list: paged KV cache).
 *
 * The softmax here is the plain two-pass one (max, then exponentials and
 * sums), in fp64, over logical token positions in order.  bf16 inputs are
 * widened to fp64 exactly.  Nothing is tiled, fused or reordered.
 *
 * Build: gcc -O2 -shared -fPIC -pthread pa_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> fp64, exact: bf16 is the top half of an fp32. */
static double bf16_to_f64(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

typedef struct {
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, page_size;
  const uint16_t *q;               /* [T, Hq, D] bf16 bits                 */
  const int32_t *query_start_loc;  /* [num_seqs + 1]; NULL: one token each */
  const uint16_t *k_pool, *v_pool; /* paged pools, bf16 bits               */
  int64_t stride_page, stride_token, stride_head; /* elements; dim stride 1 */
  const int32_t *block_tables;     /* [num_seqs, max_blocks]               */
  int32_t max_blocks;
  const int32_t *context_lens;     /* [num_seqs]                           */
  double scale;
  int32_t causal;
  /* split mode: split k covers tokens [k*split_tokens, (k+1)*split_tokens) */
  int32_t split_tokens, num_splits;
  const int64_t *rows;             /* flat (token*Hq + head), or NULL: all  */
  int64_t num_rows;
  double *out, *lse;               /* single pass: [rows, D], [rows]
                                      split mode:  [rows, S, D], [rows, S]  */
} job_t;

/* Sequence that owns query token t (query_start_loc is non-decreasing). */
static int32_t seq_of_token(const job_t *j, int64_t t) {
  if (!j->query_start_loc) return (int32_t)t;
  int32_t lo = 0, hi = j->num_seqs - 1;
  while (lo < hi) { /* last s with query_start_loc[s] <= t */
    int32_t mid = (lo + hi + 1) / 2;
    if ((int64_t)j->query_start_loc[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* Element offset of (logical token, kv head) of sequence s, via the block
 * table: page = BT[s][token / P], slot = token mod P. */
static int64_t kv_offset(const job_t *j, int32_t s, int64_t token, int32_t kvh) {
  int64_t page = j->block_tables[(int64_t)s * j->max_blocks + token / j->page_size];
  int64_t slot = token % j->page_size;
  return page * j->stride_page + slot * j->stride_token + (int64_t)kvh * j->stride_head;
}

/* Attention of one query row over the allowed tokens in [t_begin, t_end):
 * logits z_t = scale * q.k_t, M = max z, w_t = exp(z_t - M),
 * O = sum w_t v_t / sum w_t, LSE = M + ln sum w_t.  No allowed token:
 * O = 0, LSE = -inf.  z is scratch of at least t_end - t_begin doubles. */
static void attend(const job_t *j, int32_t s, const uint16_t *qrow, int32_t kvh,
                   int64_t t_begin, int64_t t_end, double *z, double *o, double *lse) {
  const int32_t D = j->head_dim;
  for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
  if (t_end <= t_begin) { *lse = -INFINITY; return; }
  double m = -INFINITY;
  for (int64_t t = t_begin; t < t_end; ++t) {
    const uint16_t *krow = j->k_pool + kv_offset(j, s, t, kvh);
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += bf16_to_f64(qrow[d]) * bf16_to_f64(krow[d]);
    z[t - t_begin] = j->scale * acc;
    if (z[t - t_begin] > m) m = z[t - t_begin];
  }
  double sum = 0.0;
  for (int64_t t = t_begin; t < t_end; ++t) {
    double w = exp(z[t - t_begin] - m);
    sum += w;
    const uint16_t *vrow = j->v_pool + kv_offset(j, s, t, kvh);
    for (int32_t d = 0; d < D; ++d) o[d] += w * bf16_to_f64(vrow[d]);
  }
  for (int32_t d = 0; d < D; ++d) o[d] /= sum;
  *lse = m + log(sum);
}

typedef struct { const job_t *j; int64_t r0, r1; int status; } slice_t;

static void *run_slice(void *arg) {
  slice_t *sl = (slice_t *)arg;
  const job_t *j = sl->j;
  const int32_t Hq = j->num_q_heads, D = j->head_dim;
  const int32_t G = Hq / j->num_kv_heads;
  int32_t max_ctx = 0;
  for (int32_t s = 0; s < j->num_seqs; ++s)
    if (j->context_lens[s] > max_ctx) max_ctx = j->context_lens[s];
  double *z = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
  if (!z) { sl->status = -1; return NULL; }
  for (int64_t r = sl->r0; r < sl->r1; ++r) {
    int64_t flat = j->rows ? j->rows[r] : r;
    int64_t t = flat / Hq;
    int32_t h = (int32_t)(flat % Hq);
    int32_t s = seq_of_token(j, t);
    int64_t q_first = j->query_start_loc ? j->query_start_loc[s] : s;
    int64_t q_len = j->query_start_loc ? j->query_start_loc[s + 1] - q_first : 1;
    int64_t i = t - q_first;
    int64_t L = j->context_lens[s];
    /* allowed set: t' < L, and t' <= L - q_len + i when causal */
    int64_t end = L;
    if (j->causal) {
      int64_t pos = L - q_len + i;
      if (pos + 1 < end) end = pos + 1;
      if (end < 0) end = 0;
    }
    const uint16_t *qrow = j->q + (t * Hq + h) * (int64_t)D;
    int32_t kvh = h / G;
    if (j->split_tokens <= 0) {
      attend(j, s, qrow, kvh, 0, end, z, j->out + r * D, j->lse + r);
    } else {
      for (int32_t k = 0; k < j->num_splits; ++k) {
        int64_t b = (int64_t)k * j->split_tokens;
        int64_t e = b + j->split_tokens;
        if (e > end) e = end;
        attend(j, s, qrow, kvh, b, e, z,
               j->out + (r * j->num_splits + k) * D, j->lse + r * j->num_splits + k);
      }
    }
  }
  free(z);
  sl->status = 0;
  return NULL;
}

static int run_job(const job_t *j, int32_t num_threads) {
  int64_t n = j->rows ? j->num_rows : 0;
  if (!j->rows) {
    int64_t T = j->query_start_loc ? j->query_start_loc[j->num_seqs] : j->num_seqs;
    n = T * j->num_q_heads;
  }
  if (num_threads < 1) num_threads = 1;
  if (num_threads > 256) num_threads = 256;
  if ((int64_t)num_threads > n) num_threads = (int32_t)(n > 0 ? n : 1);
  pthread_t th[256];
  slice_t sl[256];
  for (int32_t i = 0; i < num_threads; ++i) {
    sl[i].j = j;
    sl[i].r0 = n * i / num_threads;
    sl[i].r1 = n * (i + 1) / num_threads;
    sl[i].status = 1;
    if (pthread_create(&th[i], NULL, run_slice, &sl[i]) != 0) {
      run_slice(&sl[i]); /* fall back to the calling thread */
      th[i] = 0;
    }
  }
  int rc = 0;
  for (int32_t i = 0; i < num_threads; ++i) {
    if (th[i]) pthread_join(th[i], NULL);
    if (sl[i].status != 0) rc = -1;
  }
  return rc;
}

static int check_common(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0) return -2;
  if (Hq % Hkv != 0) return -2;
  return 0;
}

/* Single-pass attention for every row (rows == NULL) or the listed rows.
 * query_start_loc == NULL means decode: sequence s owns query token s.
 * Returns 0 on success, negative on bad arguments or allocation failure. */
int pa_oracle_attention(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, const uint16_t *q,
                        const int32_t *query_start_loc, const uint16_t *k_pool,
                        const uint16_t *v_pool, int64_t stride_page, int64_t stride_token,
                        int64_t stride_head, const int32_t *block_tables, int32_t max_blocks,
                        const int32_t *context_lens, float scale, int32_t causal,
                        const int64_t *rows, int64_t num_rows, double *out, double *lse,
                        int32_t num_threads) {
  int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  job_t j = {num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, q, query_start_loc,
             k_pool, v_pool, stride_page, stride_token, stride_head, block_tables,
             max_blocks, context_lens, (double)scale, causal, 0, 1, rows, num_rows, out, lse};
  return run_job(&j, num_threads);
}

/* Split partials: for each row, split k covers logical tokens
 * [k*split_tokens, (k+1)*split_tokens) intersected with the allowed set, and
 * yields its own normalised output O_k and lse_k (O_k = 0, lse_k = -inf when
 * empty).  out is [rows, num_splits, D], lse is [rows, num_splits]. */
int pa_oracle_partials(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size, const uint16_t *q,
                       const int32_t *query_start_loc, const uint16_t *k_pool,
                       const uint16_t *v_pool, int64_t stride_page, int64_t stride_token,
                       int64_t stride_head, const int32_t *block_tables, int32_t max_blocks,
                       const int32_t *context_lens, float scale, int32_t causal,
                       int32_t split_tokens, int32_t num_splits, const int64_t *rows,
                       int64_t num_rows, double *out, double *lse, int32_t num_threads) {
  int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size);
  if (rc) return rc;
  if (split_tokens <= 0 || num_splits <= 0) return -2;
  job_t j = {num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, q, query_start_loc,
             k_pool, v_pool, stride_page, stride_token, stride_head, block_tables,
             max_blocks, context_lens, (double)scale, causal, split_tokens, num_splits,
             rows, num_rows, out, lse};
  return run_job(&j, num_threads);
}

/* Log-sum-exp merge of split partials, per row:
 *   M = max_k lse_k; every lse_k = -inf gives O = 0, LSE = -inf;
 *   otherwise w_k = exp(lse_k - M), O = sum w_k O_k / sum w_k,
 *   LSE = M + ln sum w_k.
 * partial_o is [rows, S, D], partial_lse [rows, S]; out [rows, D], lse [rows]. */
int pa_oracle_merge(const double *partial_o, const double *partial_lse, int64_t rows,
                    int32_t num_splits, int32_t head_dim, double *out, double *lse) {
  if (rows < 0 || num_splits <= 0 || head_dim <= 0) return -2;
  for (int64_t r = 0; r < rows; ++r) {
    const double *pl = partial_lse + r * num_splits;
    double *o = out + r * head_dim;
    for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
    double M = -INFINITY;
    for (int32_t k = 0; k < num_splits; ++k) if (pl[k] > M) M = pl[k];
    if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
    double wsum = 0.0;
    for (int32_t k = 0; k < num_splits; ++k) {
      if (pl[k] == -INFINITY) continue; /* weight exactly zero */
      double w = exp(pl[k] - M);
      wsum += w;
      const double *ok = partial_o + (r * num_splits + k) * head_dim;
      for (int32_t d = 0; d < head_dim; ++d) o[d] += w * ok[d];
    }
    for (int32_t d = 0; d < head_dim; ++d) o[d] /= wsum;
    lse[r] = M + log(wsum);
  }
  return 0;
}

/* Paged KV append: copy the K and V rows of every new token into its slot.
 * k_new, v_new are [T, Hkv, D] bf16 bits, T = query_start_loc[num_seqs]
 * (or num_seqs when query_start_loc is NULL: one token per sequence).
 * For sequence s with q_s new tokens and L_s = context_lens[s], token i
 * (row query_start_loc[s] + i) is logical position L_s - q_s + i; its row
 * for kv head h goes to page BT[s][pos / P], slot pos mod P.  Sequences with
 * L_s < q_s write nothing.  pool_elems bounds every write: a position past
 * the table row or an offset past the pool returns -3 (pools may then be
 * partly written).  Returns 0 on success. */
int pa_oracle_append(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *query_start_loc, uint16_t *k_pool, uint16_t *v_pool,
                     int64_t pool_elems, int64_t stride_page, int64_t stride_token,
                     int64_t stride_head, const int32_t *block_tables, int32_t max_blocks,
                     const int32_t *context_lens) {
  if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 || max_blocks <= 0)
    return -2;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t first = query_start_loc ? query_start_loc[s] : s;
    int64_t q_s = query_start_loc ? (int64_t)query_start_loc[s + 1] - first : 1;
    int64_t L = context_lens[s];
    if (L < q_s) continue;
    for (int64_t i = 0; i < q_s; ++i) {
      int64_t pos = L - q_s + i;
      int64_t block = pos / page_size;
      if (block >= max_blocks) return -3;
      int64_t page = block_tables[(int64_t)s * max_blocks + block];
      int64_t slot = pos % page_size;
      for (int32_t h = 0; h < num_kv_heads; ++h) {
        int64_t dst = page * stride_page + slot * stride_token + (int64_t)h * stride_head;
        int64_t src = ((first + i) * num_kv_heads + h) * (int64_t)head_dim;
        if (page < 0 || dst < 0 || dst + head_dim > pool_elems) return -3;
        for (int32_t d = 0; d < head_dim; ++d) {
          k_pool[dst + d] = k_new[src + d];
          v_pool[dst + d] = v_new[src + d];
        }
      }
    }
  }
  return 0;
}
