/*
 * Float64 CPU oracle for biased, windowed paged attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline, never by the product path. It shares no code,
 * header or table with the HIP library. Semantics and layouts are documented
 * in oracle.h.
 *
 * Every row is computed the slow, obvious way: walk the visible keys in
 * ascending logical position, fetch each key and value through the block
 * table, form the score (q.k + a) * scale in float64, then take the softmax
 * weighted average of the values. No blocking, no online softmax, no reuse.
 * Build: gcc -O2 -fopenmp (never -ffast-math).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element i of an fp32 (dtype 0) or bf16 (dtype 1) array, widened exactly to
 * float64. A bf16 value is the upper half of the fp32 bit pattern. */
static double elem(const void* base, int64_t i, int32_t dtype) {
  if (dtype == 0) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Offset of element (token j, dim 0) of head h in a paged cache, found
 * through the block table row `table` (logical block j / block_size). */
static int64_t kv_offset(const int32_t* table, int32_t j, int32_t h, int32_t num_heads,
                         int32_t block_size, int32_t head_dim) {
  int64_t phys = table[j / block_size];
  int64_t slot = j % block_size;
  return ((phys * num_heads + h) * block_size + slot) * head_dim;
}

/* Whether key j is visible to a query at logical position p: the key must be
 * one of the L cached tokens; with a window W >= 1 it must satisfy
 * |p - j| < W; with chunked local attention of chunk size C >= 1 it must lie
 * in the query's chunk, floor(j / C) = floor(p / C); a causal query also
 * needs j <= p. */
static int visible(int32_t p, int32_t j, int32_t L, int32_t window, int32_t causal,
                   int32_t chunk) {
  if (j < 0 || j >= L) return 0;
  if (causal && j > p) return 0;
  if (window > 0) {
    int32_t d = p > j ? p - j : j - p;
    if (d >= window) return 0;
  }
  if (chunk > 0 && j / chunk != p / chunk) return 0;
  return 1;
}

/* One attention row: query vector q_row (offset q_off into q), keys of the
 * sequence whose block-table row is `table`, bias row `bias_row` indexed by
 * key position (NULL = no bias). Writes head_dim values to out_row.
 * `s` is scratch for L scores. */
static void attend_row(double* out_row, const void* q, int64_t q_off, const void* k_cache,
                       const void* v_cache, const int32_t* table, const float* bias_row,
                       int32_t p, int32_t L, int32_t window, int32_t causal, int32_t chunk,
                       double scale, int32_t h, int32_t num_heads, int32_t head_dim,
                       int32_t block_size, int32_t dtype, double* s) {
  for (int32_t d = 0; d < head_dim; ++d) out_row[d] = 0.0;
  double m = -INFINITY;
  for (int32_t j = 0; j < L; ++j) {
    s[j] = -INFINITY;
    if (!visible(p, j, L, window, causal, chunk)) continue;
    int64_t ko = kv_offset(table, j, h, num_heads, block_size, head_dim);
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d)
      dot += elem(q, q_off + d, dtype) * elem(k_cache, ko + d, dtype);
    double a = bias_row ? (double)bias_row[j] : 0.0;
    s[j] = (dot + a) * scale;
    if (s[j] > m) m = s[j];
  }
  if (L <= 0 || m == -INFINITY) return; /* empty or fully masked row: 0 */
  double z = 0.0;
  for (int32_t j = 0; j < L; ++j) {
    if (s[j] == -INFINITY) continue;
    double w = exp(s[j] - m);
    z += w;
    int64_t vo = kv_offset(table, j, h, num_heads, block_size, head_dim);
    for (int32_t d = 0; d < head_dim; ++d) out_row[d] += w * elem(v_cache, vo + d, dtype);
  }
  for (int32_t d = 0; d < head_dim; ++d) out_row[d] /= z;
}

static int bad_scalars(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                       int32_t sliding_window, int32_t dtype) {
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || block_size < 1) return 1;
  if (max_blocks_per_seq < 0 || max_seq_len < 0) return 1;
  if (sliding_window == 0 || sliding_window < -1) return 1;
  if (dtype != 0 && dtype != 1) return 1;
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return 1;
  return 0;
}

static int decode_rows(double* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const float* attn_bias, int32_t sliding_window, int32_t chunk,
                       double scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                       int32_t dtype) {
  if (chunk < 0) return -1;
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype))
    return -1;
  for (int32_t b = 0; b < num_seqs; ++b)
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len) return -1;
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_seq_len > 0 ? max_seq_len : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      const float* bias_row =
          attn_bias ? attn_bias + ((int64_t)b * num_heads + h) * max_seq_len : NULL;
      /* the decode query is the newest token, at position L - 1 */
      attend_row(out + bh * head_dim, q, bh * head_dim, k_cache, v_cache,
                 block_tables + (int64_t)b * max_blocks_per_seq, bias_row, L - 1, L,
                 sliding_window, 0, chunk, scale, h, num_heads, head_dim, block_size, dtype, s);
    }
    free(s);
  }
  return 0;
}

int oracle_decode_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const float* attn_bias, int32_t sliding_window, double scale,
                      int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                      int32_t dtype) {
  return decode_rows(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias,
                     sliding_window, 0, scale, num_seqs, num_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, dtype);
}

/* Chunked local attention ("[V1] Add sliding window support to Flex
 * Attention backend", review thread on attention groups: Llama 4 alternates
 * full-attention layers with chunked-local-attention layers). The page names
 * the layer type only; the reading taken here is the plain one: positions are
 * cut into consecutive chunks of chunk_size tokens, and a query sees exactly
 * the keys of its own chunk (a causal query only those up to itself). Parity
 * unpinned for that reading. chunk_size >= 1; a decode query (position L - 1)
 * sees keys chunk_size * floor((L - 1) / chunk_size) .. L - 1. */
int oracle_decode_chunked_f64(double* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const float* attn_bias,
                              int32_t chunk_size, double scale, int32_t num_seqs,
                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t dtype) {
  if (chunk_size < 1) return -1;
  return decode_rows(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias, -1,
                     chunk_size, scale, num_seqs, num_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, dtype);
}

static int prefill_rows(double* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* query_start_loc, const float* attn_bias,
                        int32_t sliding_window, int32_t causal, int32_t chunk, double scale,
                        int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                        int32_t dtype) {
  if (chunk < 0) return -1;
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype))
    return -1;
  if (causal != 0 && causal != 1) return -1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t nq = query_start_loc[b + 1] - query_start_loc[b];
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len || nq < 0 || nq > context_lens[b])
      return -1;
  }
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_seq_len > 0 ? max_seq_len : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      int32_t q0 = query_start_loc[b];
      int32_t nq = query_start_loc[b + 1] - q0;
      for (int32_t t = 0; t < nq; ++t) {
        int32_t p = L - nq + t; /* queries are the last nq positions */
        int64_t row = ((int64_t)(q0 + t) * num_heads + h) * head_dim;
        const float* bias_row =
            attn_bias
                ? attn_bias + (((int64_t)b * num_heads + h) * max_seq_len + p) * max_seq_len
                : NULL;
        attend_row(out + row, q, row, k_cache, v_cache,
                   block_tables + (int64_t)b * max_blocks_per_seq, bias_row, p, L,
                   sliding_window, causal, chunk, scale, h, num_heads, head_dim, block_size,
                   dtype, s);
      }
    }
    free(s);
  }
  return 0;
}

int oracle_prefill_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start_loc, const float* attn_bias,
                       int32_t sliding_window, int32_t causal, double scale,
                       int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                       int32_t dtype) {
  return prefill_rows(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      attn_bias, sliding_window, causal, 0, scale, num_seqs, num_heads,
                      head_dim, block_size, max_blocks_per_seq, max_seq_len, dtype);
}

int oracle_prefill_chunked_f64(double* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               const float* attn_bias, int32_t chunk_size, int32_t causal,
                               double scale, int32_t num_seqs, int32_t num_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t max_seq_len,
                               int32_t dtype) {
  if (chunk_size < 1) return -1;
  return prefill_rows(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      attn_bias, -1, causal, chunk_size, scale, num_seqs, num_heads, head_dim,
                      block_size, max_blocks_per_seq, max_seq_len, dtype);
}

/* ------------------------------------------------------------------------
 * T5 relative-position bias
 *
 * "[Kernel][Model] PagedAttention: Support custom attention bias for T5
 * model (1/2)" names an in-kernel computation of T5's relative-position bias
 * as the model-specific alternative to a materialised bias, and its T5
 * max-distance remark states that beyond the maximum distance (128 for T5)
 * the last bias value is reused. The bucketing is T5's published one:
 * relative position r = key position - query position; a bidirectional
 * (encoder) bias gives keys after the query (r > 0) the upper half of the
 * buckets and uses |r|, a unidirectional (decoder) bias uses max(-r, 0).
 * With nb buckets in the half in use, distances below nb/2 get their own
 * bucket; larger ones are spaced logarithmically up to max_distance, and
 * every distance beyond lands in the last bucket. Evaluated in float64.
 * ---------------------------------------------------------------------- */
int oracle_t5_bucket(int64_t relative_position, int32_t bidirectional, int32_t num_buckets,
                     int32_t max_distance) {
  int32_t ret = 0, nb = num_buckets;
  int64_t n;
  if (bidirectional) {
    nb = num_buckets / 2;
    if (relative_position > 0) ret = nb;
    n = relative_position < 0 ? -relative_position : relative_position;
  } else {
    n = relative_position < 0 ? -relative_position : 0;
  }
  int32_t max_exact = nb / 2;
  if (n < max_exact) return ret + (int32_t)n;
  double v = (double)max_exact + floor(log((double)n / (double)max_exact) /
                                       log((double)max_distance / (double)max_exact) *
                                       (double)(nb - max_exact));
  int32_t b = v > (double)(nb - 1) ? nb - 1 : (int32_t)v;
  return ret + b;
}

void oracle_t5_bucket_array(const int64_t* relative_position, int64_t n, int32_t bidirectional,
                            int32_t num_buckets, int32_t max_distance, int32_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = oracle_t5_bucket(relative_position[i], bidirectional, num_buckets, max_distance);
}

static int bad_relpos(int32_t num_buckets, int32_t max_distance, int32_t bidirectional) {
  int32_t nb = bidirectional ? num_buckets / 2 : num_buckets;
  if (bidirectional != 0 && bidirectional != 1) return 1;
  if (num_buckets < 2 || (bidirectional && num_buckets % 2)) return 1;
  if (nb / 2 < 1 || max_distance <= nb / 2) return 1;
  return 0;
}

/* Decode with the bias taken from a T5 bucket table rel_table [H, num_buckets]:
 * a_j = rel_table[h][bucket(j - (L-1))]; otherwise exactly oracle_decode_f64. */
int oracle_decode_relpos_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const float* rel_table, int32_t num_buckets, int32_t max_distance,
                             int32_t bidirectional, int32_t sliding_window, double scale,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                             int32_t dtype) {
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype) ||
      bad_relpos(num_buckets, max_distance, bidirectional))
    return -1;
  for (int32_t b = 0; b < num_seqs; ++b)
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len) return -1;
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    size_t n = (size_t)(max_seq_len > 0 ? max_seq_len : 1);
    double* s = (double*)malloc(sizeof(double) * n);
    float* a = (float*)malloc(sizeof(float) * n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      for (int32_t j = 0; j < L; ++j)
        a[j] = rel_table[(int64_t)h * num_buckets +
                         oracle_t5_bucket((int64_t)j - (L - 1), bidirectional, num_buckets,
                                          max_distance)];
      attend_row(out + bh * head_dim, q, bh * head_dim, k_cache, v_cache,
                 block_tables + (int64_t)b * max_blocks_per_seq, a, L - 1, L, sliding_window, 0,
                 0, scale, h, num_heads, head_dim, block_size, dtype, s);
    }
    free(s);
    free(a);
  }
  return 0;
}

/* Prefill with the T5 bias: a(p, j) = rel_table[h][bucket(j - p)]. */
int oracle_prefill_relpos_f64(double* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start_loc,
                              const float* rel_table, int32_t num_buckets, int32_t max_distance,
                              int32_t bidirectional, int32_t sliding_window, int32_t causal,
                              double scale, int32_t num_seqs, int32_t num_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int32_t dtype) {
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype) ||
      bad_relpos(num_buckets, max_distance, bidirectional))
    return -1;
  if (causal != 0 && causal != 1) return -1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t nq = query_start_loc[b + 1] - query_start_loc[b];
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len || nq < 0 || nq > context_lens[b])
      return -1;
  }
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    size_t n = (size_t)(max_seq_len > 0 ? max_seq_len : 1);
    double* s = (double*)malloc(sizeof(double) * n);
    float* a = (float*)malloc(sizeof(float) * n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      int32_t q0 = query_start_loc[b];
      int32_t nq = query_start_loc[b + 1] - q0;
      for (int32_t t = 0; t < nq; ++t) {
        int32_t p = L - nq + t;
        for (int32_t j = 0; j < L; ++j)
          a[j] = rel_table[(int64_t)h * num_buckets +
                           oracle_t5_bucket((int64_t)j - p, bidirectional, num_buckets,
                                            max_distance)];
        int64_t row = ((int64_t)(q0 + t) * num_heads + h) * head_dim;
        attend_row(out + row, q, row, k_cache, v_cache,
                   block_tables + (int64_t)b * max_blocks_per_seq, a, p, L, sliding_window,
                   causal, 0, scale, h, num_heads, head_dim, block_size, dtype, s);
      }
    }
    free(s);
    free(a);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Ragged bias layout: the variable-length alternative to padding the bias
 * to max_seq_len that the custom-bias PR description names as a later
 * optimisation. Sequence b's bias starts at element bias_start[b] of one
 * packed buffer: decode rows [H][L_b] (a = bias[start + h*L_b + j]), prefill
 * rows [H][n_q][L_b] (a = bias[start + (h*n_q + t)*L_b + j]).
 * ---------------------------------------------------------------------- */
int oracle_decode_ragged_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const float* bias, const int64_t* bias_start,
                             int32_t sliding_window, double scale, int32_t num_seqs,
                             int32_t num_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t dtype) {
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype) || !bias || !bias_start)
    return -1;
  for (int32_t b = 0; b < num_seqs; ++b)
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len) return -1;
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_seq_len > 0 ? max_seq_len : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      const float* bias_row = bias + bias_start[b] + (int64_t)h * L;
      attend_row(out + bh * head_dim, q, bh * head_dim, k_cache, v_cache,
                 block_tables + (int64_t)b * max_blocks_per_seq, bias_row, L - 1, L,
                 sliding_window, 0, 0, scale, h, num_heads, head_dim, block_size, dtype, s);
    }
    free(s);
  }
  return 0;
}

int oracle_prefill_ragged_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start_loc, const float* bias,
                              const int64_t* bias_start, int32_t sliding_window, int32_t causal,
                              double scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                              int32_t dtype) {
  if (bad_scalars(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                  sliding_window, dtype) || !bias || !bias_start)
    return -1;
  if (causal != 0 && causal != 1) return -1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int32_t nq = query_start_loc[b + 1] - query_start_loc[b];
    if (context_lens[b] < 0 || context_lens[b] > max_seq_len || nq < 0 || nq > context_lens[b])
      return -1;
  }
  int64_t pairs = (int64_t)num_seqs * num_heads;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_seq_len > 0 ? max_seq_len : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      int32_t b = (int32_t)(bh / num_heads), h = (int32_t)(bh % num_heads);
      int32_t L = context_lens[b];
      int32_t q0 = query_start_loc[b];
      int32_t nq = query_start_loc[b + 1] - q0;
      for (int32_t t = 0; t < nq; ++t) {
        int32_t p = L - nq + t;
        int64_t row = ((int64_t)(q0 + t) * num_heads + h) * head_dim;
        const float* bias_row = bias + bias_start[b] + ((int64_t)h * nq + t) * L;
        attend_row(out + row, q, row, k_cache, v_cache,
                   block_tables + (int64_t)b * max_blocks_per_seq, bias_row, p, L,
                   sliding_window, causal, 0, scale, h, num_heads, head_dim, block_size, dtype,
                   s);
      }
    }
    free(s);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * KV-cache write: the step before decode. Token t's keys and values (all
 * heads) go to physical slot slot_mapping[t] = block * block_size + offset
 * of the paged caches (the block-table layout of "Add Encoder-decoder model
 * support and T5 Model support"); a negative slot means "skip this token".
 * Element-by-element copy; slots must be distinct.
 * ---------------------------------------------------------------------- */
int oracle_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype) {
  if (num_tokens < 0 || num_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 0 ||
      (dtype != 0 && dtype != 1))
    return -1;
  const size_t es = dtype == 0 ? 4 : 2;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= num_blocks * block_size) return -1;
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int32_t h = 0; h < num_heads; ++h) {
      int64_t src = ((int64_t)t * num_heads + h) * head_dim;
      int64_t dst = ((blk * num_heads + h) * block_size + off) * head_dim;
      for (int32_t d = 0; d < head_dim; ++d) {
        memcpy((char*)k_cache + (dst + d) * es, (const char*)k_new + (src + d) * es, es);
        memcpy((char*)v_cache + (dst + d) * es, (const char*)v_new + (src + d) * es, es);
      }
    }
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
