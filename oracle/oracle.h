/*
 * Float64 CPU oracle for biased, windowed paged attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code with the HIP library.
 *
 * What it computes is the plain definition of attention with an additive bias,
 *     out = softmax((q K^T + A) / sqrt(d_k)) V,
 * as written in the description of "[Kernel][Model] PagedAttention: Support
 * custom attention bias for T5 model (1/2)" (vllm-project/vllm#11334), with
 * `scale` standing for 1/sqrt(d_k). K and V are read through a per-sequence
 * block table, one table per call; cross-attention passes the encoder table
 * ("Add Encoder-decoder model support and T5 Model support",
 * vllm-project/vllm#3117, the review thread that settles on separate self- and
 * cross-attention block tables). The optional sliding window follows
 * "[V1] Add sliding window support to Flex Attention backend"
 * (vllm-project/vllm#24089).
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes of the repository):
 *   - scores are s_j = (q.k_j + a_j) * scale: the bias is added before the
 *     1/sqrt(d_k) factor, literally as in the formula;
 *   - a query at logical position p sees key j when j < L and, with a window
 *     W >= 1, |p - j| < W; a causal query additionally needs j <= p;
 *   - decode: the query sits at position L-1 (context_lens counts the cached
 *     tokens including the current one);
 *   - prefill: the n_q queries of a sequence sit at positions L-n_q .. L-1
 *     (n_q = L for an encoder, so query t is at position t);
 *   - an empty row (L = 0) or a row whose every score is -inf gives 0;
 *   - a null bias pointer means A = 0 exactly.
 * Parity unpinned for the readings themselves: no page prints an example that
 * tells bias-before-scale from bias-after-scale, the query position, or the
 * window's edge (|p - j| < W against <= W), nor the T5 bucket boundaries
 * between the exact range and the maximum distance. The tests pin that this
 * code computes what the readings say (library cross-checks, closed forms,
 * special cases), not the readings.
 *
 * Layouts (row-major, element type chosen by `dtype`: 0 = fp32, 1 = bf16 given
 * as raw 16-bit patterns):
 *   q        decode [num_seqs, H, D]        prefill [total_q, H, D]
 *   k_cache, v_cache  [num_blocks, H, block_size, D]
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]
 *   context_lens      int32 [num_seqs]
 *   query_start_loc   int32 [num_seqs + 1]   (prefill)
 *   attn_bias   fp32, decode [num_seqs, H, max_seq_len],
 *               prefill [num_seqs, H, max_seq_len, max_seq_len], or NULL
 *   out         float64, same shape as q.
 * Return value: 0 on success, -1 on an invalid scalar argument, a length
 * outside [0, max_seq_len], or (prefill) a query count outside [0, L].
 */
#ifndef PAGED_ATTN_ORACLE_H
#define PAGED_ATTN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oracle_decode_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const float* attn_bias, int32_t sliding_window, double scale,
                      int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                      int32_t dtype);

int oracle_prefill_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start_loc, const float* attn_bias,
                       int32_t sliding_window, int32_t causal, double scale,
                       int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                       int32_t dtype);

/* Chunked local attention: as above with no window, but a query at position
 * p sees only keys j with floor(j / chunk_size) = floor(p / chunk_size) (and,
 * for a causal query, j <= p). chunk_size >= 1. Parity unpinned for this
 * reading: the page that names the layer type gives no formula. */
int oracle_decode_chunked_f64(double* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const float* attn_bias,
                              int32_t chunk_size, double scale, int32_t num_seqs,
                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t dtype);
int oracle_prefill_chunked_f64(double* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               const float* attn_bias, int32_t chunk_size, int32_t causal,
                               double scale, int32_t num_seqs, int32_t num_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t max_seq_len,
                               int32_t dtype);

/* T5 relative-position bucket of relative_position = key - query position
 * (see oracle.c for the definition); bidirectional 0 (decoder) or 1
 * (encoder). The array form fills out[i] for relative_position[i]. */
int oracle_t5_bucket(int64_t relative_position, int32_t bidirectional, int32_t num_buckets,
                     int32_t max_distance);
void oracle_t5_bucket_array(const int64_t* relative_position, int64_t n, int32_t bidirectional,
                            int32_t num_buckets, int32_t max_distance, int32_t* out);

/* Decode / prefill with the bias computed from a T5 bucket table
 * rel_table [num_heads, num_buckets] (fp32): a(p, j) = rel_table[h][bucket(j - p)]. */
int oracle_decode_relpos_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const float* rel_table, int32_t num_buckets, int32_t max_distance,
                             int32_t bidirectional, int32_t sliding_window, double scale,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                             int32_t dtype);
int oracle_prefill_relpos_f64(double* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start_loc,
                              const float* rel_table, int32_t num_buckets, int32_t max_distance,
                              int32_t bidirectional, int32_t sliding_window, int32_t causal,
                              double scale, int32_t num_seqs, int32_t num_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int32_t dtype);

/* Ragged bias layout: sequence b's bias starts at bias[bias_start[b]];
 * decode rows [H][L_b], prefill rows [H][n_q][L_b]. Otherwise as above. */
int oracle_decode_ragged_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const float* bias, const int64_t* bias_start,
                             int32_t sliding_window, double scale, int32_t num_seqs,
                             int32_t num_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t dtype);
int oracle_prefill_ragged_f64(double* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start_loc, const float* bias,
                              const int64_t* bias_start, int32_t sliding_window, int32_t causal,
                              double scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                              int32_t dtype);

/* Scatter num_tokens new key/value rows [num_tokens, num_heads, head_dim]
 * into the paged caches at physical slots slot_mapping[t] (block * block_size
 * + offset; negative = skip). Returns -1 on a slot outside the pool. */
int oracle_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype);

/* Number of OpenMP threads the oracle uses (for reporting). */
int oracle_num_threads(void);
/* Threads the following calls use (n >= 1; timing only, results do not depend on it). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
