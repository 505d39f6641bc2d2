/*
 * paged_attn.h — C ABI of the MI355X (gfx950) biased, windowed paged-attention
 * library (libpaged_attn.so).
 *
 * The library computes, per query row,
 *     out = softmax((q K^T + A) * scale) V,
 * the attention-with-additive-bias formula of "[Kernel][Model] PagedAttention:
 * Support custom attention bias for T5 model (1/2)" (vllm-project/vllm#11334,
 * PR description), with `scale` standing for 1/sqrt(d_k). A is an optional,
 * fully materialised fp32 bias padded to max_seq_len (same PR description);
 * a NULL bias pointer is a no-op (same page, review answer on whether the bias
 * is materialised when unused). Keys and values are read through a block
 * table; cross-attention simply passes the encoder's block table ("Add
 * Encoder-decoder model support and T5 Model support", vllm-project/vllm#3117,
 * the thread that settles on separate self- and cross-attention block tables).
 * The optional sliding window follows "[V1] Add sliding window support to Flex
 * Attention backend" (vllm-project/vllm#24089).
 *
 * Scores, masks and positions (readings where the pages are silent):
 *   s_j = (q . k_j + a_j) * scale          (bias added before the scale)
 *   a query at logical position p sees key j iff  0 <= j < L  and, when
 *   sliding_window = W >= 1, |p - j| < W; a causal query also needs j <= p.
 *   Decode: the query is at p = L - 1. Prefill: the n_q queries of a sequence
 *   are at p = L - n_q .. L - 1 (n_q = L for an encoder: query t at t).
 *   A row with L = 0, or whose every score is -inf, outputs 0.
 *
 * Layouts (all row-major, all device memory owned by the caller):
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim], dtype
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]; entry n is the
 *                     physical block of logical tokens 16n .. 16n+15. Entries
 *                     that back no visible token are never read (table
 *                     padding, and with a window the blocks wholly before it).
 *   context_lens      int32 [num_seqs], 0 <= L <= max_seq_len
 *   attn_bias         fp32, decode [num_seqs, num_heads, max_seq_len],
 *                     prefill [num_seqs, num_heads, max_seq_len, max_seq_len],
 *                     indexed by logical positions (prefill: [query position]
 *                     [key position]); an entry is read only when its query is
 *                     one of the call's queries and its key is visible to that
 *                     query, so every other entry may hold anything (NaN
 *                     included). NULL = no bias.
 *
 * Conventions of every entry point:
 *   - returns a pa_status_t; never aborts or throws; pa_last_error() gives a
 *     message for the last non-OK status of the calling thread;
 *   - scalar arguments, pointer nullness and alignment are validated on the
 *     host BEFORE any HIP call; the contents of device arrays (lengths, table
 *     entries) are not validated unless the environment variable
 *     PA_VALIDATE=1 is set, in which case they are copied to the host
 *     (synchronously) and range-checked first. Without it the kernels still
 *     refuse to go out of range on bad lengths: a decode sequence whose L is
 *     outside [0, max_seq_len] gets a zero output, and a prefill sequence
 *     with L > max_seq_len, n_q outside [0, L] or query rows outside
 *     [0, total_q) is skipped (its rows are left unwritten). Block-table
 *     entries are used as given: an entry outside [0, num_blocks) that backs
 *     a visible token can fault the device;
 *   - work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream); device faults surface at the caller's next sync;
 *   - the library allocates nothing and keeps no state between calls that
 *     could change a result (only a per-thread memo of the T5 bucket
 *     thresholds, a pure function of the bucket shape); calls on different
 *     streams with distinct outputs/workspaces may overlap.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

/* The two range enumerators are not dtypes: they make the enum span every
 * int32 value, so that any integer a caller passes is a valid value of the
 * type, which the library then rejects as unsupported (in C++ an enum holding
 * a value outside its enumerators' range is undefined behaviour). */
typedef enum {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1,
  PA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  PA_DTYPE_RANGE_MAX_ = 0x7fffffff
} pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                        */
  PA_ERR_INVALID_ARG = 2,  /* a scalar is out of range / PA_VALIDATE found bad data */
  PA_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head_dim, block_size ...) */
  PA_ERR_MISALIGNED = 4,   /* q/k/v/out not 16-byte aligned, bias not 4-byte     */
  PA_ERR_WORKSPACE = 5,    /* decode workspace missing or too small              */
  PA_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed          */
} pa_status_t;

/* PA_ABI_VERSION of the built library. */
int pa_abi_version(void);

/* Thread-local message describing the last non-OK status ("" if none). */
const char* pa_last_error(void);

/* Partition length (tokens, a multiple of 16) the decode path uses when
 * partition_tokens = 0 is passed, for this problem shape. */
int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                    int32_t max_seq_len, int32_t sliding_window,
                                    pa_dtype_t dtype);

/* Bytes of device workspace paged_attn_decode needs for this shape and
 * partition length (0 = the default partition). 0 means no workspace is
 * needed (every sequence fits one partition). Returns 0 also for invalid
 * arguments; paged_attn_decode reports those. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t sliding_window,
                                 int32_t partition_tokens, pa_dtype_t dtype);

/*
 * Decode attention: one query per (sequence, head), at position L-1, for
 * decoder self-attention (the sequence's own table) or cross-attention (the
 * encoder table and encoder lengths, sliding_window = -1). See the header
 * comment for the formula and visibility rule.
 *
 *   out            [num_seqs, num_heads, head_dim], dtype (written)
 *   q              [num_seqs, num_heads, head_dim], dtype
 *   k_cache/v_cache, block_tables, context_lens, attn_bias: see above
 *                  (attn_bias [num_seqs, num_heads, max_seq_len] or NULL)
 *   sliding_window -1 (off) or >= 1: the W newest tokens stay visible
 *   scale          finite; normally 1/sqrt(head_dim)
 *   num_kv_heads   must equal num_heads in this version
 *   head_dim       64 or 128;  block_size  16
 *   max_blocks_per_seq * 16 >= max_seq_len
 *   num_blocks     rows of the caches (used by PA_VALIDATE only)
 *   dtype          PA_DTYPE_F32 or PA_DTYPE_BF16 for q, caches and out
 *   partition_tokens  0 = default; else a multiple of 16 in [16, 4096]: the
 *                  split-K partition length (each partition is one workgroup;
 *                  a second kernel merges partitions in a fixed order)
 *   workspace      device memory of >= pa_decode_workspace_bytes(...) bytes,
 *                  256-byte aligned; may be NULL when that size is 0. Its
 *                  contents need no initialisation and are scratch.
 *   stream         hipStream_t or NULL
 * Errors: NULL_POINTER, INVALID_ARG, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP.
 * num_seqs == 0 returns PA_OK without launching anything.
 */
pa_status_t paged_attn_decode(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const float* attn_bias,
                              int32_t sliding_window, float scale, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                              int32_t partition_tokens, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Arguments and results are those of paged_attn_decode without
 * the workspace. When the shape needs split-K partials, they go to a
 * file-scope device array of PA_NOALLOC_SCRATCH_BYTES bytes that each GPU
 * the library runs on holds until the process ends; a shape whose
 * pa_decode_workspace_bytes(...) exceeds that size is rejected with
 * PA_ERR_WORKSPACE before any launch. The entry point calls no hipMalloc,
 * hipFree or other allocating routine (set PA_VALIDATE only where host
 * copies and a stream synchronisation are acceptable). The array's address
 * on a device is looked up on the first call there (the device of `stream`,
 * or the current device for the null stream).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, other threads) race and may return wrong
 * results; serialise them. Nothing in the array needs clearing between
 * calls (each call writes every partial it reads).
 * Errors: as paged_attn_decode, plus UNSUPPORTED for a device index >= 64.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status_t paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const float* attn_bias,
                                      int32_t sliding_window, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                                      int32_t partition_tokens, void* stream);

/*
 * Prefill attention over packed queries, for bidirectional encoder-only
 * attention (causal = 0; n_q = L per sequence) or causal decoder prompts
 * (causal = 1). Uses MFMA for both contractions.
 *
 *   out             [total_q, num_heads, head_dim], dtype (written)
 *   q               [total_q, num_heads, head_dim], dtype
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, query_start_loc[0]
 *                   = 0, query_start_loc[num_seqs] = total_q; sequence b owns
 *                   rows query_start_loc[b] .. query_start_loc[b+1]-1 and
 *                   0 <= n_q <= L must hold
 *   attn_bias       [num_seqs, num_heads, max_seq_len, max_seq_len] fp32, or NULL
 *   causal          0 or 1
 *   dtype           PA_DTYPE_F32 or PA_DTYPE_BF16 (bf16: bf16 MFMA with fp32
 *                   accumulation; the softmax weights enter P.V as bf16.
 *                   fp32: fp32 accuracy; at head_dim 64 both contractions run
 *                   on the bf16 matrix cores with every fp32 operand split
 *                   exactly into three bf16 parts, at 128 on fp32 MFMA)
 *   Other arguments as for paged_attn_decode. No workspace is needed.
 *   The launch has one workgroup per (sequence, head) and per 64 or 128
 *   query rows of max_seq_len; those past a sequence's own length only read
 *   its metadata and exit, so a max_seq_len far above the batch's longest
 *   sequence costs launch time (e.g. 256 sequences of 128 tokens: 2.6x the
 *   time with max_seq_len 1024 as with 128).
 *   total_q = 0 computes nothing and returns PA_OK after the scalar checks;
 *   then no device pointer is read and any of them may be NULL (the same
 *   holds for the ragged-bias variant below; the relpos variant still checks
 *   its bucket table).
 * Errors: NULL_POINTER, INVALID_ARG, UNSUPPORTED, MISALIGNED, HIP.
 */
pa_status_t paged_attn_prefill(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               const float* attn_bias, int32_t sliding_window, int32_t causal,
                               float scale, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t max_seq_len,
                               int64_t num_blocks, int64_t total_q, pa_dtype_t dtype,
                               void* stream);

/*
 * In-kernel T5 relative-position bias: the same decode / prefill, with the
 * bias of key j for a query at position p computed from a bucket table
 * instead of read from a materialised matrix — the model-specific
 * alternative named in "[Kernel][Model] PagedAttention: Support custom
 * attention bias for T5 model (1/2)" (PR description, and its T5
 * max-distance remark: beyond the maximum distance the last value is reused).
 *
 *   a(p, j) = rel_table[h * num_buckets + bucket(j - p)]
 *
 * T5 bucketing of r = j - p: a unidirectional (decoder) table uses
 * n = max(-r, 0) over all num_buckets buckets; a bidirectional (encoder)
 * table gives r > 0 the upper half (offset num_buckets/2) and uses n = |r|.
 * Within a direction of `half` buckets, n < half/2 is its own bucket; larger
 * n get half/2 + floor(log(n / (half/2)) / log(max_distance / (half/2)) *
 * (half - half/2)), capped at half - 1, evaluated in float64 on the host.
 * Scores are (q.k + a) * scale as with a materialised bias, so a table whose
 * buckets reproduce a materialised bias gives the identical result.
 *
 *   rel_table      fp32 [num_heads, num_buckets], device memory, not NULL
 *   num_buckets    2..64 (even when bidirectional); T5 uses 32
 *   max_distance   (half/2, 1024]; T5 uses 128
 *   bidirectional  0 (decoder self-attention) or 1 (encoder)
 * Everything else as for paged_attn_decode / paged_attn_prefill (there is no
 * attn_bias argument). Errors as there, plus INVALID_ARG / NULL_POINTER /
 * MISALIGNED for the table arguments.
 */
pa_status_t paged_attn_decode_relpos(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const float* rel_table,
                                     int32_t num_buckets, int32_t max_distance,
                                     int32_t bidirectional, int32_t sliding_window, float scale,
                                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size,
                                     int32_t max_blocks_per_seq, int32_t max_seq_len,
                                     int64_t num_blocks, pa_dtype_t dtype,
                                     int32_t partition_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream);

pa_status_t paged_attn_prefill_relpos(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens,
                                      const int32_t* query_start_loc, const float* rel_table,
                                      int32_t num_buckets, int32_t max_distance,
                                      int32_t bidirectional, int32_t sliding_window,
                                      int32_t causal, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len, int64_t num_blocks, int64_t total_q,
                                      pa_dtype_t dtype, void* stream);

/*
 * Ragged (unpadded) bias layout — the "variable len bias matrix" the custom
 * bias PR description lists as a later optimisation of the padded layout.
 * One packed fp32 buffer holds every sequence's bias back to back; sequence
 * b's part starts at element bias_start[b]:
 *   decode   rows [num_heads][L_b]:       a(b,h,j)   = attn_bias[bias_start[b] + h*L_b + j]
 *   prefill  rows [num_heads][n_q][L_b]:  a(b,h,t,j) = attn_bias[bias_start[b] + (h*n_q + t)*L_b + j]
 * (t = query index within the sequence, j = key position). attn_bias and
 * bias_start (int64 [num_seqs], 8-byte aligned) are device memory and must
 * not be NULL (except for a prefill with total_q = 0). Everything else as for
 * paged_attn_decode / paged_attn_prefill.
 */
pa_status_t paged_attn_decode_ragged_bias(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, const float* attn_bias,
                                          const int64_t* bias_start, int32_t sliding_window,
                                          float scale, int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq,
                                          int32_t max_seq_len, int64_t num_blocks,
                                          pa_dtype_t dtype, int32_t partition_tokens,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

pa_status_t paged_attn_prefill_ragged_bias(void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens,
                                           const int32_t* query_start_loc,
                                           const float* attn_bias, const int64_t* bias_start,
                                           int32_t sliding_window, int32_t causal, float scale,
                                           int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_blocks_per_seq,
                                           int32_t max_seq_len, int64_t num_blocks,
                                           int64_t total_q, pa_dtype_t dtype, void* stream);

/*
 * Chunked local attention ("[V1] Add sliding window support to Flex Attention
 * backend", the attention-groups thread: Llama 4 alternates full-attention
 * layers with chunked-local-attention layers, a mask family beside the
 * sliding window). The page names the layer type only; these entry points
 * take its plain reading: positions are cut into consecutive chunks of
 * chunk_size tokens (chunk c holds positions c*chunk_size ..
 * c*chunk_size + chunk_size - 1), and a query at position p sees exactly the
 * keys of its own chunk, floor(j / chunk_size) == floor(p / chunk_size); a
 * causal prefill query also needs j <= p. The decode query (position L-1)
 * therefore sees keys chunk_size * floor((L-1) / chunk_size) .. L-1; blocks
 * before that chunk are never read.
 *
 * Arguments are those of paged_attn_decode / paged_attn_prefill with
 * chunk_size (>= 1, else PA_ERR_INVALID_ARG) in place of sliding_window; there
 * is no window. The optional attn_bias is the padded materialised bias of the
 * base entry points. The decode workspace is sized by
 * pa_decode_workspace_bytes with sliding_window = chunk_size (a chunk spans
 * at most as many tokens as a window of that size). With PA_VALIDATE=1 the
 * block-table entries from the first query's chunk onwards are checked.
 */
pa_status_t paged_attn_decode_chunked(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const float* attn_bias,
                                      int32_t chunk_size, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream);

pa_status_t paged_attn_prefill_chunked(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens,
                                       const int32_t* query_start_loc, const float* attn_bias,
                                       int32_t chunk_size, int32_t causal, float scale,
                                       int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, int64_t num_blocks, int64_t total_q,
                                       pa_dtype_t dtype, void* stream);

/*
 * KV-cache write, the step that precedes decode: token t's keys and values
 * (all heads) are stored at physical slot slot_mapping[t] = block * 16 +
 * offset of the paged caches (layout above; the block tables themselves are
 * the caller's). A negative slot skips the token. Slots must be distinct
 * within one call (otherwise the surviving row is unspecified).
 *
 *   k_cache, v_cache  [num_blocks, num_kv_heads, 16, head_dim], dtype (written)
 *   k_new, v_new      [num_tokens, num_heads, head_dim], dtype, 16-byte aligned
 *   slot_mapping      int64 [num_tokens], device memory, 8-byte aligned
 *   num_blocks        rows of the caches (PA_VALIDATE range-checks the slots)
 * Errors: NULL_POINTER, INVALID_ARG, UNSUPPORTED, MISALIGNED, HIP.
 * num_tokens == 0 returns PA_OK without launching.
 */
pa_status_t paged_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, pa_dtype_t dtype, void* stream);

/*
 * Sliding-window eviction: the first logical block a decode query of a
 * sequence with context_len tokens (query at context_len - 1) can read under
 * sliding_window; every later decode step of the same sequence starts at or
 * after it. Blocks before it will never be read again by paged_attn_decode
 * with this window and may be freed or reused (their block-table entries are
 * never read either) — the condition under which "[V1] Add sliding window
 * support to Flex Attention backend" (end-to-end remark) lets in-window
 * iteration skip evicted blocks. 0 when there is no window. No HIP call.
 */
int32_t pa_window_first_live_block(int32_t context_len, int32_t sliding_window);

/*
 * Host-side range check of decode/prefill metadata held in HOST memory (the
 * check PA_VALIDATE=1 runs on copies): every L in [0, max_seq_len], every
 * block-table entry that backs a visible token in [0, num_blocks), and, when
 * query_start_loc is not NULL, 0 = qsl[0] <= ... <= qsl[num_seqs] = total_q
 * with 0 <= n_q <= L. Returns PA_OK or PA_ERR_INVALID_ARG (message in
 * pa_last_error()). Makes no HIP call.
 */
pa_status_t pa_check_metadata(const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t sliding_window,
                              int32_t causal, int32_t num_seqs, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int64_t num_blocks, int64_t total_q);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_ATTN_H */
