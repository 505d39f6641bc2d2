// Host side of the C ABI declared in include/paged_attn.h: argument
// validation (before any HIP call), partition sizing, workspace carving,
// optional range checks of device metadata, and kernel dispatch.
#include "paged_attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local char g_err[512] = "";

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

pa_status_t ok() {
  g_err[0] = '\0';
  return PA_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Tokens a decode partition grid must cover per sequence: every visible token
// plus the part of the first block before the window.
int32_t decode_span(int32_t max_seq_len, int32_t window) {
  if (window > 0 && (int64_t)window + pa::kBlockSize - 1 < max_seq_len)
    return window + pa::kBlockSize - 1;
  return max_seq_len;
}

int32_t round_up16(int32_t x) { return (x + pa::kBlockSize - 1) / pa::kBlockSize * pa::kBlockSize; }

int32_t default_partition(int32_t num_seqs, int32_t num_heads, int32_t max_seq_len,
                          int32_t window) {
  const int32_t span = decode_span(max_seq_len, window);
  const int64_t pairs = (int64_t)num_seqs * num_heads;
  // Long partitions stream best (fewer partial blocks, no merge launch):
  // split only until there are >= 512 workgroups (2 per CU), never below
  // 128 tokens. Measured on MI355X: one partition per (sequence, head) is
  // fastest from 512 pairs up (T5-small decode 14.6 us vs 19.1 us at P=128).
  int32_t P = pa::kMaxPartition;
  while (P > 128 && pairs * ((span + P - 1) / P) < 512) P /= 2;
  if (span <= P) P = span > 0 ? round_up16(span) : pa::kBlockSize;  // one partition
  return P;
}

struct DecodePlan {
  int32_t partition;
  int32_t num_partitions;
  size_t ws_bytes;
  size_t off_m, off_l;   // byte offsets of the m and l arrays (o starts at 0)
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                       int32_t max_seq_len, int32_t window, int32_t partition) {
  DecodePlan p{};
  p.partition = partition > 0 ? partition : default_partition(num_seqs, num_heads, max_seq_len,
                                                               window);
  const int32_t span = decode_span(max_seq_len, window);
  p.num_partitions = span > 0 ? (span + p.partition - 1) / p.partition : 1;
  if (p.num_partitions <= 1) {
    p.num_partitions = 1;
    p.ws_bytes = 0;
    return p;
  }
  const size_t rows = (size_t)num_seqs * num_heads * p.num_partitions;
  auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
  p.off_m = up256(rows * head_dim * sizeof(float));
  p.off_l = p.off_m + up256(rows * sizeof(float));
  p.ws_bytes = p.off_l + up256(rows * sizeof(float));
  return p;
}

pa_status_t check_common(const void* out, const void* q, const void* k, const void* v,
                         const int32_t* bt, const int32_t* cl, const float* bias,
                         int32_t window, float scale, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks, int32_t max_seq_len, int64_t num_blocks,
                         pa_dtype_t dtype) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d is not supported (0 = fp32, 1 = bf16)", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  if (block_size != pa::kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d is not supported (16)", block_size);
  if (num_heads < 1 || num_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_heads %d out of range [1, 65535]", num_heads);
  if (num_kv_heads != num_heads)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads (%d) must equal num_heads (%d)", num_kv_heads,
                num_heads);
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d out of range [0, 65535]", num_seqs);
  if (max_seq_len < 0 || max_blocks < 0 || num_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size (max_seq_len %d, max_blocks_per_seq %d, "
                "num_blocks %lld)", max_seq_len, max_blocks, (long long)num_blocks);
  if ((int64_t)max_blocks * pa::kBlockSize < max_seq_len)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * 16 (%lld) < max_seq_len (%d)",
                (long long)max_blocks * pa::kBlockSize, max_seq_len);
  if (window == 0 || window < -1)
    return fail(PA_ERR_INVALID_ARG, "sliding_window %d: use -1 (off) or >= 1", window);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k || !v || !bt || !cl)
    return fail(PA_ERR_NULL_POINTER, "a required pointer is NULL (out %p q %p k %p v %p "
                "block_tables %p context_lens %p)", out, q, k, v, (const void*)bt,
                (const void*)cl);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(PA_ERR_MISALIGNED, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(bt, 4) || !aligned(cl, 4) || (bias && !aligned(bias, 4)))
    return fail(PA_ERR_MISALIGNED, "block_tables, context_lens and attn_bias must be 4-byte "
                "aligned");
  return PA_OK;
}

// T5 bucket of a non-negative distance within one direction, in float64 (the
// precision the bucket decision is taken in): exact below max_exact, then
// max_exact + floor(log(n / max_exact) / log(max_distance / max_exact) *
// (half - max_exact)), capped at half - 1.
int32_t rel_half_bucket_f64(int64_t n, int32_t half, int32_t max_exact, int32_t max_distance) {
  if (n < max_exact) return (int32_t)n;
  const double v = (double)max_exact +
                   std::floor(std::log((double)n / (double)max_exact) /
                              std::log((double)max_distance / (double)max_exact) *
                              (double)(half - max_exact));
  return v > (double)(half - 1) ? half - 1 : (int32_t)v;
}

// Fill the kernel-side description of a T5 bias: thresholds thr[k] = the
// smallest distance whose bucket is >= max_exact + 1 + k. Memoised per
// thread on (half, max_distance): a pure function of the bucket shape.
pa_status_t make_relpos(const float* table, int32_t num_buckets, int32_t max_distance,
                        int32_t bidirectional, pa::RelPos* r) {
  if (!table) return fail(PA_ERR_NULL_POINTER, "rel_table is NULL");
  if (!aligned(table, 4)) return fail(PA_ERR_MISALIGNED, "rel_table must be 4-byte aligned");
  if (bidirectional != 0 && bidirectional != 1)
    return fail(PA_ERR_INVALID_ARG, "bidirectional must be 0 or 1");
  if (num_buckets < 2 || num_buckets > 2 * pa::kMaxRelThresholds ||
      (bidirectional && num_buckets % 2 != 0))
    return fail(PA_ERR_INVALID_ARG, "num_buckets %d: use 2..%d (even when bidirectional)",
                num_buckets, 2 * pa::kMaxRelThresholds);
  const int32_t half = bidirectional ? num_buckets / 2 : num_buckets;
  const int32_t max_exact = half / 2;
  if (max_exact < 1)
    return fail(PA_ERR_INVALID_ARG, "num_buckets %d leaves no exact bucket", num_buckets);
  if (max_distance <= max_exact || max_distance > pa::kMaxRelDistance)
    return fail(PA_ERR_INVALID_ARG, "max_distance %d: use (%d, %d]", max_distance, max_exact,
                pa::kMaxRelDistance);
  struct Memo {
    int32_t half = -1, max_distance = -1, nthr = 0;
    int32_t thr[pa::kMaxRelThresholds];
  };
  static thread_local Memo memo;
  if (memo.half != half || memo.max_distance != max_distance) {
    int32_t nthr = 0, cur = max_exact;
    for (int64_t n = max_exact; n <= max_distance && cur < half - 1; ++n) {
      const int32_t bk = rel_half_bucket_f64(n, half, max_exact, max_distance);
      while (cur < bk && cur < half - 1) {   // buckets cur+1 .. bk start at n
        memo.thr[nthr++] = (int32_t)n;
        ++cur;
      }
    }
    memo.half = half;
    memo.max_distance = max_distance;
    memo.nthr = nthr;
  }
  r->table = table;
  r->num_buckets = num_buckets;
  r->half = half;
  r->max_exact = max_exact;
  r->max_distance = max_distance;
  r->bidirectional = bidirectional;
  r->nthr = memo.nthr;
  for (int32_t k = 0; k < memo.nthr; ++k) r->thr[k] = memo.thr[k];
  return PA_OK;
}

// Host check of the metadata a call would read (pa_check_metadata, and the
// PA_VALIDATE path with chunked local attention as well): lengths, query
// offsets, and the block-table entries of every block a query can see.
pa_status_t check_metadata_impl(const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc, int32_t sliding_window,
                                int32_t chunk, int32_t causal, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int32_t max_seq_len,
                                int64_t num_blocks, int64_t total_q) {
  (void)causal;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
  // the table rows must cover max_seq_len: every entry read below then lies
  // inside the num_seqs x max_blocks_per_seq array
  if (max_seq_len < 0 || max_blocks_per_seq < 0 ||
      (int64_t)max_blocks_per_seq * pa::kBlockSize < max_seq_len)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d does not cover max_seq_len %d",
                max_blocks_per_seq, max_seq_len);
  if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables)))
    return fail(PA_ERR_NULL_POINTER, "metadata pointer is NULL");
  if (query_start_loc) {
    if (query_start_loc[0] != 0)
      return fail(PA_ERR_INVALID_ARG, "query_start_loc[0] = %d, expected 0", query_start_loc[0]);
    if (query_start_loc[num_seqs] != total_q)
      return fail(PA_ERR_INVALID_ARG, "query_start_loc[%d] = %d, expected total_q = %lld",
                  num_seqs, query_start_loc[num_seqs], (long long)total_q);
  }
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t L = context_lens[b];
    if (L < 0 || L > max_seq_len)
      return fail(PA_ERR_INVALID_ARG, "context_lens[%d] = %d outside [0, %d]", b, L, max_seq_len);
    int32_t first_pos = L - 1;   // decode: the one query
    if (query_start_loc) {
      const int32_t nq = query_start_loc[b + 1] - query_start_loc[b];
      if (nq < 0 || nq > L)
        return fail(PA_ERR_INVALID_ARG, "sequence %d has %d queries for %d keys", b, nq, L);
      if (nq == 0) continue;
      first_pos = L - nq;
    }
    if (L == 0) continue;
    int32_t lo = 0;
    if (sliding_window > 0 && first_pos - sliding_window + 1 > 0)
      lo = first_pos - sliding_window + 1;
    if (chunk > 0) lo = first_pos / chunk * chunk;   // the first query's chunk
    for (int32_t n = lo / pa::kBlockSize; n < (L + pa::kBlockSize - 1) / pa::kBlockSize; ++n) {
      const int32_t id = block_tables[(int64_t)b * max_blocks_per_seq + n];
      if (id < 0 || id >= num_blocks)
        return fail(PA_ERR_INVALID_ARG, "block_tables[%d][%d] = %d outside [0, %lld)", b, n, id,
                    (long long)num_blocks);
    }
  }
  return ok();
}


bool validate_env() {
  const char* e = std::getenv("PA_VALIDATE");
  return e && e[0] && std::strcmp(e, "0") != 0;
}

pa_status_t validate_device(const int32_t* bt, const int32_t* cl, const int32_t* qsl,
                            int32_t window, int32_t chunk, int32_t causal, int32_t num_seqs,
                            int32_t max_blocks, int32_t max_seq_len, int64_t num_blocks,
                            int64_t total_q, hipStream_t stream) {
  std::vector<int32_t> hbt((size_t)num_seqs * max_blocks), hcl(num_seqs), hqsl;
  hipError_t e = hipMemcpyAsync(hcl.data(), cl, sizeof(int32_t) * num_seqs,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && !hbt.empty())
    e = hipMemcpyAsync(hbt.data(), bt, sizeof(int32_t) * hbt.size(), hipMemcpyDeviceToHost,
                       stream);
  if (e == hipSuccess && qsl) {
    hqsl.resize(num_seqs + 1);
    e = hipMemcpyAsync(hqsl.data(), qsl, sizeof(int32_t) * hqsl.size(), hipMemcpyDeviceToHost,
                       stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "PA_VALIDATE copy failed: %s", hipGetErrorString(e));
  return check_metadata_impl(hbt.data(), hcl.data(), qsl ? hqsl.data() : nullptr, window, chunk,
                             causal, num_seqs, max_blocks, max_seq_len, num_blocks, total_q);
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_last_error(void) { return g_err; }

int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                    int32_t max_seq_len, int32_t sliding_window,
                                    pa_dtype_t dtype) {
  (void)head_dim;
  (void)dtype;
  if (num_seqs < 0 || num_heads < 1 || max_seq_len < 0) return 0;
  return default_partition(num_seqs, num_heads, max_seq_len, sliding_window);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t sliding_window,
                                 int32_t partition_tokens, pa_dtype_t dtype) {
  (void)dtype;
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || max_seq_len < 0) return 0;
  if (partition_tokens < 0 || partition_tokens % pa::kBlockSize != 0 ||
      partition_tokens > pa::kMaxPartition)
    return 0;
  return plan_decode(num_seqs, num_heads, head_dim, max_seq_len, sliding_window,
                     partition_tokens).ws_bytes;
}

pa_status_t pa_check_metadata(const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t sliding_window,
                              int32_t causal, int32_t num_seqs, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int64_t num_blocks, int64_t total_q) {
  return check_metadata_impl(block_tables, context_lens, query_start_loc, sliding_window, 0,
                             causal, num_seqs, max_blocks_per_seq, max_seq_len, num_blocks,
                             total_q);
}

}  // extern "C"

namespace {

// Split-K scratch of paged_attn_decode_noalloc: the partition partials of one
// call, in the layout of the decode workspace. Each GPU holds its own copy for
// the life of the process; every call on a GPU reuses it (so calls that
// overlap on one GPU race). Host code never uses the array's name as an
// address: noalloc_scratch looks up each device's copy once.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of `scratch` on the device `stream` runs on (the current
// device for the null stream), looked up with that device current on its
// first use and kept.
pa_status_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "cannot find the stream's device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices "
                "0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    const bool other = e == hipSuccess && cur != dev;
    if (other) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = other ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || back != hipSuccess || !p)
      return fail(PA_ERR_HIP, "no-allocation scratch lookup on device %d failed: %s", dev,
                  hipGetErrorString(e != hipSuccess ? e : back));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

pa_status_t decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const float* attn_bias, const int64_t* bias_start,
                        const pa::RelPos* rel, int32_t sliding_window, float scale,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                        int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                        void* stream, int32_t chunk = 0, bool noalloc = false) {
  pa_status_t st = check_common(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias,
                                sliding_window, scale, num_seqs, num_heads, num_kv_heads,
                                head_dim, block_size, max_blocks_per_seq, max_seq_len,
                                num_blocks, dtype);
  if (st != PA_OK) return st;
#ifdef PA_NO_BIAS
  if (attn_bias)
    return fail(PA_ERR_UNSUPPORTED, "this comparison build has no materialised-bias decode");
#endif
  if (partition_tokens < 0 || partition_tokens % pa::kBlockSize != 0 ||
      partition_tokens > pa::kMaxPartition)
    return fail(PA_ERR_INVALID_ARG, "partition_tokens %d: use 0 or a multiple of 16 in "
                "[16, %d]", partition_tokens, pa::kMaxPartition);
  if (num_seqs == 0) return ok();
  // a chunk bounds the visible span like a window of the chunk's size
  const DecodePlan plan = plan_decode(num_seqs, num_heads, head_dim, max_seq_len,
                                      chunk > 0 ? chunk : sliding_window, partition_tokens);
  if (plan.num_partitions > 65535)
    return fail(PA_ERR_INVALID_ARG, "too many partitions (%d)", plan.num_partitions);
  if (noalloc && plan.ws_bytes > 0) {
    if (plan.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
      return fail(PA_ERR_WORKSPACE, "this shape needs %zu bytes of split-K scratch; the "
                  "no-allocation entry point holds %zu (use paged_attn_decode with a "
                  "workspace, or longer partitions)", plan.ws_bytes,
                  (size_t)PA_NOALLOC_SCRATCH_BYTES);
    st = noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (st != PA_OK) return st;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "decode workspace of %zu bytes needed, %zu given (%p)",
                  plan.ws_bytes, workspace_bytes, workspace);
    if (!aligned(workspace, 256))
      return fail(PA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_env()) {
    st = validate_device(block_tables, context_lens, nullptr, sliding_window, chunk, 0, num_seqs,
                         max_blocks_per_seq, max_seq_len, num_blocks, 0, s);
    if (st != PA_OK) return st;
  }
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.attn_bias = attn_bias;
  a.bias_start = bias_start;
  a.window = sliding_window;
  a.chunk = chunk;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.dtype = (int32_t)dtype;
  a.partition = plan.partition;
  a.num_partitions = plan.num_partitions;
  if (rel) a.rel = *rel;
  if (plan.ws_bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_m = reinterpret_cast<float*>(ws + plan.off_m);
    a.ws_l = reinterpret_cast<float*>(ws + plan.off_l);
  }
  hipError_t e = pa::launch_decode(a, s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

pa_status_t prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, const float* attn_bias,
                         const int64_t* bias_start, const pa::RelPos* rel,
                         int32_t sliding_window, int32_t causal,
                         float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t max_seq_len, int64_t num_blocks, int64_t total_q,
                         pa_dtype_t dtype, void* stream, int32_t chunk = 0) {
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d out of range [0, 65535]", num_seqs);
  if (total_q < 0 || total_q > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "total_q %lld out of range", (long long)total_q);
  // no queries: scalars are still checked, but no pointer is needed (an empty
  // tensor's data pointer may be NULL)
  pa_status_t st = check_common(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias,
                                sliding_window, scale, total_q == 0 ? 0 : num_seqs, num_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                max_seq_len, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (num_seqs == 0 || total_q == 0) return ok();
  if (!query_start_loc) return fail(PA_ERR_NULL_POINTER, "query_start_loc is NULL");
  if (!aligned(query_start_loc, 4))
    return fail(PA_ERR_MISALIGNED, "query_start_loc must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_env()) {
    st = validate_device(block_tables, context_lens, query_start_loc, sliding_window, chunk,
                         causal, num_seqs, max_blocks_per_seq, max_seq_len, num_blocks, total_q,
                         s);
    if (st != PA_OK) return st;
  }
  if (total_q == 0 || max_seq_len == 0) return ok();
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.attn_bias = attn_bias;
  a.bias_start = bias_start;
  a.window = sliding_window;
  a.chunk = chunk;
  a.causal = causal;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.dtype = (int32_t)dtype;
  a.total_q = (int32_t)total_q;
  if (rel) a.rel = *rel;
  hipError_t e = dtype == PA_DTYPE_F32 ? pa::launch_prefill_f32(a, s) : pa::launch_prefill_bf16(a, s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

pa_status_t paged_attn_decode(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const float* attn_bias,
                              int32_t sliding_window, float scale, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                              int32_t partition_tokens, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias, nullptr,
                     nullptr, sliding_window, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, max_seq_len, num_blocks, dtype,
                     partition_tokens, workspace, workspace_bytes, stream);
}

pa_status_t paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const float* attn_bias,
                                      int32_t sliding_window, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                                      int32_t partition_tokens, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias, nullptr,
                     nullptr, sliding_window, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, max_seq_len, num_blocks, dtype,
                     partition_tokens, nullptr, 0, stream, 0, true);
}

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
                                     size_t workspace_bytes, void* stream) {
  pa::RelPos rel{};
  pa_status_t st = make_relpos(rel_table, num_buckets, max_distance, bidirectional, &rel);
  if (st != PA_OK) return st;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, nullptr, nullptr,
                     &rel, sliding_window, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, max_seq_len, num_blocks, dtype,
                     partition_tokens, workspace, workspace_bytes, stream);
}

pa_status_t paged_attn_prefill(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               const float* attn_bias, int32_t sliding_window, int32_t causal,
                               float scale, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t max_seq_len,
                               int64_t num_blocks, int64_t total_q, pa_dtype_t dtype,
                               void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      attn_bias, nullptr, nullptr, sliding_window, causal, scale, num_seqs,
                      num_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                      num_blocks, total_q, dtype, stream);
}

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
                                      pa_dtype_t dtype, void* stream) {
  pa::RelPos rel{};
  pa_status_t st = make_relpos(rel_table, num_buckets, max_distance, bidirectional, &rel);
  if (st != PA_OK) return st;
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      nullptr, nullptr, &rel, sliding_window, causal, scale, num_seqs,
                      num_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                      num_blocks, total_q, dtype, stream);
}

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
                                          void* stream) {
  if (num_seqs > 0 && (!attn_bias || !bias_start))
    return fail(PA_ERR_NULL_POINTER, "attn_bias and bias_start are required");
  if (bias_start && !aligned(bias_start, 8))
    return fail(PA_ERR_MISALIGNED, "bias_start must be 8-byte aligned");
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias, bias_start,
                     nullptr, sliding_window, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, max_seq_len, num_blocks, dtype,
                     partition_tokens, workspace, workspace_bytes, stream);
}

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
                                           int64_t total_q, pa_dtype_t dtype, void* stream) {
  if (num_seqs > 0 && total_q > 0 && (!attn_bias || !bias_start))
    return fail(PA_ERR_NULL_POINTER, "attn_bias and bias_start are required");
  if (bias_start && !aligned(bias_start, 8))
    return fail(PA_ERR_MISALIGNED, "bias_start must be 8-byte aligned");
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      attn_bias, bias_start, nullptr, sliding_window, causal, scale, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                      max_seq_len, num_blocks, total_q, dtype, stream);
}

pa_status_t paged_attn_decode_chunked(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const float* attn_bias,
                                      int32_t chunk_size, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len, int64_t num_blocks, pa_dtype_t dtype,
                                      int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (chunk_size < 1) return fail(PA_ERR_INVALID_ARG, "chunk_size %d: must be >= 1", chunk_size);
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, attn_bias, nullptr,
                     nullptr, -1, scale, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, max_seq_len, num_blocks, dtype, partition_tokens,
                     workspace, workspace_bytes, stream, chunk_size);
}

pa_status_t paged_attn_prefill_chunked(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens,
                                       const int32_t* query_start_loc, const float* attn_bias,
                                       int32_t chunk_size, int32_t causal, float scale,
                                       int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, int64_t num_blocks, int64_t total_q,
                                       pa_dtype_t dtype, void* stream) {
  if (chunk_size < 1) return fail(PA_ERR_INVALID_ARG, "chunk_size %d: must be >= 1", chunk_size);
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      attn_bias, nullptr, nullptr, -1, causal, scale, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_seq_len,
                      num_blocks, total_q, dtype, stream, chunk_size);
}

int32_t pa_window_first_live_block(int32_t context_len, int32_t sliding_window) {
  if (context_len <= 0 || sliding_window <= 0 || context_len <= sliding_window) return 0;
  return (context_len - sliding_window) / pa::kBlockSize;
}

pa_status_t paged_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, pa_dtype_t dtype, void* stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d is not supported (0 = fp32, 1 = bf16)", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  if (block_size != pa::kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d is not supported (16)", block_size);
  if (num_heads < 1 || num_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_heads %d out of range [1, 65535]", num_heads);
  if (num_kv_heads != num_heads)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads (%d) must equal num_heads (%d)", num_kv_heads,
                num_heads);
  if (num_tokens < 0 || num_tokens > 0x7fffffff || num_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "num_tokens %lld / num_blocks %lld out of range",
                (long long)num_tokens, (long long)num_blocks);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_MISALIGNED, "caches and new rows must be 16-byte aligned, "
                "slot_mapping 8-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_env()) {
    std::vector<int64_t> hs(num_tokens);
    hipError_t e = hipMemcpyAsync(hs.data(), slot_mapping, sizeof(int64_t) * num_tokens,
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
      return fail(PA_ERR_HIP, "PA_VALIDATE copy failed: %s", hipGetErrorString(e));
    for (int64_t t = 0; t < num_tokens; ++t)
      if (hs[t] >= num_blocks * pa::kBlockSize)
        return fail(PA_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld outside the %lld-slot pool",
                    (long long)t, (long long)hs[t], (long long)(num_blocks * pa::kBlockSize));
  }
  pa::KvWriteArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.dtype = (int32_t)dtype;
  hipError_t e = pa::launch_kv_write(a, s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv write launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
