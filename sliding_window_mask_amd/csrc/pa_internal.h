// Internal declarations shared by the host API (pa_api.cpp) and the gfx950
// kernels (pa_decode.hip, pa_prefill.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;        // tokens per KV-cache block
constexpr int kDecodeThreads = 256;   // 4 wave64s per decode workgroup
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kMaxPartition = 4096;   // tokens per split-K partition, upper bound

constexpr int kMaxRelThresholds = 32; // relative-position bucket thresholds
constexpr int kMaxRelDistance = 1024;  // largest supported max_distance

// T5 relative-position bias, in the form the kernels use: the bias of key j
// for a query at position p is table[h * num_buckets + bucket(j - p)], where
// for r = j - p <= 0 the bucket is half_bucket(-r), and for r > 0 it is
// half + half_bucket(r) (bidirectional) or 0 (unidirectional).
// half_bucket(n) = n for n < max_exact, else max_exact + #{k : n >= thr[k]}.
// The host derives thr from the float64 bucket formula.
struct RelPos {
  const float* table;          // [num_heads, num_buckets] fp32, or null
  int32_t num_buckets;         // buckets per head (both directions)
  int32_t half;                // buckets per direction
  int32_t max_exact;           // distances with a bucket of their own
  int32_t max_distance;        // every distance >= this shares the last bucket
  int32_t bidirectional;
  int32_t nthr;
  int32_t thr[kMaxRelThresholds];
};

// Arguments of one decode call, as validated by the host API.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* attn_bias;     // may be null
  const int64_t* bias_start;  // null: bias padded [B,H,max_seq_len]; else sequence b's
                              // rows [H][L_b] start at attn_bias + bias_start[b]
  int32_t window;             // -1 or >= 1
  int32_t chunk;              // chunked local attention: chunk size >= 1, or 0 (window is -1)
  float scale_log2;           // scale * log2(e): scores are kept in base 2
  int32_t num_seqs, num_heads, head_dim, max_blocks, max_seq_len;
  int32_t dtype;              // 0 fp32, 1 bf16
  int32_t partition;          // tokens per partition (multiple of 16)
  int32_t num_partitions;     // partitions per (seq, head) in the grid
  float* ws_m;                // [B*H*NP] running max (base 2), or null
  float* ws_l;                // [B*H*NP] running sum
  float* ws_o;                // [B*H*NP*D] unnormalised outputs
  RelPos rel;                 // used when rel.table is set (attn_bias is then null)
};

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  const float* attn_bias;     // may be null
  const int64_t* bias_start;  // null: bias padded [B,H,MS,MS]; else sequence b's rows
                              // [H][n_q][L_b] start at attn_bias + bias_start[b]
  int32_t window;             // -1 or >= 1
  int32_t chunk;              // chunked local attention: chunk size >= 1, or 0 (window is -1)
  int32_t causal;             // 0 or 1
  float scale_log2;
  int32_t num_seqs, num_heads, head_dim, max_blocks, max_seq_len;
  int32_t dtype;
  int32_t total_q;            // rows of q and out
  int32_t num_qtiles;         // query tiles per sequence in the grid (set by the launcher)
  RelPos rel;                 // used when rel.table is set (attn_bias is then null)
};

// Visible key interval [lo, hi) for query positions [p0, p1] of a sequence
// of length L (caller guarantees p0 <= p1 < L): all keys, keys up to the
// last query for a causal prompt, with a window W only |p - j| < W, and with
// chunked local attention of chunk size C only the keys of each query's
// chunk, floor(j / C) = floor(p / C).
__device__ __forceinline__ void prefill_key_range(int p0, int p1, int L, int window, int chunk,
                                                  int causal, int& lo, int& hi) {
  lo = 0;
  hi = causal ? p1 + 1 : L;
  if (window > 0) {
    lo = max(0, p0 - window + 1);
    if (!causal) hi = min(L, p1 + window);
  } else if (chunk > 0) {
    lo = p0 / chunk * chunk;
    if (!causal) hi = min(L, p1 / chunk * chunk + chunk);
  }
}

// Masks of the windowed prefill path, for a query at position p of a
// sequence of length L (key j, d = p - j): key j is visible iff
// dlo < d < dhi. Window W: dhi = W and d > -W; chunk C: the key lies in p's
// chunk [p - p % C, p - p % C + C), i.e. p % C - C < d < p % C + 1. Both
// also need j < L (d > p - L), and causal queries j <= p (d > -1).
// Banded launches only: window >= 1, or window <= 0 and chunk >= 1; p >= 0.
__device__ __forceinline__ void prefill_row_bounds(int p, int L, int window, int chunk,
                                                   bool causal, int& dlo, int& dhi) {
  int lo = p - L;
  if (causal) lo = max(lo, -1);
  if (window > 0) {
    lo = max(lo, -window);
    dhi = window;
  } else {
    const int r = p % chunk;
    lo = max(lo, r - chunk);
    dhi = r + 1;
  }
  dlo = lo;
}

// Keys [wlo, whi) that every position in [p0, p1] may see under its window or
// chunk (the sequence end and a causal limit are checked separately).
// Banded launches only, as prefill_row_bounds.
__device__ __forceinline__ void prefill_common_keys(int p0, int p1, int window, int chunk,
                                                    int& wlo, int& whi) {
  if (window > 0) {
    wlo = p1 - window + 1;
    whi = p0 + window;
  } else {
    wlo = p1 / chunk * chunk;
    whi = p0 / chunk * chunk + chunk;
  }
}

constexpr int kXcds = 8;   // XCDs of an MI355X

constexpr int kRankMaxSeqs = 63;   // batches ranked by length inside the kernel

// Workgroup id -> (sequence b, head h, query tile), the sequence's length L
// and its packed query rows q0 .. q0 + nq - 1; false for ids past the last
// (sequence, head) pair (uniform over the workgroup). The grid has
// ceil(pairs / 8) * 8 * num_qtiles workgroups. Every query tile of one
// (sequence, head) runs on the same XCD: the dispatcher deals consecutive
// workgroup ids round-robin over the XCDs, so ids n with the same n % 8 share
// an XCD and its L2.
// Without a window, a workgroup's work grows with its sequence's length, so
// for batches of at most 63 sequences the pairs are dealt longest sequence
// first (ties by index): the longest workgroups start first and the launch
// does not end on a few long ones still running. Wave 0 reads every length
// and query offset in one coalesced load (lane j: sequence j), ranks the
// sequences by the distinct keys (L << 6) | (63 - j) (vector compares
// against keys broadcast from LDS, four per read; needs max_seq_len < 2^25)
// and hands its sequence's values to the other waves through LDS (one
// barrier). Windowed and chunked launches (bounded work per workgroup) and larger
// batches keep index order.
// Metadata outside the documented ranges (0 <= n_q <= L <= max_seq_len, the
// sequence's query rows inside [0, total_q)) also returns false: such a
// workgroup writes nothing rather than read or write out of bounds (the
// host checks these ranges only under PA_VALIDATE).
__device__ __forceinline__ bool prefill_work_of(int n, const PrefillArgs& a, int& b, int& h,
                                                int& tile, int& L, int& q0, int& nq) {
  const int H = a.num_heads;
  const int B = a.num_seqs;
  const int slot = n / kXcds;
  const int pr = (slot / a.num_qtiles) * kXcds + n % kXcds;   // pair in dispatch order
  tile = slot % a.num_qtiles;
  if (pr >= B * H) return false;
  const int r = pr / H;   // rank of the sequence in dispatch order
  h = pr % H;
  if (B <= kRankMaxSeqs && a.window <= 0 && a.chunk <= 0 && a.max_seq_len < (1 << 25)) {
    __shared__ int picked[4];
    __shared__ __attribute__((aligned(16))) unsigned keys[64];
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int Lj = lane < B ? a.context_lens[lane] : 0;
      const int Qj = lane <= B ? a.query_start_loc[lane] : 0;
      // distinct for lanes < B (lengths are validated to [0, max_seq_len]);
      // the zero keys of lanes >= B are below all of them
      const unsigned kj = lane < B ? ((unsigned)Lj << 6) | (63u - (unsigned)lane) : 0u;
      keys[lane] = kj;   // read back by this wave only: LDS order within a wave
      int rank = 0;      // keys above lane's
      for (int i = 0; i < B; i += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(&keys[i]);
        rank += (k4.x > kj ? 1 : 0) + (k4.y > kj ? 1 : 0) + (k4.z > kj ? 1 : 0) +
                (k4.w > kj ? 1 : 0);
      }
      // ranks are a permutation of 0 .. B-1: exactly one lane holds r
      const int sb = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < B && rank == r));
      if (lane == 0) {
        const int qb = __builtin_amdgcn_readlane(Qj, sb);
        picked[0] = sb;
        picked[1] = __builtin_amdgcn_readlane(Lj, sb);
        picked[2] = qb;
        picked[3] = __builtin_amdgcn_readlane(Qj, sb + 1) - qb;
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(picked[0]);
    L = __builtin_amdgcn_readfirstlane(picked[1]);
    q0 = __builtin_amdgcn_readfirstlane(picked[2]);
    nq = __builtin_amdgcn_readfirstlane(picked[3]);
  } else {
    b = r;
    L = a.context_lens[b];
    q0 = a.query_start_loc[b];
    nq = a.query_start_loc[b + 1] - q0;
  }
  return b >= 0 && b < B && L <= a.max_seq_len && nq >= 0 && nq <= L && q0 >= 0 &&
         q0 <= a.total_q - nq;
}

// Bucket of a non-negative distance within one direction (see RelPos).
__device__ __forceinline__ int rel_half_bucket(int n, const RelPos& r) {
  if (n < r.max_exact) return n;
  int b = r.max_exact;
  for (int k = 0; k < r.nthr; ++k) b += n >= r.thr[k] ? 1 : 0;
  return b;
}

// Bias value of relative position rel = key - query position for one head.
__device__ __forceinline__ float rel_bias(int rel, const RelPos& r, const float* head_row) {
  int bucket;
  if (rel > 0)
    bucket = r.bidirectional ? r.half + rel_half_bucket(rel, r) : 0;
  else
    bucket = rel_half_bucket(-rel, r);
  return head_row[bucket];
}

struct KvWriteArgs {
  void* k_cache;
  void* v_cache;
  const void* k_new;            // [num_tokens, H, D]
  const void* v_new;
  const int64_t* slot_mapping;  // [num_tokens], block * 16 + offset, < 0 = skip
  int64_t num_tokens;
  int32_t num_heads, head_dim, dtype;
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32x3(PrefillArgs a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
