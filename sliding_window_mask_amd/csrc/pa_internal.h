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

// Arguments of one decode call, as validated by the host API.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* attn_bias;     // may be null
  int32_t window;             // -1 or >= 1
  float scale_log2;           // scale * log2(e): scores are kept in base 2
  int32_t num_seqs, num_heads, head_dim, max_blocks, max_seq_len;
  int32_t dtype;              // 0 fp32, 1 bf16
  int32_t partition;          // tokens per partition (multiple of 16)
  int32_t num_partitions;     // partitions per (seq, head) in the grid
  float* ws_m;                // [B*H*NP] running max (base 2), or null
  float* ws_l;                // [B*H*NP] running sum
  float* ws_o;                // [B*H*NP*D] unnormalised outputs
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
  int32_t window;             // -1 or >= 1
  int32_t causal;             // 0 or 1
  float scale_log2;
  int32_t num_seqs, num_heads, head_dim, max_blocks, max_seq_len;
  int32_t dtype;
  int32_t num_qtiles;         // query tiles per sequence in the grid (set by the launcher)
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
