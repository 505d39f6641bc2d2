// Split-K paged-attention decode for gfx950 (CDNA4, wave64).
//
// Computes, for one query per (sequence b, head h) at position L-1,
//   out = softmax((q K^T + A) * scale) V
// (attention with an additive bias, "[Kernel][Model] PagedAttention: Support
// custom attention bias for T5 model (1/2)", formula in the PR description),
// reading K/V through the block table and, when given, the bias row
// A[b, h, :] padded to max_seq_len. With a sliding window W only the W newest
// tokens are visible ("[V1] Add sliding window support to Flex Attention
// backend"); the blocks before the window are never touched, and neither are
// their block-table entries (the same review notes that in-window iteration
// may skip evicted blocks).
//
// Kernel 1 (pa_decode_partition): one workgroup of 4 wave64s (8 in launches
// of under 1024 workgroups) per (head, partition, sequence). A partition is
// `partition` consecutive tokens starting at the 16-aligned block that holds
// the first visible token. The workgroup
//   1. stages q and the partition's block-table entries in LDS;
//   2. K pass: each of the W waves takes every W-th 16-token block (4 or 8
//      blocks in flight per wave, non-temporal loads); a block of one head
//      is 16*D contiguous elements, read with 16-byte loads where lane l reads
//      bytes [16 l, 16 l + 16) of every 1 KiB slice, so each load instruction
//      is one fully coalesced 1 KiB segment; a token's row spans LPT lanes,
//      whose partial dot products are summed with DPP row operations;
//   3. scores s = (q.k + a) * scale * log2(e) (bias added before the scale;
//      masked tokens get -inf), workgroup max, p = 2^(s - m), workgroup sum;
//   4. V pass: same lane layout, o[d] += p_j v_j[d] in fp32;
//   5. writes (m, l, o) of the partition, or the final o / l when the whole
//      call has a single partition per sequence.
// Kernel 2 (pa_decode_merge): one workgroup per (sequence, head) merges the
// partitions in ascending order (log-sum-exp rescaling), so results are
// bit-reproducible run to run.
#include "pa_internal.h"

#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// First key the decode query (position L - 1) may see: the first of the W
// newest tokens with a window, the start of the query's chunk with chunked
// local attention, else 0.
__device__ __forceinline__ int decode_first_key(const DecodeArgs& a, int L) {
  if (a.chunk > 0) return L > 0 ? (L - 1) / a.chunk * a.chunk : 0;
  return (a.window > 0 && L > a.window) ? L - a.window : 0;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xf, 0xf, false);
}

// Sum over aligned groups of N consecutive lanes (N = 8, 16 or 32); every lane
// of a group ends with the group sum. Each step adds two equal partial sums
// (commutative), so all lanes of a group hold bit-identical results.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp<0x141>(v);   // row_half_mirror: the other quad of the 8-lane half
  if constexpr (N >= 16) v += dpp<0x140>(v);   // row_mirror: other half-row
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// per-(dtype, head_dim) lane geometry
// ---------------------------------------------------------------------------
template <int DT, int D>
struct Geo {
  static constexpr int kEsize = DT == 0 ? 4 : 2;
  static constexpr int kRowBytes = D * kEsize;         // one token of one head
  static constexpr int kLPT = kRowBytes / 16;           // lanes per token
  static constexpr int kTPL = 64 / kLPT;                // tokens per load
  static constexpr int kNLoad = kBlockSize / kTPL;      // loads per lane per block
  static constexpr int kEPL = 16 / kEsize;              // elements per lane per load
  static constexpr int kBlockBytes = kBlockSize * kRowBytes;
  static_assert(kLPT == 8 || kLPT == 16 || kLPT == 32, "unsupported row size");
};

// Partial dot product of one 16-byte slice of a key row with the matching
// slice of q (held as raw 32-bit words).
template <int DT>
__device__ __forceinline__ float slice_dot(const uint4& k, const uint4& q) {
  if constexpr (DT == 0) {
    float d = __uint_as_float(k.x) * __uint_as_float(q.x);
    d = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), d);
    d = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), d);
    d = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), d);
    return d;
  } else {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    float d = 0.0f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x),
                                        __builtin_bit_cast(bf16x2, q.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y),
                                        __builtin_bit_cast(bf16x2, q.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z),
                                        __builtin_bit_cast(bf16x2, q.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w),
                                        __builtin_bit_cast(bf16x2, q.w), d, false);
    return d;
  }
}

// acc[0..EPL) += p * v (v one 16-byte slice of a value row).
template <int DT>
__device__ __forceinline__ void slice_axpy(float* acc, float p, const uint4& v) {
  if constexpr (DT == 0) {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  } else {
    acc[0] = fmaf(p, bf16_lo(v.x), acc[0]);
    acc[1] = fmaf(p, bf16_hi(v.x), acc[1]);
    acc[2] = fmaf(p, bf16_lo(v.y), acc[2]);
    acc[3] = fmaf(p, bf16_hi(v.y), acc[3]);
    acc[4] = fmaf(p, bf16_lo(v.z), acc[4]);
    acc[5] = fmaf(p, bf16_hi(v.z), acc[5]);
    acc[6] = fmaf(p, bf16_lo(v.w), acc[6]);
    acc[7] = fmaf(p, bf16_hi(v.w), acc[7]);
  }
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16-byte load of streamed K/V data. Each K/V byte is read exactly once per
// call, so the loads are non-temporal: they do not displace the block table,
// bias and q lines from the caches (worth ~11% of HBM bandwidth on MI355X).
__device__ __forceinline__ uint4 load16(const char* p) {
#if PA_DECODE_NT
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// 16-token blocks each wave keeps in flight per loop iteration: 8 for bf16
// at head_dim 64 (2 KiB per block and head, 16 loads of 16 bytes per lane,
// within 5+ waves per SIMD), 4 otherwise
#ifndef PA_DECODE_UNROLL
#define PA_DECODE_UNROLL 4
#endif
#ifndef PA_DECODE_UNROLL_BF16_64
#define PA_DECODE_UNROLL_BF16_64 8
#endif
template <int DT, int D>
constexpr int unroll_of() { return DT == 1 && D == 64 ? PA_DECODE_UNROLL_BF16_64 : PA_DECODE_UNROLL; }
// bias entries per thread fetched before the key pass
constexpr int kBiasPre = 4;

template <int DT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (DT == 0)
    static_cast<float*>(out)[idx] = v;
  else
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// kernel 1: one partition of one (sequence, head)
// ---------------------------------------------------------------------------
// BIAS: 0 none, 1 materialised row attn_bias[b, h, :], 2 T5 relative-position
// bias from a bucket table (a.rel).
// W: waves per workgroup (4, or 8 for launches too small to fill the chip)
template <int DT, int D, int BIAS, bool SINGLE, int W>
__global__ void __launch_bounds__(64 * W)
pa_decode_partition(DecodeArgs a) {
  using G = Geo<DT, D>;
  constexpr int kUnroll = unroll_of<DT, D>();
  constexpr int kDecodeThreads = 64 * W;   // shadows the 4-wave default
  constexpr int kDecodeWaves = W;
  const int h = blockIdx.x;
  const int part = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = a.num_heads;
  const int P = a.partition;

  // a length outside [0, max_seq_len] (unchecked unless PA_VALIDATE is set)
  // is treated as an empty sequence rather than read past the table row
  const int L = a.context_lens[b];
  const int lo = decode_first_key(a, L);
  const int start = lo & ~(kBlockSize - 1);
  const int t0 = start + part * P;                     // first token of partition
  if (L <= 0 || L > a.max_seq_len || t0 >= L) {
    if (SINGLE && part == 0 && tid < D)                 // empty sequence: zeros
      store_out<DT>(a.out, ((int64_t)b * H + h) * D + tid, 0.0f);
    return;
  }
  const int t1 = min(t0 + P, L);                       // one past the last token
  const int nblk = (t1 - t0 + kBlockSize - 1) / kBlockSize;
  const int nb0 = t0 / kBlockSize;                     // first logical block

  // LDS: q slices | reductions | per-wave outputs | scores | block ids |
  //      relative-position bias by distance (BIAS == 2)
  extern __shared__ uint4 smem_u4[];
  uint4* q_lds = smem_u4;                              // [LPT] 16-byte slices
  float* red_lds = reinterpret_cast<float*>(q_lds + G::kLPT);   // [2 W]
  float* o_lds = red_lds + 2 * W;                      // [W][D]
  float* s_lds = o_lds + kDecodeWaves * D;             // [P] scores, then weights
  int* tbl_lds = reinterpret_cast<int*>(s_lds + P);    // [P/16] physical ids
  float* rel_lds = reinterpret_cast<float*>(tbl_lds + P / kBlockSize);  // [max_distance + 1]

  // stage q and the block-table slice
  const int64_t row = (int64_t)b * H + h;
  if (tid < G::kLPT)
    q_lds[tid] = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + row * G::kRowBytes)[tid];
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks + nb0;
  for (int i = tid; i < nblk; i += kDecodeThreads) tbl_lds[i] = table[i];
  if constexpr (BIAS == 2) {
    // bias of a key at distance d = (L-1) - j before the query, d <= max_distance
    // (every longer distance shares the last bucket)
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int d = tid; d <= a.rel.max_distance; d += kDecodeThreads)
      rel_lds[d] = rel_bias(-d, a.rel, head_row);
  }
  __syncthreads();

  const int seg = lane % G::kLPT;
  const uint4 qv = q_lds[seg];
  const int64_t head_off = (int64_t)h * G::kBlockBytes + lane * 16;
  const int64_t blk_stride = (int64_t)H * G::kBlockBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + head_off;
  const char* vbase = static_cast<const char*>(a.v_cache) + head_off;

  // ---- K pass: raw dot products into s_lds ----
  // (bias entries of this thread's first tokens are requested first, so they
  // arrive while the keys stream in)
  const float* bias_row =
      BIAS != 1 ? nullptr
                : (a.bias_start ? a.attn_bias + a.bias_start[b] + (int64_t)h * L   // ragged
                                : a.attn_bias + row * a.max_seq_len);               // padded
  const int ntok = nblk * kBlockSize;
  float bpre[kBiasPre];
#pragma unroll
  for (int k = 0; k < kBiasPre; ++k) {
    const int j = t0 + tid + k * kDecodeThreads;
    bpre[k] = 0.0f;
    if (BIAS == 1 && tid + k * kDecodeThreads < ntok && j >= lo && j < L) bpre[k] = bias_row[j];
  }
  for (int n0 = wave; n0 < nblk; n0 += kUnroll * kDecodeWaves) {
    int64_t ph[kUnroll];
    uint4 kx[kUnroll][G::kNLoad];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * kDecodeWaves;
      ph[u] = __builtin_amdgcn_readfirstlane(tbl_lds[n < nblk ? n : n0]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (n0 + u * kDecodeWaves < nblk) {
#pragma unroll
        for (int i = 0; i < G::kNLoad; ++i)
          kx[u][i] = load16(kbase + ph[u] * blk_stride + i * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * kDecodeWaves;
      if (n < nblk) {
#pragma unroll
        for (int i = 0; i < G::kNLoad; ++i) {
          float d = group_sum<G::kLPT>(slice_dot<DT>(kx[u][i], qv));
          if (seg == 0) s_lds[n * kBlockSize + i * G::kTPL + lane / G::kLPT] = d;
        }
      }
    }
  }
  __syncthreads();

  // ---- scores, max, weights, sum ----
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kBiasPre; ++k) {
    const int i = tid + k * kDecodeThreads;
    const int j = t0 + i;
    if (i < ntok) {
      float s = -INFINITY;
      if (j >= lo && j < L) {
        float t = s_lds[i];
        if constexpr (BIAS == 1) t = t + bpre[k];
        if constexpr (BIAS == 2) t = t + rel_lds[min(L - 1 - j, a.rel.max_distance)];
        s = t * a.scale_log2;
      }
      s_lds[i] = s;
      mx = fmaxf(mx, s);
    }
  }
  for (int i = tid + kBiasPre * kDecodeThreads; i < ntok; i += kDecodeThreads) {
    const int j = t0 + i;
    float s = -INFINITY;
    if (j >= lo && j < L) {
      float t = s_lds[i];
      if constexpr (BIAS == 1) t = t + bias_row[j];
      if constexpr (BIAS == 2) t = t + rel_lds[min(L - 1 - j, a.rel.max_distance)];
      s = t * a.scale_log2;
    }
    s_lds[i] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red_lds[wave] = mx;
  __syncthreads();
  float m = red_lds[0];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) m = fmaxf(m, red_lds[w]);
  const float m_use = (m == -INFINITY) ? 0.0f : m;     // fully masked: all p = 0
  float sum = 0.0f;
  for (int i = tid; i < ntok; i += kDecodeThreads) {
    const float p = __builtin_amdgcn_exp2f(s_lds[i] - m_use);
    s_lds[i] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __syncthreads();                                      // red_lds reuse + s_lds
  if (lane == 0) red_lds[W + wave] = sum;
  __syncthreads();
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) l += red_lds[W + w];

  // ---- V pass ----
  float acc[G::kEPL];
#pragma unroll
  for (int e = 0; e < G::kEPL; ++e) acc[e] = 0.0f;
  const int tl = lane / G::kLPT;                        // token within a load
  for (int n0 = wave; n0 < nblk; n0 += kUnroll * kDecodeWaves) {
    int64_t ph[kUnroll];
    uint4 vx[kUnroll][G::kNLoad];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * kDecodeWaves;
      ph[u] = __builtin_amdgcn_readfirstlane(tbl_lds[n < nblk ? n : n0]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (n0 + u * kDecodeWaves < nblk) {
#pragma unroll
        for (int i = 0; i < G::kNLoad; ++i)
          vx[u][i] = load16(vbase + ph[u] * blk_stride + i * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * kDecodeWaves;
      if (n < nblk) {
        // tokens outside [lo, L) may hold anything (even NaN): zero their slices
        const int j1 = t0 + n * kBlockSize;
        if (j1 < lo || j1 + kBlockSize > L) {
#pragma unroll
          for (int i = 0; i < G::kNLoad; ++i) {
            const int j = j1 + i * G::kTPL + tl;
            if (j < lo || j >= L) vx[u][i] = zero_u4();
          }
        }
#pragma unroll
        for (int i = 0; i < G::kNLoad; ++i)
          slice_axpy<DT>(acc, s_lds[n * kBlockSize + i * G::kTPL + tl], vx[u][i]);
      }
    }
  }
  // sum the token groups of the wave (lanes with equal seg), then the waves
#pragma unroll
  for (int o = G::kLPT; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < G::kEPL; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  if (lane < G::kLPT) {
#pragma unroll
    for (int e = 0; e < G::kEPL; ++e) o_lds[wave * D + seg * G::kEPL + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float o = o_lds[tid];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) o += o_lds[w * D + tid];
    if constexpr (SINGLE) {
      store_out<DT>(a.out, row * D + tid, l > 0.0f ? o / l : 0.0f);
    } else {
      const int64_t pi = row * a.num_partitions + part;
      a.ws_o[pi * D + tid] = o;
      if (tid == 0) {
        a.ws_m[pi] = m;
        a.ws_l[pi] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// kernel 2: merge the partitions of one (sequence, head), in fixed order
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ void __launch_bounds__(D) pa_decode_merge(DecodeArgs a) {
  const int64_t row = blockIdx.x;                     // b * H + h
  const int b = (int)(row / a.num_heads);
  const int tid = threadIdx.x;
  const int L = a.context_lens[b];
  const int lo = decode_first_key(a, L);
  const int start = lo & ~(kBlockSize - 1);
  const int np = L > 0 && L <= a.max_seq_len ? (L - start + a.partition - 1) / a.partition : 0;
  const int64_t base = row * a.num_partitions;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_m[base + p]);
  float den = 0.0f, num = 0.0f;
  if (M != -INFINITY) {
    for (int p = 0; p < np; ++p) {
      const float w = __builtin_amdgcn_exp2f(a.ws_m[base + p] - M);
      den = fmaf(w, a.ws_l[base + p], den);
      num = fmaf(w, a.ws_o[(base + p) * D + tid], num);
    }
  }
  store_out<DT>(a.out, row * D + tid, den > 0.0f ? num / den : 0.0f);
}

// Launches of fewer workgroups than this (4 per CU) take 8 waves per
// workgroup: each (sequence, head) then has twice the blocks in flight, which
// launches too small to fill the chip need more than occupancy. Measured on
// T5-small-shaped self-attention (512 workgroups): 10.7 against 11.45 us;
// at 4096 workgroups (T5-large-shaped) 8 waves lose (62 against 55.5 us).
// 0 keeps every launch at 4 waves.
#ifndef PA_DECODE_WIDE_BELOW
#define PA_DECODE_WIDE_BELOW 1024
#endif

template <int DT, int D, int BIAS, int W>
hipError_t launch_waves(const DecodeArgs& a, hipStream_t stream) {
  using G = Geo<DT, D>;
  size_t lds = sizeof(float) * a.partition + sizeof(int) * (a.partition / kBlockSize) +
               sizeof(float) * (W * D + 2 * W) + 16 * G::kLPT;
  if (BIAS == 2) lds += sizeof(float) * (a.rel.max_distance + 1);
  dim3 grid(a.num_heads, a.num_partitions, a.num_seqs);
  if (a.num_partitions == 1) {
    hipLaunchKernelGGL((pa_decode_partition<DT, D, BIAS, true, W>), grid, dim3(64 * W), lds,
                       stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((pa_decode_partition<DT, D, BIAS, false, W>), grid, dim3(64 * W), lds,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pa_decode_merge<DT, D>), dim3((unsigned)a.num_seqs * a.num_heads),
                     dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D, int BIAS>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (PA_DECODE_WIDE_BELOW > 0) {
    const int64_t wgs = (int64_t)a.num_heads * a.num_partitions * a.num_seqs;
    if (wgs < PA_DECODE_WIDE_BELOW) return launch_waves<DT, D, BIAS, 8>(a, stream);
  }
  return launch_waves<DT, D, BIAS, kDecodeWaves>(a, stream);
}

template <int DT, int D>
hipError_t launch_bias(const DecodeArgs& a, hipStream_t stream) {
  if (a.rel.table) return launch_typed<DT, D, 2>(a, stream);
#ifdef PA_NO_BIAS
  return launch_typed<DT, D, 0>(a, stream);
#else
  return a.attn_bias ? launch_typed<DT, D, 1>(a, stream) : launch_typed<DT, D, 0>(a, stream);
#endif
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == 0)
    return a.head_dim == 64 ? launch_bias<0, 64>(a, stream) : launch_bias<0, 128>(a, stream);
  return a.head_dim == 64 ? launch_bias<1, 64>(a, stream) : launch_bias<1, 128>(a, stream);
}

}  // namespace pa
