// Measurement probes for bench.py (gfx950): hardware rates that the design
// notes compare the kernels against. Not part of the attention library.
//
//   pb_mfma        independent accumulator chains of one matrix instruction
//                  per wave, registers only (optionally with v_exp_f32 work
//                  interleaved): the rate that instruction sustains
//   pb_lds         conflict-free LDS reads (ds_read_b128 or the transposing
//                  ds_read_b64_tr_b16): the LDS read rate per CU
//   pb_stream      a streaming read of a large buffer with non-temporal
//                  16-byte loads: the HBM read rate without any gather
//   pb_gather      the decode kernel's K/V access pattern (one workgroup of 4
//                  waves per (head, sequence), 16-token blocks through the
//                  block table, 4 blocks in flight per wave, lane l reading
//                  bytes [16 l, 16 l + 16) of every 1 KiB slice, K pass then V
//                  pass, non-temporal loads) with no arithmetic, and two
//                  variants of it (ordinary loads; K and V read together)
//   pb_bias        a materialised prefill bias read in the order the prefill
//                  kernels walk it, with no arithmetic
//   pb_mix         waves running only matrix instructions beside waves
//                  running only vector instructions on the same SIMDs
//   pb_valu        independent chains of one vector instruction
//   pb_clock       the shader clock under matrix or vector load (s_memtime
//                  against the constant s_memrealtime counter)
//
// Every probe writes one 32-bit value per thread of its grid to `out`
// (vector stores), so the caller sizes `out` as grid * block values; all
// other accesses stay inside the buffers the caller passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;   // 4 waves per workgroup

// KIND 0: v_mfma_f32_16x16x32_bf16, 1: v_mfma_f32_32x32x16_bf16,
//      2: v_mfma_f32_16x16x4_f32,   3: v_mfma_f32_32x32x2_f32
template <int KIND, int CH, int NEXP>
__global__ void __launch_bounds__(kProbeThreads) pb_mfma_kernel(float* out, int iters, float seed) {
  const int tid = threadIdx.x;
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = seed * (float)(tid + i) * 1e-3f;
  float r = 0.0f;
  if constexpr (KIND == 0 || KIND == 1) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (float)(tid + i));
      b[i] = (__bf16)(seed * (float)(i - tid));
    }
    typedef typename std::conditional<KIND == 0, f4_t, f16_t>::type acc_t;
    constexpr int kN = KIND == 0 ? 4 : 16;
    acc_t acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < kN; ++i) acc[c][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (KIND == 0)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int x = 0; x < NEXP; ++x) e[x & 7] = __builtin_amdgcn_exp2f(e[x & 7]) * -0.5f;
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) r += acc[c][0] + acc[c][kN - 1];
  } else {
    const float a = seed * (float)tid, b = seed * (float)(tid ^ 5);
    typedef typename std::conditional<KIND == 2, f4_t, f16_t>::type acc_t;
    constexpr int kN = KIND == 2 ? 4 : 16;
    acc_t acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < kN; ++i) acc[c][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (KIND == 2)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int x = 0; x < NEXP; ++x) e[x & 7] = __builtin_amdgcn_exp2f(e[x & 7]) * -0.5f;
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) r += acc[c][0] + acc[c][kN - 1];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) r += e[i];
  out[(int64_t)blockIdx.x * kProbeThreads + tid] = r;
}

// 32 KiB of LDS read in 1 KiB rows: KIND 0 lane l reads bytes [16 l, 16 l +
// 16) of a row (ds_read_b128); KIND 1 lane l reads bytes [8 l, 8 l + 8) with
// the transposing read. Rows rotate per read; every address is in the array.
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) pb_lds_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned int buf[8192];
  const int tid = threadIdx.x;
  for (int i = tid; i < 8192; i += kProbeThreads) buf[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  unsigned acc = 0;
  typedef __attribute__((address_space(3))) i16x4_t lds_t;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = ((it * 8 + u) * 5 + (tid >> 6)) & 31;
      if constexpr (KIND == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(&buf[row * 256 + (tid & 63) * 4]);
        acc += v.x ^ v.y ^ v.z ^ v.w;
      } else {
        const uint2 v = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)&buf[row * 256 + (tid & 63) * 2]));
        acc += v.x ^ v.y;
      }
    }
  }
  out[(int64_t)blockIdx.x * kProbeThreads + tid] = (float)acc;
}

__device__ __forceinline__ uint4 nt_load16(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// A grid-stride loop over the buffer's 16-byte pieces, consecutive threads
// reading consecutive pieces, four pieces (one grid stride apart) in flight
// per thread.
__global__ void __launch_bounds__(kProbeThreads)
pb_stream_kernel(const char* src, int64_t pieces, float* out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  unsigned acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < pieces;
       i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < pieces) v[u] = nt_load16(src + (i + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < pieces) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = (float)acc;
}

__device__ __forceinline__ uint4 load16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// The decode gather without arithmetic: grid (heads, 1, sequences).
// MODE 0: K pass then V pass, non-temporal loads (the decode kernel's order);
// MODE 1: the same with ordinary loads; MODE 2: K and V of each block read
// together (the order of a one-pass online-softmax decode), non-temporal, two
// blocks of each in flight so that a wave holds the same 16 KiB as in MODE 0.
template <int MODE>
__global__ void __launch_bounds__(kProbeThreads)
pb_gather_kernel(const char* k_cache, const char* v_cache, const int32_t* block_tables,
                 const int32_t* context_lens, int heads, int block_bytes, int max_blocks,
                 float* out) {
  const int h = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = context_lens[b];
  const int nblk = (L + 15) / 16;
  const int nslice = block_bytes / 1024;            // 1 KiB slices per block and head
  const int64_t stride = (int64_t)heads * block_bytes;
  const int32_t* table = block_tables + (int64_t)b * max_blocks;
  unsigned acc = 0;
  const int64_t hoff = (int64_t)h * block_bytes + lane * 16;
  if constexpr (MODE == 2) {
    for (int n0 = wave; n0 < nblk; n0 += 8) {
      uint4 x[2][2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int n = n0 + 4 * u;
        if (n < nblk) {
          const int64_t ph = __builtin_amdgcn_readfirstlane(table[n]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < nslice) {
              x[u][0][i] = nt_load16(k_cache + hoff + ph * stride + i * 1024);
              x[u][1][i] = nt_load16(v_cache + hoff + ph * stride + i * 1024);
            }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (n0 + 4 * u < nblk)
#pragma unroll
          for (int kv = 0; kv < 2; ++kv)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < nslice) acc ^= x[u][kv][i].x ^ x[u][kv][i].y ^ x[u][kv][i].z ^ x[u][kv][i].w;
    }
  } else {
    for (int pass = 0; pass < 2; ++pass) {
      const char* base = (pass == 0 ? k_cache : v_cache) + hoff;
      for (int n0 = wave; n0 < nblk; n0 += 16) {
        uint4 x[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int n = n0 + 4 * u;
          if (n < nblk) {
            const int64_t ph = __builtin_amdgcn_readfirstlane(table[n]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < nslice)
                x[u][i] = MODE == 0 ? nt_load16(base + ph * stride + i * 1024)
                                    : load16(base + ph * stride + i * 1024);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (n0 + 4 * u < nblk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < nslice) acc ^= x[u][i].x ^ x[u][i].y ^ x[u][i].z ^ x[u][i].w;
      }
    }
  }
  out[((int64_t)b * heads + h) * kProbeThreads + threadIdx.x] = (float)acc;
}

// A materialised prefill bias read by (128-query tile, head, sequence)
// workgroups as the prefill kernels walk it: wave w reads rows 32 w .. +31 of
// its tile (rows below L only), W bytes of each row per iteration from the
// first key on, with 16-byte non-temporal loads in which G consecutive bytes
// of a row are read by G / 16 consecutive lanes; all W / 32 loads of an
// iteration are in flight together. bias: [seqs, heads, max_len, max_len]
// fp32; max_len a multiple of W / 4.
template <int W, int G>
__global__ void __launch_bounds__(kProbeThreads)
pb_bias_kernel(const float* bias, const int32_t* lens, int heads, int max_len, float* out) {
  constexpr int kInst = W / 32;               // 1 KiB loads per wave and iteration
  constexpr int kLanesPerRow = G / 16;
  constexpr int kRowsPerInst = 64 / kLanesPerRow;
  constexpr int kRowBlocks = 32 / kRowsPerInst;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = lens[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = tile * 128 + wave * 32;
  unsigned acc = 0;
  if (row0 < L) {
    const float* base = bias + (((int64_t)b * heads + h) * max_len) * max_len;
    const int nkeys = (L + W / 4 - 1) / (W / 4) * (W / 4);
    for (int k0 = 0; k0 < nkeys; k0 += W / 4) {
      uint4 x[kInst];
#pragma unroll
      for (int n = 0; n < kInst; ++n) {
        const int row = row0 + (n % kRowBlocks) * kRowsPerInst + lane / kLanesPerRow;
        const int col = k0 + ((n / kRowBlocks) * G + (lane % kLanesPerRow) * 16) / 4;
        x[n] = row < L ? nt_load16(reinterpret_cast<const char*>(base + (int64_t)row * max_len + col))
                       : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int n = 0; n < kInst; ++n) acc ^= x[n].x ^ x[n].y ^ x[n].z ^ x[n].w;
    }
  }
  out[(((int64_t)b * heads + h) * gridDim.x + tile) * kProbeThreads + threadIdx.x] = (float)acc;
}

// Whether matrix and vector work of different waves on one SIMD overlap:
// 8-wave workgroups (waves w and w + 4 share a SIMD); waves 0-3 run four
// independent v_mfma_f32_32x32x16_bf16 chains, waves 4-7 a vector loop of
// 8 v_exp_f32 and 16 v_fma_f32 per iteration, both `iters` iterations.
// MODE 0: only the matrix waves work, 1: only the vector waves, 2: both;
// MODE 3 and 4 as 0 and 2 with the four products of an iteration chained
// into one accumulator (each depends on the one before).
template <int MODE>
__global__ void __launch_bounds__(512) pb_mix_kernel(float* out, int iters, float seed) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  float r = 0.0f;
  if (wave < 4 && (MODE == 3 || MODE == 4)) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (float)(tid + i));
      b[i] = (__bf16)(seed * (float)(i - tid));
    }
    f16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    r += acc[0] + acc[15];
  }
  if (wave < 4 && (MODE == 0 || MODE == 2)) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (float)(tid + i));
      b[i] = (__bf16)(seed * (float)(i - tid));
    }
    f16_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) r += acc[c][0] + acc[c][15];
  }
  if (wave >= 4 && (MODE == 1 || MODE == 2 || MODE == 4)) {
    float e[8], f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = seed * (float)(tid + i) * 1e-3f;
      f[i] = seed * (float)(tid - i);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = __builtin_amdgcn_exp2f(e[i]) * -0.5f;
        f[i] = fmaf(f[i], 0.999f, e[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) r += e[i] + f[i];
  }
  out[(int64_t)blockIdx.x * 512 + tid] = r;
}

// Shader clock under load: each workgroup runs four v_mfma_f32_32x32x16_bf16
// chains per wave (KIND 0) or eight v_exp_f32 chains per thread (KIND 1) for
// `iters` iterations, and thread 0 writes the shader-clock (s_memtime) and
// constant 100 MHz (s_memrealtime) counter differences across that work to
// out[2 blockIdx], out[2 blockIdx + 1] (vector stores).
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) pb_clock_kernel(float* out, int iters, float seed) {
  const int tid = threadIdx.x;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float r = 0.0f;
  if constexpr (KIND == 0) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (float)(tid + i));
      b[i] = (__bf16)(seed * (float)(i - tid));
    }
    f16_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) r += acc[c][0];
  } else {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = seed * (float)(tid + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) r += x[i];
  }
  // the counters are read after the work's results exist
  __builtin_amdgcn_s_waitcnt(0);
  const float rr = __builtin_amdgcn_readfirstlane(__float_as_uint(r)) == 0x7fc00001u ? 1.0f : 0.0f;
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[2 * blockIdx.x] = (float)(t1 - t0) + rr;
    out[2 * blockIdx.x + 1] = (float)(r1 - r0);
  }
}

// Vector instruction rate: 8 independent chains per thread of v_add_f32
// (KIND 0), v_fma_f32 (1) or v_exp_f32 on the negated value (2).
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) pb_valu_kernel(float* out, int iters, float seed) {
  const int tid = threadIdx.x;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = seed * (float)(tid + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0) x[i] = x[i] + 0.5f;
      else if constexpr (KIND == 1) x[i] = fmaf(x[i], 0.999f, 0.25f);
      else x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += x[i];
  out[(int64_t)blockIdx.x * kProbeThreads + tid] = r;
}

template <int KIND, int CH, int NEXP>
int launch_mfma(float* out, int grid, int iters, hipStream_t s) {
  hipLaunchKernelGGL((pb_mfma_kernel<KIND, CH, NEXP>), dim3(grid), dim3(kProbeThreads), 0, s,
                     out, iters, 0.01f);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// grid = number of 4-wave workgroups; out holds grid * 256 floats.
// kind as above; chains 2, 4 or 8; exps 0, 1, 2 or 4 per product.
int pb_mfma(int kind, int chains, int exps, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
#define PB_CASE(K, C, E) \
  if (kind == K && chains == C && exps == E) return launch_mfma<K, C, E>(out, grid, iters, s);
#define PB_KIND(K) PB_CASE(K, 2, 0) PB_CASE(K, 4, 0) PB_CASE(K, 8, 0) PB_CASE(K, 2, 2) \
                   PB_CASE(K, 2, 4) PB_CASE(K, 4, 1) PB_CASE(K, 4, 2)
  PB_KIND(0) PB_KIND(1) PB_KIND(2) PB_KIND(3)
#undef PB_KIND
#undef PB_CASE
  return -1;
}

int pb_lds(int kind, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL((pb_lds_kernel<0>), dim3(grid), dim3(kProbeThreads), 0, s, out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL((pb_lds_kernel<1>), dim3(grid), dim3(kProbeThreads), 0, s, out, iters);
  else
    return -1;
  return (int)hipGetLastError();
}

// src: `bytes` of device memory (a multiple of 16); out: grid * 256 floats.
int pb_stream(const void* src, int64_t bytes, int grid, float* out, void* stream) {
  if (bytes % 16 != 0) return -1;
  hipLaunchKernelGGL(pb_stream_kernel, dim3(grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

// k_cache / v_cache: [num_blocks, heads, 16, D] (block_bytes = 16 * D * element
// size, a multiple of 1 KiB and at most 4 KiB); block_tables [seqs,
// max_blocks] with valid entries below ceil(L / 16); out: seqs * heads * 256
// floats.
// mode 0, 1 or 2 as for pb_gather_kernel.
int pb_gather(int mode, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              const int32_t* context_lens, int seqs, int heads, int block_bytes, int max_blocks,
              float* out, void* stream) {
  if (block_bytes % 1024 != 0 || block_bytes > 4096 || block_bytes <= 0) return -1;
  const char* k = static_cast<const char*>(k_cache);
  const char* v = static_cast<const char*>(v_cache);
  const dim3 grid(heads, 1, seqs);
  hipStream_t s = (hipStream_t)stream;
  if (mode == 0)
    hipLaunchKernelGGL(pb_gather_kernel<0>, grid, dim3(kProbeThreads), 0, s, k, v, block_tables,
                       context_lens, heads, block_bytes, max_blocks, out);
  else if (mode == 1)
    hipLaunchKernelGGL(pb_gather_kernel<1>, grid, dim3(kProbeThreads), 0, s, k, v, block_tables,
                       context_lens, heads, block_bytes, max_blocks, out);
  else if (mode == 2)
    hipLaunchKernelGGL(pb_gather_kernel<2>, grid, dim3(kProbeThreads), 0, s, k, v, block_tables,
                       context_lens, heads, block_bytes, max_blocks, out);
  else
    return -1;
  return (int)hipGetLastError();
}

// bias [seqs, heads, max_len, max_len] fp32, lens [seqs]; (w, g) one of
// (128, 128), (512, 128), (512, 512), (256, 256); out: ceil(max_len / 128) *
// heads * seqs * 256 floats.
int pb_bias(const float* bias, const int32_t* lens, int seqs, int heads, int max_len, int w,
            int g, float* out, void* stream) {
  if (max_len % 128 != 0) return -1;
  const dim3 grid(max_len / 128, heads, seqs);
  hipStream_t s = (hipStream_t)stream;
  if (w == 128 && g == 128)
    hipLaunchKernelGGL((pb_bias_kernel<128, 128>), grid, dim3(kProbeThreads), 0, s, bias, lens,
                       heads, max_len, out);
  else if (w == 512 && g == 128)
    hipLaunchKernelGGL((pb_bias_kernel<512, 128>), grid, dim3(kProbeThreads), 0, s, bias, lens,
                       heads, max_len, out);
  else if (w == 512 && g == 512)
    hipLaunchKernelGGL((pb_bias_kernel<512, 512>), grid, dim3(kProbeThreads), 0, s, bias, lens,
                       heads, max_len, out);
  else if (w == 256 && g == 256)
    hipLaunchKernelGGL((pb_bias_kernel<256, 256>), grid, dim3(kProbeThreads), 0, s, bias, lens,
                       heads, max_len, out);
  else
    return -1;
  return (int)hipGetLastError();
}

// kind 0 or 1 as for pb_clock_kernel; out: 2 * grid floats.
int pb_clock(int kind, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(pb_clock_kernel<0>, dim3(grid), dim3(kProbeThreads), 0, s, out, iters, 0.01f);
  else if (kind == 1)
    hipLaunchKernelGGL(pb_clock_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, s, out, iters, 0.01f);
  else
    return -1;
  return (int)hipGetLastError();
}

// kind 0, 1 or 2 as for pb_valu_kernel; out: grid * 256 floats.
int pb_valu(int kind, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(pb_valu_kernel<0>, dim3(grid), dim3(kProbeThreads), 0, s, out, iters, 0.01f);
  else if (kind == 1)
    hipLaunchKernelGGL(pb_valu_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, s, out, iters, 0.01f);
  else if (kind == 2)
    hipLaunchKernelGGL(pb_valu_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, s, out, iters, 0.01f);
  else
    return -1;
  return (int)hipGetLastError();
}

// mode 0 to 4 as for pb_mix_kernel; out: grid * 512 floats.
int pb_mix(int mode, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (mode == 0)
    hipLaunchKernelGGL(pb_mix_kernel<0>, dim3(grid), dim3(512), 0, s, out, iters, 0.01f);
  else if (mode == 1)
    hipLaunchKernelGGL(pb_mix_kernel<1>, dim3(grid), dim3(512), 0, s, out, iters, 0.01f);
  else if (mode == 2)
    hipLaunchKernelGGL(pb_mix_kernel<2>, dim3(grid), dim3(512), 0, s, out, iters, 0.01f);
  else if (mode == 3)
    hipLaunchKernelGGL(pb_mix_kernel<3>, dim3(grid), dim3(512), 0, s, out, iters, 0.01f);
  else if (mode == 4)
    hipLaunchKernelGGL(pb_mix_kernel<4>, dim3(grid), dim3(512), 0, s, out, iters, 0.01f);
  else
    return -1;
  return (int)hipGetLastError();
}

}  // extern "C"
