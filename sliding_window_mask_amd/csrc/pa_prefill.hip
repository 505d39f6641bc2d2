// MFMA prefill attention over a paged KV cache for gfx950 (CDNA4, wave64).
//
// Every query row computes softmax((q K^T + A) * scale) V ("[Kernel][Model]
// PagedAttention: Support custom attention bias for T5 model (1/2)", formula
// in the PR description) over the keys it may see: all L keys of its sequence
// for bidirectional encoder-only attention, keys j <= p for a causal prompt,
// and with a sliding window W only |p - j| < W ("[V1] Add sliding window
// support to Flex Attention backend": bidirectional attention with a per-layer
// window). Both contractions run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, fp32 products and accumulation).
//
// Work decomposition: one workgroup of 4 wave64s per (64-query tile, head,
// sequence); wave w owns 16 query rows. The workgroup walks the keys its rows
// can see in tiles of 64 keys (32 at D = 128), gathering each block through the
// block table into LDS (K and V, rows padded by 4 floats against bank
// conflicts) while the previous tile is being multiplied: the next tile's
// global loads are issued into registers before the current tile's MFMAs.
// Key tiles, and 16-key chunks within them, that no row of a wave can see are
// skipped, so a window of 64 costs about the band, not the full square.
//
// MFMA operand layout (16x16x4, lane l, g = l / 16, c = l % 16):
//   A[i][k] from lane (i + 16 k), B[k][j] from lane (j + 16 k),
//   D[4 g + r][c] in accumulator register r of lane l.
// S^T = K Q^T: A = 16 keys x 4 dims, B = 4 dims x 16 queries. Step kd of the
//   D/4 steps contracts dims {kd + (D/4) g}: lane l feeds K[key c][(D/4) g + kd]
//   and Q[query c][(D/4) g + kd], i.e. a contiguous run of D/4 floats per lane.
//   Lane l then holds S^T[key 4 g + r][query c]: one query per lane column.
// O^T = V^T P^T: for output slice dt (D/16 slices) and key quad kk, A row i is
//   dim (D/16) i + dt and column k is key 4 k + kk; B[k][j] = P^T[key 4k+kk][j]
//   is exactly register kk of lane (j + 16 k) from the S^T step. Lane l ends
//   holding query c, dims (D/4) g + (D/16) r + dt: a contiguous run of D/4.
// The online softmax therefore never moves scores between lanes except for
// the row max (lanes c, c+16, c+32, c+48 share a query).
#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kQTile = 64;      // queries per workgroup (16 per wave)
constexpr int kPad = 4;         // floats of padding per LDS row

// Keys per LDS tile: 4 blocks at D = 64, 2 at D = 128 (K + V tiles stay
// under 64 KiB of LDS either way).
template <int D>
constexpr int key_tile() { return D == 64 ? 64 : 32; }

__device__ __forceinline__ float4_t mfma16x16x4(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Visible key interval [lo, hi) for query positions [p0, p1] of a sequence of
// length L (caller guarantees p0 <= p1 < L).
__device__ __forceinline__ void key_range(int p0, int p1, int L, int window, int causal,
                                          int& lo, int& hi) {
  lo = 0;
  hi = causal ? p1 + 1 : L;
  if (window > 0) {
    lo = max(0, p0 - window + 1);
    if (!causal) hi = min(L, p1 + window);
  }
}

template <int D, bool HAS_BIAS>
__global__ void __launch_bounds__(kThreads)
pa_prefill_f32(PrefillArgs a) {
  constexpr int kKTile = key_tile<D>();
  constexpr int kChunks = kKTile / 16;    // 16-key chunks per tile
  constexpr int kRow = D + kPad;          // LDS row stride (floats)
  constexpr int kDQ = D / 4;              // dims per lane group in the S^T step
  constexpr int kNDT = D / 16;            // output slices of 16 dims
  constexpr int kLoads = kKTile * D / 4 / kThreads;  // 16-byte loads per thread per tile

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int H = a.num_heads;

  const int L = a.context_lens[b];
  const int q0 = a.query_start_loc[b];
  const int nq = a.query_start_loc[b + 1] - q0;
  const int t_first = tile * kQTile;
  if (t_first >= nq) return;
  const int pos0 = L - nq;                 // position of query 0

  // workgroup and wave query ranges (positions), clamped to valid rows
  const int wg_last = min(t_first + kQTile, nq) - 1;
  int wg_lo, wg_hi;
  key_range(pos0 + t_first, pos0 + wg_last, L, a.window, a.causal, wg_lo, wg_hi);
  const int w_first = t_first + wave * 16;
  const bool wave_active = w_first < nq;
  const int w_last = min(w_first + 16, nq) - 1;
  int wv_lo = 0, wv_hi = 0;
  if (wave_active) key_range(pos0 + w_first, pos0 + w_last, L, a.window, a.causal, wv_lo, wv_hi);

  // this lane's query row
  const int t = w_first + c;
  const bool row_ok = t < nq;
  const int p = pos0 + t;

  // Q operand: D/4 contiguous floats per lane
  float qreg[kDQ];
  {
    // rows past n_q read the tile's first (valid) row and are zeroed
    const int tq = row_ok ? t : t_first;
    const float* qrow = static_cast<const float*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + kDQ * g;
#pragma unroll
    for (int i = 0; i < kDQ; i += 4) {
      float4_t v = *reinterpret_cast<const float4_t*>(qrow + i);
      if (!row_ok) v = float4_t{0, 0, 0, 0};
      qreg[i] = v[0]; qreg[i + 1] = v[1]; qreg[i + 2] = v[2]; qreg[i + 3] = v[3];
    }
  }

  __shared__ float k_lds[kKTile * kRow];
  __shared__ float v_lds[kKTile * kRow];

  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int kstart = wg_lo & ~(kBlockSize - 1);
  const int ntiles = wg_hi > kstart ? (wg_hi - kstart + kKTile - 1) / kKTile : 0;

  // global -> register staging of one key tile (zeros for keys >= L)
  float4_t kst[kLoads], vst[kLoads];
  auto fetch = [&](int tk) {
    const int base = kstart + tk * kKTile;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = (i * kThreads + tid) * 4;      // float index within the tile
      const int r = e / D, col = e % D;
      const int j = base + r;
      if (j < L) {
        const int64_t phys = table[j / kBlockSize];
        const int64_t off = ((phys * H + h) * kBlockSize + (j % kBlockSize)) * D + col;
        kst[i] = *reinterpret_cast<const float4_t*>(kc + off);
        vst[i] = *reinterpret_cast<const float4_t*>(vc + off);
      } else {
        kst[i] = float4_t{0, 0, 0, 0};
        vst[i] = float4_t{0, 0, 0, 0};
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = (i * kThreads + tid) * 4;
      const int r = e / D, col = e % D;
      *reinterpret_cast<float4_t*>(&k_lds[r * kRow + col]) = kst[i];
      *reinterpret_cast<float4_t*>(&v_lds[r * kRow + col]) = vst[i];
    }
  };

  float4_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) acc[dt] = float4_t{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;
  const float* bias_row =
      (HAS_BIAS && row_ok)
          ? a.attn_bias + (((int64_t)b * H + h) * a.max_seq_len + p) * a.max_seq_len
          : nullptr;

  if (ntiles > 0) fetch(0);
  for (int tk = 0; tk < ntiles; ++tk) {
    __syncthreads();                     // everyone is done reading the old tile
    stash();
    __syncthreads();
    if (tk + 1 < ntiles) fetch(tk + 1);  // in flight during this tile's math
    const int base = kstart + tk * kKTile;
    if (!wave_active || base >= wv_hi || base + kKTile <= wv_lo) continue;

    // ---- S^T = K Q^T for the chunks of 16 keys ----
    float4_t s[kChunks];
    bool live[kChunks];
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      const int c0 = base + ch * 16;
      live[ch] = c0 < wv_hi && c0 + 16 > wv_lo;
      s[ch] = float4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      if (!live[ch]) continue;
      const float* krow = &k_lds[(ch * 16 + c) * kRow + kDQ * g];
#pragma unroll
      for (int i = 0; i < kDQ; i += 4) {
        const float4_t kv = *reinterpret_cast<const float4_t*>(krow + i);
        s[ch] = mfma16x16x4(kv[0], qreg[i], s[ch]);
        s[ch] = mfma16x16x4(kv[1], qreg[i + 1], s[ch]);
        s[ch] = mfma16x16x4(kv[2], qreg[i + 2], s[ch]);
        s[ch] = mfma16x16x4(kv[3], qreg[i + 3], s[ch]);
      }
    }

    // ---- scores, mask, online softmax (query c, keys 4g + r of each chunk) ----
    float mt = -INFINITY;
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = base + ch * 16 + 4 * g + r;
        bool vis = live[ch] && row_ok && j < L;
        if (a.causal) vis = vis && j <= p;
        if (a.window > 0) vis = vis && abs(p - j) < a.window;
        float x = -INFINITY;
        if (vis) {
          float tsum = s[ch][r];
          if constexpr (HAS_BIAS) tsum = tsum + bias_row[j];
          x = tsum * a.scale_log2;
        }
        s[ch][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(s[ch][r] - m_use);
        s[ch][r] = pr;
        lsum += pr;
      }
    }
    l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
    for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      if (!live[ch]) continue;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float* vrow = &v_lds[(ch * 16 + 4 * g + kk) * kRow + kNDT * c];
        float vv[kNDT];
#pragma unroll
        for (int i = 0; i < kNDT; i += 4) {
          const float4_t x = *reinterpret_cast<const float4_t*>(vrow + i);
          vv[i] = x[0]; vv[i + 1] = x[1]; vv[i + 2] = x[2]; vv[i + 3] = x[3];
        }
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acc[dt] = mfma16x16x4(vv[dt], s[ch][kk], acc[dt]);
      }
    }
  }

  // ---- epilogue: out = O / l ----
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* orow = static_cast<float*>(a.out) + ((int64_t)(q0 + t) * H + h) * D + kDQ * g;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int dt = 0; dt < kNDT; dt += 4) {
      float4_t o = {acc[dt][r] * inv, acc[dt + 1][r] * inv, acc[dt + 2][r] * inv,
                    acc[dt + 3][r] * inv};
      *reinterpret_cast<float4_t*>(orow + kNDT * r + dt) = o;
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  dim3 grid((a.max_seq_len + kQTile - 1) / kQTile, a.num_heads, a.num_seqs);
  if (a.attn_bias)
    hipLaunchKernelGGL((pa_prefill_f32<D, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_f32<D, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.dtype != 0) return hipErrorInvalidValue;   // host API rejects bf16 first
  return a.head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace pa
