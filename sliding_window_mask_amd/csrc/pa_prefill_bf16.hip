// bf16 MFMA prefill attention over a paged KV cache for gfx950 (CDNA4).
//
// Same computation as the fp32 prefill (softmax((q K^T + A) * scale) V over
// the keys a row may see: bidirectional, causal, sliding window, optional
// bias), for bf16 q / K / V / out, on v_mfma_f32_16x16x32_bf16: bf16 products
// accumulated in fp32. The softmax runs in fp32; the weights P are rounded to
// bf16 for the P.V contraction and the row sums are taken over the same
// rounded weights, so out = sum(P~ V) / sum(P~) is an exact weighted mean.
//
// One workgroup of 4 wave64s per (64-query tile, head, sequence), numbered
// so that all query tiles of a (sequence, head) share an XCD. Keys are
// walked in 32-key tiles through a double-buffered LDS ring (tile k+2 in
// flight from memory while tile k is multiplied, block-table entries one
// tile further ahead).
//
// Operand layout (16x16x32, lane l, g = l / 16, c = l % 16; every lane feeds
// 8 bf16 of A and B, and lanes of one group g contract the same 8 positions):
// * S^T = K Q^T, step st of D/32: lane l feeds K[key c][(D/4) g + 8 st + e]
//   and Q[query c][same dim] (e = 0..7) -- 16 contiguous bytes each. Lane l
//   ends holding S^T[key 4g + r][query c], r = 0..3, for each 16-key chunk.
// * O^T = V^T P^T over the tile's 32 keys: element e of lane group g is key
//   4g + e (e < 4, first chunk) or 16 + 4g + e - 4 (second chunk), so the
//   P operand is exactly the lane's own 8 softmax weights. The V operand
//   needs 8 keys of one dim; V is therefore staged into LDS transposed,
//   V^T[dim][key] (row stride 36 bf16: conflict-free 8-byte reads and
//   writes), and lane l reads V^T[16 dt + c][4g .. 4g+3] and [16 + 4g ..].
//   Lane l ends holding O^T[dim 16 dt + 4g + r][query c].
#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kQT = 64;         // queries per workgroup (16 per wave)
constexpr int kKT = 32;         // keys per tile (one 32-deep P.V contraction)
constexpr int kVRow = kKT + 4;  // V^T row stride (bf16)

__device__ __forceinline__ float4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                              float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// BIAS: 0 none, 1 materialised (padded or ragged) fp32 bias, 2 T5 relative
// position bias from a bucket table.
template <int D, int BIAS, bool CAUSAL, bool WINDOW>
__global__ void __launch_bounds__(kThreads)
pa_prefill_bf16(PrefillArgs a) {
  constexpr int kKRow = D + 8;                 // K row stride in LDS (bf16)
  constexpr int kSteps = D / 32;               // 8-element steps per lane group
  constexpr int kNDT = D / 16;                 // 16-dim output slices
  constexpr int kKLoads = kKT * D / 8 / kThreads;        // 16-byte K loads per thread
  constexpr int kVUnits = (D / 2) * (kKT / 4) / kThreads;  // (2 dims x 4 keys) units
  static_assert(kKLoads >= 1 && kVUnits >= 1, "tile shape");

  const int H = a.num_heads;
  int pair, tile;
  prefill_tile_of(blockIdx.x, a.num_qtiles, pair, tile);
  if (pair >= a.num_seqs * H) return;
  const int b = pair / H;
  const int h = pair % H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;

  const int L = a.context_lens[b];
  const int q0 = a.query_start_loc[b];
  const int nq = a.query_start_loc[b + 1] - q0;
  const int t_first = tile * kQT;
  if (t_first >= nq) return;
  const int pos0 = L - nq;

  const int wg_last = min(t_first + kQT, nq) - 1;
  int wg_lo, wg_hi;
  prefill_key_range(pos0 + t_first, pos0 + wg_last, L, a.window, CAUSAL, wg_lo, wg_hi);
  const int w_first = t_first + wave * 16;
  const bool wave_active = w_first < nq;
  const int w_last = min(w_first + 16, nq) - 1;
  const bool wave_full = w_last == w_first + 15;
  int wv_lo = 0, wv_hi = 0;
  if (wave_active) prefill_key_range(pos0 + w_first, pos0 + w_last, L, a.window, CAUSAL, wv_lo, wv_hi);
  const int wp0 = pos0 + w_first, wp1 = pos0 + w_last;

  const int t = w_first + c;
  const bool row_ok = t < nq;
  const int p = pos0 + t;
  const float cs = a.scale_log2;

  // Q operand: kSteps x 8 bf16 (rows past n_q are zero)
  bf16x8_t qv[kSteps];
  {
    const int tq = row_ok ? t : t_first;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + (D / 4) * g);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      uint4 v = qrow[st];
      if (!row_ok) v = make_uint4(0u, 0u, 0u, 0u);
      qv[st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  __shared__ uint16_t k_lds[2][kKT * kKRow];   // K tile, row-major [key][dim]
  __shared__ uint16_t v_lds[2][D * kVRow];     // V tile, transposed [dim][key]
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 1 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md; i += kThreads)
      rel_lds[i] = rel_bias(i - rel_md, a.rel, head_row) * cs;
  }

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int kstart = wg_lo & ~(kBlockSize - 1);
  const int ntiles = wg_hi > kstart ? (wg_hi - kstart + kKT - 1) / kKT : 0;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;

  int tb[2];                                   // block ids of one tile (uniform)
  auto load_table = [&](int tk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = (kstart + tk * kKT) / kBlockSize + i;
      tb[i] = blk < nblk_seq ? table[blk] : 0;
    }
  };
  // global -> registers: K as 16-byte row pieces, V as 4-byte (2-dim) pieces
  // of 4 consecutive keys, repacked below into V^T rows
  uint4 kst[kKLoads];
  uint32_t vst[kVUnits][4];
  auto fetch = [&](int tk) {
    const int base = kstart + tk * kKT;
    const bool tail = base + kKT > L;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;        // 16-byte piece index in the tile
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      const int j = base + r;
      const int64_t off = (((int64_t)tb[r / kBlockSize] * H + h) * kBlockSize + j % kBlockSize) * D + col;
      kst[i] = (!tail || j < L) ? *reinterpret_cast<const uint4*>(kc + off)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kVUnits; ++u) {
      const int e = u * kThreads + tid;
      const int dp = e % (D / 2), kg = e / (D / 2);   // dims 2dp, 2dp+1; keys 4kg..4kg+3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kg + i;
        const int j = base + r;
        const int64_t off = (((int64_t)tb[r / kBlockSize] * H + h) * kBlockSize + j % kBlockSize) * D + 2 * dp;
        vst[u][i] = (!tail || j < L) ? *reinterpret_cast<const uint32_t*>(vc + off) : 0u;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][r * kKRow + col]) = kst[i];
    }
#pragma unroll
    for (int u = 0; u < kVUnits; ++u) {
      const int e = u * kThreads + tid;
      const int dp = e % (D / 2), kg = e / (D / 2);
      // low halves = dim 2dp of keys 4kg..4kg+3, high halves = dim 2dp+1
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(vst[u][1], vst[u][0], 0x05040100u),
                                  __builtin_amdgcn_perm(vst[u][3], vst[u][2], 0x05040100u));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(vst[u][1], vst[u][0], 0x07060302u),
                                  __builtin_amdgcn_perm(vst[u][3], vst[u][2], 0x07060302u));
      *reinterpret_cast<uint2*>(&v_lds[buf][(2 * dp) * kVRow + 4 * kg]) = lo;
      *reinterpret_cast<uint2*>(&v_lds[buf][(2 * dp + 1) * kVRow + 4 * kg]) = hi;
    }
  };

  float4_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) acc[dt] = float4_t{0, 0, 0, 0};
  float m_ref = -INFINITY, l_run = 0.0f;
  const int tb_row = row_ok ? t : t_first;
  const float* bias_row = nullptr;
  if (BIAS == 1)
    bias_row = a.bias_start
                   ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                   : a.attn_bias + (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) *
                                       a.max_seq_len;

  if (ntiles > 0) {
    load_table(0);
    fetch(0);
    stash(0);
    if (ntiles > 1) {
      load_table(1);
      fetch(1);
      if (ntiles > 2) load_table(2);
    }
  }
  __syncthreads();

  for (int tk = 0; tk < ntiles; ++tk) {
    const int buf = tk & 1;
    const int base = kstart + tk * kKT;
    if (wave_active && base < wv_hi && base + kKT > wv_lo) {
      // ---- S^T for the two 16-key chunks ----
      float4_t s[2] = {float4_t{0, 0, 0, 0}, float4_t{0, 0, 0, 0}};
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const uint4 kv = *reinterpret_cast<const uint4*>(
              &k_lds[buf][(ch * 16 + c) * kKRow + (D / 4) * g + 8 * st]);
          s[ch] = mfma_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[st], s[ch]);
        }
      }
      // ---- scale, bias, mask (base-2 scores) ----
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int c0 = base + ch * 16;
        const int j0 = c0 + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[ch][r] * cs;
          if constexpr (BIAS == 1) x = x + bias_row[min(j0 + r, L - 1)] * cs;
          if constexpr (BIAS == 2) x = x + rel_lds[min(max(j0 + r - p, -rel_md), rel_md) + rel_md];
          s[ch][r] = x;
        }
        bool whole = wave_full && c0 + 16 <= L;
        if constexpr (CAUSAL) whole = whole && c0 + 15 <= wp0;
        if constexpr (WINDOW) whole = whole && wp1 - c0 < a.window && c0 + 15 - wp0 < a.window;
        if (!whole) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            bool vis = row_ok && j < L;
            if constexpr (CAUSAL) vis = vis && j <= p;
            if constexpr (WINDOW) vis = vis && abs(p - j) < a.window;
            s[ch][r] = vis ? s[ch][r] : -INFINITY;
          }
        }
      }
      // ---- online softmax with a lazily moved reference (as in fp32) ----
      float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      const bool move = mt > m_ref + 8.0f;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;
        m_ref = move ? mt : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
      bf16x8_t pw;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(s[ch][r] - m_use);
          pw[4 * ch + r] = pb;
          l_run += bf16_bits_to_f32(__builtin_bit_cast(uint16_t, pb));
        }
      }
      // ---- O^T += V^T P^T over the tile's 32 keys ----
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
        const uint16_t* vrow = &v_lds[buf][(16 * dt + c) * kVRow + 4 * g];
        const uint2 v0 = *reinterpret_cast<const uint2*>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 16);
        const uint4 vv = make_uint4(v0.x, v0.y, v1.x, v1.y);
        acc[dt] = mfma_bf16(__builtin_bit_cast(bf16x8_t, vv), pw, acc[dt]);
      }
    }
    if (tk + 1 < ntiles) stash(buf ^ 1);
    if (tk + 2 < ntiles) {
      fetch(tk + 2);
      if (tk + 3 < ntiles) load_table(tk + 3);
    }
    __syncthreads();
  }

  // ---- epilogue: out = O / l, rounded to bf16 ----
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + t) * H + h) * D;
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t o = {(__bf16)(acc[dt][0] * inv), (__bf16)(acc[dt][1] * inv),
                  (__bf16)(acc[dt][2] * inv), (__bf16)(acc[dt][3] * inv)};
    *reinterpret_cast<bf16x4_t*>(orow + 16 * dt + 4 * g) = o;
  }
}

template <int D, int BIAS>
void launch_mask(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.causal) {
    if (a.window > 0)
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, true, true>), grid, dim3(kThreads), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, true, false>), grid, dim3(kThreads), 0,
                         stream, a);
  } else {
    if (a.window > 0)
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, false, true>), grid, dim3(kThreads), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, false, false>), grid, dim3(kThreads), 0,
                         stream, a);
  }
}

template <int D>
hipError_t launch_d(PrefillArgs a, hipStream_t stream) {
  a.num_qtiles = (a.max_seq_len + kQT - 1) / kQT;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  const int64_t nwg = (pairs + kXcds - 1) / kXcds * kXcds * a.num_qtiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  if (a.rel.table)
    launch_mask<D, 2>(a, grid, stream);
  else if (a.attn_bias)
    launch_mask<D, 1>(a, grid, stream);
  else
    launch_mask<D, 0>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace pa
