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
// sequence); wave w owns 16 query rows. Workgroups are numbered so that every
// query tile of one (sequence, head) lands on the same XCD (the hardware
// deals consecutive workgroup ids round-robin over the 8 XCDs): the K/V of a
// sequence is then pulled into one XCD's L2 and re-read from there by all of
// its query tiles. Without a window, and for batches of up to 63 sequences,
// the (sequence, head) pairs are dealt longest sequence first, so that the
// launch does not end on a few long workgroups that started last.
//
// The workgroup walks the keys its rows can see in tiles of 16 keys. Tiles are gathered through the block table into a double-buffered
// LDS ring (rows padded by 4 floats against bank conflicts) with one barrier
// per tile: while tile k is multiplied, tile k+1 sits in the other LDS buffer
// and tile k+2 is in flight from memory into registers; the block-table
// entries are read one more tile ahead, so no key load waits on a table load.
// Tiles that no row of a wave can see are skipped by that wave, so a window
// of 64 costs about the band, not the full square; 16-key chunks that every
// row of the wave sees whole skip the per-element mask. Causal and windowed
// masks are compile-time variants, so the full-attention kernel carries no
// mask arithmetic at all except at the sequence end.
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
constexpr int kWaves = kThreads / 64;
// 16-query groups per wave at D = 64 (the workgroup covers 64 * groups queries)
#ifndef PA_PREFILL_GROUPS
#define PA_PREFILL_GROUPS 1
#endif
#ifndef PA_PREFILL_PAD
#define PA_PREFILL_PAD 4
#endif
constexpr int kPad = PA_PREFILL_PAD;   // floats of padding per LDS row

// Keys per LDS tile at D = 64 (16 at D = 128). 16-key tiles keep the two
// K + V buffers at 17 KiB, so 6-7 waves per SIMD fit (32-key tiles: 34 KiB,
// 4 workgroups per CU); measured on the ModernBERT-shaped layers, full
// attention runs equally fast with either and window-64 layers 6% faster
// with 16 (the band's edges waste less of a tile).
#ifndef PA_PREFILL_KTILE64
#define PA_PREFILL_KTILE64 16
#endif
template <int D>
constexpr int key_tile() { return D == 64 ? PA_PREFILL_KTILE64 : 16; }

__device__ __forceinline__ float4_t mfma16x16x4(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// IEEE maximum (NaN-propagating): maps onto v_maximum3_f32 with no operand
// canonicalisation, which fmaxf needs on raw MFMA results.
__device__ __forceinline__ float vmax(float x, float y) {
  return __builtin_elementwise_maximum(x, y);
}

// BIAS: 0 none, 1 materialised attn_bias[b, h, p, j], 2 T5 relative-position
// bias from a bucket table (a.rel).
// BAND: 0 no band, 1 sliding window, 2 chunked local attention (separate
// variants so that the window's mask stays a compare against a uniform W).
template <int D, int NG, int BIAS, bool CAUSAL, int BAND>
__global__ void __launch_bounds__(kThreads)
pa_prefill_f32(PrefillArgs a) {
  constexpr bool WINDOW = BAND != 0;   // banded: window or chunks
  constexpr int kKTile = key_tile<D>();
  constexpr int kChunks = kKTile / 16;               // 16-key chunks per tile
  constexpr int kRow = D + kPad;                     // LDS row stride (floats)
  constexpr int kDQ = D / 4;                         // dims per lane group (S^T step)
  constexpr int kNDT = D / 16;                       // output slices of 16 dims
  constexpr int kLoads = kKTile * D / 4 / kThreads;  // 16-byte loads per thread per tile
  constexpr int kRowsPerLoad = kThreads * 4 / D;     // tile rows one load instruction covers
  constexpr int kWaveRows = 16 * NG;                 // query rows per wave
  constexpr int kQT = kWaves * kWaveRows;            // query rows per workgroup
  static_assert(kLoads >= 1 && kRowsPerLoad <= 16 && 16 % kRowsPerLoad == 0, "tile shape");

  // ---- XCD-aware workgroup numbering, longest sequences first ----
  const int H = a.num_heads;
  int b, h, tile, L, q0, nq;
  if (!prefill_work_of(blockIdx.x, a, b, h, tile, L, q0, nq)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int c = lane & 15;
  const int g = lane >> 4;

  const int t_first = tile * kQT;
  if (t_first >= nq) return;
  const int pos0 = L - nq;                 // position of query 0

  // workgroup and wave query ranges (positions), clamped to valid rows
  const int wg_last = min(t_first + kQT, nq) - 1;
  int wg_lo, wg_hi;
  prefill_key_range(pos0 + t_first, pos0 + wg_last, L, a.window, a.chunk, CAUSAL, wg_lo,
                    wg_hi);
  const int w_first = t_first + wave * kWaveRows;
  const bool wave_active = w_first < nq;
  int wv_lo = 0, wv_hi = 0;
  if (wave_active)
    prefill_key_range(pos0 + w_first, pos0 + min(w_first + kWaveRows, nq) - 1, L, a.window,
                      a.chunk, CAUSAL, wv_lo, wv_hi);

  // per query group: first/last existing position, this lane's row. Masking
  // of partly visible chunks: with d = p - j for key j = c0 + 4g + r,
  // d = dq - c0 - r, and the key is visible iff dlo < d (j < L, causal
  // j <= p, window p - j > -W, chunk start) and, with a window or chunks,
  // d < dhi (window W, or the end of p's chunk). Keys [wlo, whi) are inside
  // the window or chunk of every row of the group.
  // Rows past n_q see no key at all (their dlo is the largest int), and where
  // a chunk is seen whole by the group they read the bias row of the group's
  // first existing query (fr): the bias entries of keys a row cannot see are
  // never read. A group with no existing row (possible only with NG > 1)
  // takes the workgroup's last query as its only row.
  int gp0[NG], gp1[NG], fr[NG], t[NG], p[NG], dq[NG], dlo[NG], dhi[NG], wlo[NG], whi[NG];
  bool row_ok[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int first = w_first + 16 * q;
    fr[q] = min(first, nq - 1);
    gp0[q] = pos0 + fr[q];
    gp1[q] = pos0 + max(min(first + 16, nq) - 1, fr[q]);
    t[q] = first + c;
    row_ok[q] = t[q] < nq;
    p[q] = pos0 + t[q];
    dq[q] = p[q] - 4 * g;
    if constexpr (BAND == 1) {
      dlo[q] = max(CAUSAL ? max(p[q] - L, -1) : p[q] - L, -a.window);
      dhi[q] = wlo[q] = whi[q] = 0;
    } else if constexpr (BAND == 2) {
      prefill_row_bounds(p[q], L, a.window, a.chunk, CAUSAL, dlo[q], dhi[q]);
      prefill_common_keys(gp0[q], gp1[q], a.window, a.chunk, wlo[q], whi[q]);
    } else {
      dlo[q] = CAUSAL ? max(p[q] - L, -1) : p[q] - L;
      dhi[q] = wlo[q] = whi[q] = 0;
    }
    if (!row_ok[q]) dlo[q] = 0x7fffffff;
  }

  // Q operands: D/4 contiguous floats per lane, pre-multiplied by
  // scale * log2(e) so that S^T comes out of the matrix cores already in the
  // base-2 score domain (rows past n_q are zero)
  const float cs = a.scale_log2;
  float qreg[NG][kDQ];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int tq = row_ok[q] ? t[q] : t_first;
    const float* qrow =
        static_cast<const float*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + kDQ * g;
#pragma unroll
    for (int i = 0; i < kDQ; i += 4) {
      float4_t v = *reinterpret_cast<const float4_t*>(qrow + i);
      if (!row_ok[q]) v = float4_t{0, 0, 0, 0};
      qreg[q][i] = v[0] * cs; qreg[q][i + 1] = v[1] * cs; qreg[q][i + 2] = v[2] * cs;
      qreg[q][i + 3] = v[3] * cs;
    }
  }

  __shared__ float kv_lds[2][2][kKTile * kRow];      // [buffer][K, V][row * kRow + col]
  // T5 bias of relative position r = j - p, for r in [-max_distance, max_distance]
  // (longer distances share the end buckets), pre-multiplied by scale * log2(e)
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 1 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md; i += kThreads)
      rel_lds[i] = rel_bias(i - rel_md, a.rel, head_row) * a.scale_log2;
  }

  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int kstart = wg_lo & ~(kBlockSize - 1);
  const int ntiles = wg_hi > kstart ? (wg_hi - kstart + kKTile - 1) / kKTile : 0;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;
  // Windowed launches visit the workgroup's key tiles in a rotated order:
  // first the 64-key segment of the band whose index (key / 64) is a
  // multiple of 3, then the following ones, wrapping round. Each segment is
  // read by about three neighbouring query tiles, and this way all of them
  // read it in the same third of their loop, while it is still in L2.
  int rot = 0;
  if constexpr (WINDOW) {
    const int seg0 = kstart / 64;
    const int first = (seg0 + (3 - seg0 % 3) % 3) * 64;
    if (first > kstart && first < kstart + ntiles * kKTile) rot = (first - kstart) / kKTile;
  }
  auto tile_base = [&](int tk) {
    int p = tk + rot;
    if (p >= ntiles) p -= ntiles;
    return kstart + p * kKTile;
  };

  // block-table entries of one tile (uniform across the workgroup)
  constexpr int kTB = (kKTile + kBlockSize - 1) / kBlockSize;
  int tb[kTB];
  auto load_table = [&](int tk) {
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const int blk = tile_base(tk) / kBlockSize + i;
      tb[i] = blk < nblk_seq ? table[blk] : 0;
    }
  };
  // global -> registers: one tile of K and V. One load instruction covers
  // whole rows of one cache block, so its address is a uniform block base
  // plus a per-lane offset that is the same for every tile. Rows at or past
  // L are read from the sequence's last block, or from block 0 for a block
  // past it (both in the pool): K there only feeds scores the mask drops,
  // and V is zeroed so that a zero weight never meets a NaN.
  float4_t kst[kLoads], vst[kLoads];
  auto fetch = [&](int tk) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = i * kRowsPerLoad + tid / (D / 4);
      const int col = (tid % (D / 4)) * 4;
      const int64_t blk_off = ((int64_t)tb[(i * kRowsPerLoad) / kBlockSize] * H + h) *
                              (kBlockSize * D);
      const uint32_t in_blk = (uint32_t)((r % kBlockSize) * D + col);
      kst[i] = *reinterpret_cast<const float4_t*>(kc + blk_off + in_blk);
      vst[i] = *reinterpret_cast<const float4_t*>(vc + blk_off + in_blk);
    }
  };
  // V rows at or past L are zeroed here, when the registers are stored, not
  // in fetch: a select right after the loads would make every wave wait for
  // them at once instead of a tile later
  auto stash = [&](int buf, int tk) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = i * kRowsPerLoad + tid / (D / 4);
      const int col = (tid % (D / 4)) * 4;
      *reinterpret_cast<float4_t*>(&kv_lds[buf][0][r * kRow + col]) = kst[i];
      *reinterpret_cast<float4_t*>(&kv_lds[buf][1][r * kRow + col]) = vst[i];
    }
    const int base = tile_base(tk);
    if (base + kKTile > L) {   // uniform: only a sequence's last tile
      // the zero is made here, not hoisted into a register held across the loop
      float z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = i * kRowsPerLoad + tid / (D / 4);
        const int col = (tid % (D / 4)) * 4;
        if (base + r >= L)
          *reinterpret_cast<float4_t*>(&kv_lds[buf][1][r * kRow + col]) = float4_t{z, z, z, z};
      }
    }
  };

  float4_t acc[NG][kNDT];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int dt = 0; dt < kNDT; ++dt) acc[q][dt] = float4_t{0, 0, 0, 0};
  // Online softmax with a lazily moved reference: weights are 2^(s - m_ref);
  // m_ref only moves (rescaling acc and l) when a row's max exceeds it by
  // more than 2^8, so weights stay <= 256 and the rescale is rare.
  float m_ref[NG], neg_m[NG], l_run[NG];   // neg_m = -m_ref once m_ref is finite
  const float* bias_row[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    m_ref[q] = -INFINITY;
    neg_m[q] = 0.0f;
    l_run[q] = 0.0f;
    // rows past n_q read the group's first existing row (see above)
    const int tb_row = row_ok[q] ? t[q] : fr[q];     // query index within the sequence
    if (BIAS != 1)
      bias_row[q] = nullptr;
    else if (a.bias_start)                           // ragged rows [H][n_q][L]
      bias_row[q] = a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L;
    else                                             // padded [B, H, MS, MS]
      bias_row[q] = a.attn_bias +
                    (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) * a.max_seq_len;
  }
  // A lane's 4 bias entries of a chunk (keys c0 + 4g .. + 3) are contiguous:
  // where the group sees the chunk whole they are read as one 16-byte load,
  // if every lane's row is 16-byte aligned (uniform per group)
  bool bias_vec[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q)
    bias_vec[q] = BIAS == 1 &&
                  __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(bias_row[q]) & 15) != 0) == 0;
  // whether every key of the 16-key chunk at c0 is visible to every existing
  // row of group q (uniform): no per-element mask is needed there
  auto chunk_whole = [&](int q, int c0) {
    bool whole = c0 + 16 <= L;
    if constexpr (CAUSAL) whole = whole && c0 + 15 <= gp0[q];
    if constexpr (BAND == 1)
      whole = whole && gp1[q] - c0 < a.window && c0 + 15 - gp0[q] < a.window;
    if constexpr (BAND == 2) whole = whole && c0 >= wlo[q] && c0 + 16 <= whi[q];
    return whole;
  };

  // ---- prologue: tile 0 into LDS buffer 0, tile 1 in flight, table of tile 2 ----
  if (ntiles > 0) {
    load_table(0);
    fetch(0);
    stash(0, 0);
    if (ntiles > 1) {
      load_table(1);
      fetch(1);
      if (ntiles > 2) load_table(2);
    }
  }
  __syncthreads();

  // one key tile; the LDS buffer is a compile-time constant so that every
  // LDS address is a per-lane base plus an immediate
  auto tile_step = [&](int tk, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int base = tile_base(tk);
    if (wave_active && base < wv_hi && base + kKTile > wv_lo) {
      const float* k_lds = kv_lds[buf][0];
      const float* v_lds = kv_lds[buf][1];

      // 16-key chunks that no row of the wave can see (window edges, causal
      // diagonal) skip both products: bit ch of `live` (uniform)
      int live = (1 << kChunks) - 1;
      if constexpr ((WINDOW || CAUSAL) && kChunks == 2) {
        live = 0;
#pragma unroll
        for (int ch = 0; ch < kChunks; ++ch) {
          const int c0 = base + ch * 16;
          live |= (c0 < wv_hi && c0 + 16 > wv_lo) ? 1 << ch : 0;
        }
      }
      // bias of the chunks seen whole, requested before the products
      float4_t bpre[NG][kChunks];
      if constexpr (BIAS == 1) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int ch = 0; ch < kChunks; ++ch) {
            const int c0 = base + ch * 16;
            bpre[q][ch] = float4_t{0, 0, 0, 0};
            if (bias_vec[q] && ((live >> ch) & 1) && chunk_whole(q, c0))
              bpre[q][ch] = *reinterpret_cast<const float4_t*>(bias_row[q] + c0 + 4 * g);
          }
      }
      // ---- S^T = K Q^T (base-2 scores); each K operand feeds every group ----
      float4_t s[NG][kChunks];
#pragma unroll
      for (int q = 0; q < NG; ++q)
#pragma unroll
        for (int ch = 0; ch < kChunks; ++ch) s[q][ch] = float4_t{0, 0, 0, 0};
      auto qk = [&](auto live_c) {
        constexpr int lv = decltype(live_c)::value;
#pragma unroll
        for (int i = 0; i < kDQ; i += 4) {
#pragma unroll
          for (int ch = 0; ch < kChunks; ++ch) {
            if (((lv >> ch) & 1) != 0) {   // folded once the loop is unrolled
              const float4_t kv = *reinterpret_cast<const float4_t*>(
                  &k_lds[(ch * 16 + c) * kRow + kDQ * g + i]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < NG; ++q)
                  s[q][ch] = mfma16x16x4(kv[e], qreg[q][i + e], s[q][ch]);
            }
          }
        }
      };
      if constexpr (kChunks == 2) {
        if (live == 3)
          qk(IntC<3>{});
        else if (live == 1)
          qk(IntC<1>{});
        else
          qk(IntC<2>{});
      } else {
        qk(IntC<(1 << kChunks) - 1>{});
      }

#pragma unroll
      for (int q = 0; q < NG; ++q) {
#pragma unroll
        for (int ch = 0; ch < kChunks; ++ch) {
          const int c0 = base + ch * 16;
          const int j0 = c0 + 4 * g;
          if (!((live >> ch) & 1)) {
            s[q][ch] = float4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            continue;
          }
          if constexpr (BIAS == 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s[q][ch][r] = s[q][ch][r] + rel_lds[min(max(j0 + r - p[q], -rel_md), rel_md) + rel_md];
          }
          // per-element mask only where some existing row of the group does
          // not see the whole chunk (sequence end, window edges, diagonal);
          // a materialised bias (added as a * scale * log2(e): the same sum as
          // (q.k + a) * scale) is read only for visible keys
          if (chunk_whole(q, c0)) {
            if constexpr (BIAS == 1) {
              if (bias_vec[q]) {
#pragma unroll
                for (int r = 0; r < 4; ++r) s[q][ch][r] = s[q][ch][r] + bpre[q][ch][r] * cs;
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  s[q][ch][r] = s[q][ch][r] + bias_row[q][j0 + r] * cs;
              }
            }
          } else {
            const int d0 = dq[q] - c0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int d = d0 - r;
              bool vis = d > dlo[q];
              if constexpr (BAND == 1) vis = vis && d < a.window;
              if constexpr (BAND == 2) vis = vis && d < dhi[q];
              if constexpr (BIAS == 1) {
                float x = -INFINITY;
                if (vis) x = s[q][ch][r] + bias_row[q][j0 + r] * cs;
                s[q][ch][r] = x;
              } else {
                s[q][ch][r] = vis ? s[q][ch][r] : -INFINITY;
              }
            }
          }
        }

        // ---- row max over the tile: 4 values per chunk, then lanes c + 16 g ----
        float mt = vmax(vmax(s[q][0][0], s[q][0][1]), vmax(s[q][0][2], s[q][0][3]));
#pragma unroll
        for (int ch = 1; ch < kChunks; ++ch)
          mt = vmax(mt, vmax(vmax(s[q][ch][0], s[q][ch][1]), vmax(s[q][ch][2], s[q][ch][3])));
        {
          const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt),
                                                            __float_as_uint(mt), false, false);
          mt = vmax(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
          const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                            __float_as_uint(mt), false, false);
          mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
        }
        const bool move = mt > m_ref[q] + 8.0f;        // false while mt = -inf
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          // rows that do not move keep alpha = 1 (their m_ref may still be
          // -inf: exp2(-inf - -inf) would be NaN); a first move from -inf
          // gives alpha = 0 on an empty accumulator
          const float alpha = move ? __builtin_amdgcn_exp2f(m_ref[q] - mt) : 1.0f;
          m_ref[q] = move ? mt : m_ref[q];
          neg_m[q] = move ? -mt : neg_m[q];
          l_run[q] *= alpha;
#pragma unroll
          for (int dt = 0; dt < kNDT; ++dt) acc[q][dt] *= alpha;
        }
#pragma unroll
        for (int ch = 0; ch < kChunks; ++ch) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[q][ch][r] + neg_m[q]);
            s[q][ch][r] = pr;
            l_run[q] += pr;
          }
        }
      }

      // ---- O^T += V^T P^T; each V operand feeds every group ----
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        if (!((live >> ch) & 1)) continue;      // all its weights are 0
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
          for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
            for (int q = 0; q < NG; ++q)
              acc[q][dt] = mfma16x16x4(vv[dt], s[q][ch][kk], acc[q][dt]);
        }
      }
    }
    // refill: tile tk+1 (in registers) -> the other buffer, tile tk+2 -> registers
    if (tk + 1 < ntiles) stash(buf ^ 1, tk + 1);
    if (tk + 2 < ntiles) {
      fetch(tk + 2);
      if (tk + 3 < ntiles) load_table(tk + 3);
    }
    __syncthreads();
  };
  for (int tk = 0; tk < ntiles; tk += 2) {
    tile_step(tk, IntC<0>{});
    if (tk + 1 < ntiles) tile_step(tk + 1, IntC<1>{});
  }

  // ---- epilogue: out = O / l ----
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    float l_tot = l_run[q];
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!row_ok[q]) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* orow = static_cast<float*>(a.out) + ((int64_t)(q0 + t[q]) * H + h) * D + kDQ * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int dt = 0; dt < kNDT; dt += 4) {
        float4_t o = {acc[q][dt][r] * inv, acc[q][dt + 1][r] * inv, acc[q][dt + 2][r] * inv,
                      acc[q][dt + 3][r] * inv};
        *reinterpret_cast<float4_t*>(orow + kNDT * r + dt) = o;
      }
    }
  }
}

template <int D, int NG, int BIAS, int BAND>
void launch_band(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.causal)
    hipLaunchKernelGGL((pa_prefill_f32<D, NG, BIAS, true, BAND>), grid, dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_f32<D, NG, BIAS, false, BAND>), grid, dim3(kThreads), 0,
                       stream, a);
}

template <int D, int NG, int BIAS>
void launch_mask(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.window > 0)
    launch_band<D, NG, BIAS, 1>(a, grid, stream);
  else if (a.chunk > 0)
    launch_band<D, NG, BIAS, 2>(a, grid, stream);
  else
    launch_band<D, NG, BIAS, 0>(a, grid, stream);
}

template <int D, int NG>
hipError_t launch_d(PrefillArgs a, hipStream_t stream) {
  constexpr int kQT = kWaves * 16 * NG;
  a.num_qtiles = (a.max_seq_len + kQT - 1) / kQT;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  const int64_t groups = (pairs + kXcds - 1) / kXcds;
  const int64_t nwg = groups * kXcds * a.num_qtiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  if (a.rel.table)
    launch_mask<D, NG, 2>(a, grid, stream);
  else if (a.attn_bias)
    launch_mask<D, NG, 1>(a, grid, stream);
  else
    launch_mask<D, NG, 0>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace

#ifndef PA_PREFILL_F32X3
#define PA_PREFILL_F32X3 1
#endif
#ifndef PA_PREFILL_F32X3_BAND
#define PA_PREFILL_F32X3_BAND 1
#endif

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  // launches at head_dim 64 run on the bf16 matrix cores with operands split
  // into three bf16 parts (pa_prefill_f32x3.hip); PA_PREFILL_F32X3_BAND = 0
  // keeps causal, windowed and chunked ones here
  const bool banded = a.causal || a.window > 0 || a.chunk > 0;
  if (PA_PREFILL_F32X3 && a.head_dim == 64 && (PA_PREFILL_F32X3_BAND || !banded))
    return launch_prefill_f32x3(a, stream);
  return a.head_dim == 64 ? launch_d<64, PA_PREFILL_GROUPS>(a, stream)
                          : launch_d<128, 1>(a, stream);
}

}  // namespace pa
