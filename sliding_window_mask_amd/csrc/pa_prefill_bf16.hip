// bf16 MFMA prefill attention over a paged KV cache for gfx950 (CDNA4).
//
// Same computation as the fp32 prefill (softmax((q K^T + A) * scale) V over
// the keys a row may see: bidirectional, causal, sliding window, optional
// bias), for bf16 q / K / V / out, on the bf16 MFMA instructions: bf16
// products accumulated in fp32. The softmax runs in fp32; the weights P are
// rounded to bf16 for the P.V contraction and the row sums are taken over the
// same rounded weights (one more MFMA against an all-ones operand, or
// v_dot2_f32_bf16 against (1, 1)), so out = sum(P~ V) / sum(P~) is an exact
// weighted mean.
//
// Scores stay unscaled (q.k + a) until the exponent, where the scale enters
// through one fma: p = 2^(x * scale * log2(e) - m). The running max is then
// taken on unscaled scores, which needs a positive multiplier: a negative
// scale is folded into q and the bias (both negated, multiplier |scale|), and
// a zero scale, under which every visible score is 0, into q = 0 with no bias
// and multiplier 1.
//
// Two kernels share this design. Bidirectional launches without a window,
// and causal ones without a window at head_dim 64, go to a 32-query-per-wave
// kernel on v_mfma_f32_32x32x16_bf16 (second half of this file); other causal
// launches and windowed ones to the kernel below.
//
// One workgroup per (64-query tile, head, sequence), numbered so that all
// query tiles of a (sequence, head) share an XCD, longest sequences first
// (launches without a window, batches of up to 63 sequences). Each wave owns kSub
// sub-tiles of 16 queries and multiplies every K and V operand it reads from
// LDS into all of them. The default is 4 waves x 1 sub-tile; 2 waves x 2
// sub-tiles (PA_PREFILL_BF16_SUB64=2, head_dim 64) halves the LDS reads per
// MFMA but needs ~130 VGPRs, and measured slower on the ModernBERT-shaped
// layers (3-4 waves per SIMD instead of 5). Keys are walked in 32-key tiles through a
// double-buffered LDS ring (tile k+2 in flight from memory while tile k is
// multiplied, block-table entries one tile further ahead).
//
// Operand layout (16x16x32, lane l, g = l / 16, c = l % 16; every lane feeds
// 8 bf16 of A and B, and lanes of one group g contract the same 8 positions):
// * S^T = K Q^T, step st of D/32: lane l feeds K[key c][(D/4) g + 8 st + e]
//   and Q[query c][same dim] (e = 0..7) -- 16 contiguous bytes each. Lane l
//   ends holding S^T[key 4g + r][query c], r = 0..3, for each 16-key chunk.
// * O^T = V^T P^T over the tile's 32 keys: element e of lane group g is key
//   4g + e (e < 4, first chunk) or 16 + 4g + e - 4 (second chunk), so the
//   P operand is exactly the lane's own 8 softmax weights. The V operand
//   needs 8 keys of one dim, a column of the row-major V tile: gfx950's
//   transposing LDS read (ds_read_b64_tr_b16) provides it. Within each group
//   of 16 lanes it treats the 16 8-byte pieces the lanes point at as a 16x4
//   matrix M of 16-bit values and returns M[a][e], M[a+4][e], M[a+8][e],
//   M[a+12][e] to lane 4a + e. Lane j of group g therefore points at key
//   4g + j/4, dims 16 dt + 4 (j%4) .. +3, and receives keys 4g .. 4g+3 of dim
//   16 dt + j; a second read 16 rows further gives keys 16 + 4g .. 16 + 4g + 3.
//   V rows are padded to D + 16 bf16, so the 16 rows one read touches fall in
//   distinct bank windows (the 2-cycle minimum for 512 bytes). Lane l ends
//   holding O^T[dim 16 dt + 4g + r][query c].
#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

#ifndef PA_PREFILL_BF16_SUB64
#define PA_PREFILL_BF16_SUB64 1     // 16-query sub-tiles per wave, head_dim 64
#endif

constexpr int kQT = 64;         // queries per workgroup
constexpr int kKT = 32;         // keys per tile (one 32-deep P.V contraction)
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct Cfg {
  static constexpr int kSub = D == 64 ? PA_PREFILL_BF16_SUB64 : 1;
  static constexpr int kWaves = kQT / (16 * kSub);
  static constexpr int kThreads = 64 * kWaves;
};

__device__ __forceinline__ float4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                              float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// BIAS: 0 none, 1 materialised (padded or ragged) fp32 bias, 2 T5 relative
// position bias from a bucket table.
template <int D, int BIAS, bool CAUSAL, bool WINDOW>
__global__ void __launch_bounds__(Cfg<D>::kThreads)
pa_prefill_bf16(PrefillArgs a) {
  constexpr int kSub = Cfg<D>::kSub;
  constexpr int kThreads = Cfg<D>::kThreads;
  constexpr int kKRow = D + 8;                 // K row stride in LDS (bf16)
  constexpr int kSteps = D / 32;               // 8-element steps per lane group
  constexpr int kNDT = D / 16;                 // 16-dim output slices
  constexpr int kKLoads = kKT * D / 8 / kThreads;        // 16-byte K loads per thread
  constexpr int kVRow = D + 16;                // V row stride in LDS (bf16)
  static_assert(kKLoads >= 1, "tile shape");
  static_assert(D == 64 || D == 128, "head_dim");

  const int H = a.num_heads;
  int b, h, tile, L, q0, nq;
  if (!prefill_work_of(blockIdx.x, a, b, h, tile, L, q0, nq)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int c = lane & 15;
  const int g = lane >> 4;

  const int t_first = tile * kQT;
  if (t_first >= nq) return;
  const int pos0 = L - nq;

  const int wg_last = min(t_first + kQT, nq) - 1;
  int wg_lo, wg_hi;
  prefill_key_range(pos0 + t_first, pos0 + wg_last, L, a.window, a.chunk, CAUSAL, wg_lo,
                    wg_hi);
  const int w_first = t_first + wave * 16 * kSub;
  const bool wave_active = w_first < nq;
  int wv_lo = 0, wv_hi = 0;
  if (wave_active)
    prefill_key_range(pos0 + w_first, pos0 + min(w_first + 16 * kSub, nq) - 1, L, a.window,
                      a.chunk, CAUSAL, wv_lo, wv_hi);

  // exponent multiplier (> 0) and the sign the unscaled scores carry
  const float cs = a.scale_log2 == 0.0f ? 1.0f : fabsf(a.scale_log2);
  const float bmul = a.scale_log2 == 0.0f ? 0.0f : (a.scale_log2 < 0.0f ? -1.0f : 1.0f);

  // per sub-tile: query row of lane c, its position, whether it exists; the
  // sub-tile's first / last existing position (uniform). Masking of partly
  // visible chunks: with d = p - j for key j = c0 + 4g + r, d = dq - c0 - r,
  // and the key is visible iff dlo < d (j < L, causal j <= p, window
  // p - j > -W, chunk start) and, with a window or chunks, d < dhi (window
  // W, or the end of p's chunk). Keys [wlo, whi) are inside the window or
  // chunk of every row of the sub-tile.
  // Rows past n_q see no key at all (their dlo is the largest int), and where
  // a chunk is seen whole by the sub-tile they read the bias row of its first
  // existing query (fr): the bias entries of keys a row cannot see are never
  // read. A sub-tile with no existing row (possible only with kSub > 1) takes
  // the workgroup's last query as its only row.
  int t_row[kSub], p_row[kSub], sp0[kSub], sp1[kSub], fr[kSub], dq[kSub], dlo[kSub], dhi[kSub];
  int wlo[kSub], whi[kSub];
  bool row_ok[kSub];
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb) {
    const int f = w_first + 16 * sb;
    fr[sb] = min(f, nq - 1);
    t_row[sb] = f + c;
    row_ok[sb] = t_row[sb] < nq;
    p_row[sb] = pos0 + t_row[sb];
    sp0[sb] = pos0 + fr[sb];
    sp1[sb] = pos0 + max(min(f + 15, nq - 1), fr[sb]);
    dq[sb] = p_row[sb] - 4 * g;
    if constexpr (WINDOW) {
      prefill_row_bounds(p_row[sb], L, a.window, a.chunk, CAUSAL, dlo[sb], dhi[sb]);
      prefill_common_keys(sp0[sb], sp1[sb], a.window, a.chunk, wlo[sb], whi[sb]);
    } else {
      dlo[sb] = CAUSAL ? max(p_row[sb] - L, -1) : p_row[sb] - L;
      dhi[sb] = wlo[sb] = whi[sb] = 0;
    }
    if (!row_ok[sb]) dlo[sb] = 0x7fffffff;
  }
  // the keys [bjlo, bjhi] a row sees (empty for rows past n_q): partly seen
  // chunks read their bias entries with the key clamped into this range, so
  // that they can be requested with the whole chunks, before the products,
  // and still read only visible entries
  int bjlo[kSub], bjhi[kSub];
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb) {
    bjlo[sb] = 0;
    bjhi[sb] = -1;
    if (BIAS == 1 && row_ok[sb]) {
      bjhi[sb] = p_row[sb] - dlo[sb] - 1;
      if constexpr (WINDOW) bjlo[sb] = max(p_row[sb] - dhi[sb] + 1, 0);
    }
  }

  // Q operands: kSteps x 8 bf16 per sub-tile (rows past n_q, and every row
  // under a zero scale, are zero; a negative scale flips the sign bits)
  bf16x8_t qv[kSub][kSteps];
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb) {
    const int tq = row_ok[sb] ? t_row[sb] : t_first;
    const bool qzero = !row_ok[sb] || bmul == 0.0f;
    const uint32_t qsign = bmul < 0.0f ? 0x80008000u : 0u;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + (D / 4) * g);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      uint4 v = qrow[st];
      v = qzero ? make_uint4(0u, 0u, 0u, 0u)
                : make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      qv[sb][st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  __shared__ uint16_t k_lds[2][kKT * kKRow];   // K tile, row-major [key][dim]
  __shared__ uint16_t v_lds[2][kKT * kVRow];   // V tile, row-major [key][dim]
  // T5 bias of relative position r = j - p at rel_lds[r + md + 3] for r in
  // [-md - 3, md + 3]; distances past md repeat the end buckets, so a lane's
  // four consecutive keys clamp their first distance once and read four
  // neighbouring entries
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 7 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md + 6; i += kThreads)
      rel_lds[i] = bmul == 0.0f ? 0.0f
                                : rel_bias(min(max(i - 3 - rel_md, -rel_md), rel_md), a.rel,
                                           head_row) * bmul;
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
  // global -> registers: K and V as 16-byte row pieces (8 dims of one key).
  // A cache block holds 2D pieces, a multiple of 64, so each wave's pieces of
  // one load lie in one block: the address is a uniform block base plus a
  // per-lane offset that is the same for every tile. Rows at or past L are
  // read from the sequence's last block, or from block 0 for a block past it
  // (both in the pool): K there only feeds scores the mask drops, and V is
  // zeroed so that a zero weight never meets a NaN.
  // (vectors rather than arrays, so that they stay in registers)
  typedef uint32_t st_t __attribute__((ext_vector_type(4 * kKLoads)));
  st_t kst, vst;
  auto fetch = [&](int tk) {
    const int base = kstart + tk * kKT;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;        // 16-byte piece index in the tile
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      const int sel = (i * kThreads + wave * 64) / (D / 8) / kBlockSize;
      const int64_t blk = ((int64_t)tb[sel] * H + h) * (kBlockSize * D);
      const uint32_t off = (uint32_t)((r % kBlockSize) * D + col);
      const uint4 kv = *reinterpret_cast<const uint4*>(kc + blk + off);
      const uint4 vv = *reinterpret_cast<const uint4*>(vc + blk + off);
      kst[4 * i] = kv.x;
      kst[4 * i + 1] = kv.y;
      kst[4 * i + 2] = kv.z;
      kst[4 * i + 3] = kv.w;
      vst[4 * i] = vv.x;
      vst[4 * i + 1] = vv.y;
      vst[4 * i + 2] = vv.z;
      vst[4 * i + 3] = vv.w;
    }
    if (base + kKT > L) {   // uniform: only a sequence's last tile
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {
        const int r = (i * kThreads + tid) / (D / 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) vst[4 * i + w] = base + r < L ? vst[4 * i + w] : 0u;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][r * kKRow + col]) =
          make_uint4(kst[4 * i], kst[4 * i + 1], kst[4 * i + 2], kst[4 * i + 3]);
      *reinterpret_cast<uint4*>(&v_lds[buf][r * kVRow + col]) =
          make_uint4(vst[4 * i], vst[4 * i + 1], vst[4 * i + 2], vst[4 * i + 3]);
    }
  };

  float4_t acc[kSub][kNDT];
  // row sums: lacc[sb][r] = sum of the rounded weights of query c (every r)
  float4_t lacc[kSub];
  float m_ref[kSub], neg_m[kSub];   // running reference (base 2), and -m_ref once finite
  const float* bias_row[kSub];
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb) {
#pragma unroll
    for (int dt = 0; dt < kNDT; ++dt) acc[sb][dt] = float4_t{0, 0, 0, 0};
    lacc[sb] = float4_t{0, 0, 0, 0};
    m_ref[sb] = -INFINITY;
    neg_m[sb] = 0.0f;
    bias_row[sb] = nullptr;
    if (BIAS == 1) {
      const int tb_row = row_ok[sb] ? t_row[sb] : fr[sb];
      bias_row[sb] = a.bias_start
                         ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                         : a.attn_bias + (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) *
                                             a.max_seq_len;
    }
  }
  // A lane's 4 bias entries of a chunk (keys c0 + 4g .. + 3) are contiguous:
  // where the sub-tile sees the chunk whole they are read as one 16-byte
  // load, if every lane's row is 16-byte aligned (uniform per sub-tile)
  bool bias_vec[kSub];
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb)
    bias_vec[sb] = BIAS == 1 &&
                   __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(bias_row[sb]) & 15) != 0) == 0;
  // whether every key of the 16-key chunk at c0 is visible to every existing
  // row of sub-tile sb (uniform): no per-element mask is needed there
  auto chunk_whole = [&](int sb, int c0) {
    bool whole = c0 + 16 <= L;
    if constexpr (CAUSAL) whole = whole && c0 + 15 <= sp0[sb];
    if constexpr (WINDOW) whole = whole && c0 >= wlo[sb] && c0 + 16 <= whi[sb];
    return whole;
  };
  bf16x8_t ones = __builtin_bit_cast(
      bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

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

  // one key tile; the LDS buffer is a compile-time constant so that every
  // LDS address is a per-lane base plus an immediate
  auto tile_step = [&](int tk, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    asm("" : "+v"(ones));   // keep the all-ones operand resident, not rebuilt per tile
    const int base = kstart + tk * kKT;
    if (wave_active && base < wv_hi && base + kKT > wv_lo) {
      // 16-key chunks that no row of the wave can see (window edges, causal
      // diagonal) skip their S^T products: bit ch of `live` (uniform)
      int live = 3;
      if constexpr (WINDOW || CAUSAL) {
        live = 0;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int c0 = base + ch * 16;
          live |= (c0 < wv_hi && c0 + 16 > wv_lo) ? 1 << ch : 0;
        }
      }
      // bias of the tile's live chunks, requested before the products:
      // chunks seen whole in one 16-byte load when the rows are aligned,
      // otherwise entry by entry with the key clamped into the row's range
      float4_t bpre[kSub][2];
      if constexpr (BIAS == 1) {
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const int c0 = base + ch * 16;
            const int j0 = c0 + 4 * g;
            bpre[sb][ch] = float4_t{0, 0, 0, 0};
            if ((live >> ch) & 1) {
              if (bias_vec[sb] && chunk_whole(sb, c0)) {
                bpre[sb][ch] = *reinterpret_cast<const float4_t*>(bias_row[sb] + j0);
              } else if (bjlo[sb] <= bjhi[sb]) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  bpre[sb][ch][r] = bias_row[sb][min(max(j0 + r, bjlo[sb]), bjhi[sb])];
              }
            }
          }
      }
      // ---- S^T for the two 16-key chunks of every sub-tile ----
      float4_t s[kSub][2];
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) s[sb][0] = s[sb][1] = float4_t{0, 0, 0, 0};
      auto qk = [&](auto live_c) {
        constexpr int lv = decltype(live_c)::value;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            if (((lv >> ch) & 1) != 0) {   // folded once the loop is unrolled
              const uint4 kv = *reinterpret_cast<const uint4*>(
                  &k_lds[buf][(ch * 16 + c) * kKRow + (D / 4) * g + 8 * st]);
#pragma unroll
              for (int sb = 0; sb < kSub; ++sb)
                s[sb][ch] = mfma_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[sb][st], s[sb][ch]);
            }
          }
        }
      };
      if (live == 3)
        qk(IntC<3>{});
      else if (live == 1)
        qk(IntC<1>{});
      else
        qk(IntC<2>{});
      // V^T operands of this tile (read after the softmax: reading them before
      // it measured slower)
      uint4 vv[kNDT];
      auto read_v = [&]() {
        // lane j of group g points at key 4g + j/4, dims 16dt + 4(j%4) .. +3;
        // the transposing read hands lane j keys 4g .. 4g+3 of dim 16dt + j
        // (and, 16 rows further, keys 16 + 4g .. 16 + 4g + 3)
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) {
          const uint16_t* p = &v_lds[buf][(4 * g + (c >> 2)) * kVRow + 16 * dt + 4 * (c & 3)];
          const uint2 lo = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 16 * kVRow)));
          vv[dt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      };
      bf16x8_t pw[kSub];
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) {
        // ---- bias and mask (unscaled scores) ----
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int c0 = base + ch * 16;
          const int j0 = c0 + 4 * g;
          if (!((live >> ch) & 1)) {
            s[sb][ch] = float4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            continue;
          }
          if constexpr (BIAS == 2) {
            const int e0 = min(max(j0 - p_row[sb], -rel_md - 3), rel_md) + rel_md + 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[sb][ch][r] += rel_lds[e0 + r];
          }
          // per-element mask only where some existing row of the sub-tile
          // does not see the whole chunk; a materialised bias is read only
          // for visible keys
          if (chunk_whole(sb, c0)) {
            if constexpr (BIAS == 1) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                s[sb][ch][r] = fmaf(bpre[sb][ch][r], bmul, s[sb][ch][r]);
            }
          } else {
            const int d0 = dq[sb] - c0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int d = d0 - r;
              bool vis = d > dlo[sb];
              if constexpr (WINDOW) vis = vis && d < dhi[sb];
              if constexpr (BIAS == 1) {
                s[sb][ch][r] = vis ? fmaf(bpre[sb][ch][r], bmul, s[sb][ch][r]) : -INFINITY;
              } else {
                s[sb][ch][r] = vis ? s[sb][ch][r] : -INFINITY;
              }
            }
          }
        }
        // ---- online softmax with a lazily moved reference (as in fp32), in
        // base-2 units: m_ref is a scaled score ----
        float mt = vmax(vmax(vmax(s[sb][0][0], s[sb][0][1]), vmax(s[sb][0][2], s[sb][0][3])),
                        vmax(vmax(s[sb][1][0], s[sb][1][1]), vmax(s[sb][1][2], s[sb][1][3])));
        {
          const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt),
                                                            __float_as_uint(mt), false, false);
          mt = vmax(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
          const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                            __float_as_uint(mt), false, false);
          mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1])) * cs;
        }
        const bool move = mt > m_ref[sb] + 8.0f;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float alpha = move ? __builtin_amdgcn_exp2f(m_ref[sb] - mt) : 1.0f;
          m_ref[sb] = move ? mt : m_ref[sb];
          neg_m[sb] = move ? -mt : neg_m[sb];
          lacc[sb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < kNDT; ++dt) acc[sb][dt] *= alpha;
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pw[sb][4 * ch + r] =
                (__bf16)__builtin_amdgcn_exp2f(fmaf(s[sb][ch][r], cs, neg_m[sb]));
        }
      }
      read_v();
      // ---- O^T += V^T P^T over the tile's 32 keys, row sums alongside ----
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb) lacc[sb] = mfma_bf16(ones, pw[sb], lacc[sb]);
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb)
          acc[sb][dt] = mfma_bf16(__builtin_bit_cast(bf16x8_t, vv[dt]), pw[sb], acc[sb][dt]);
      }
    }
    if (tk + 1 < ntiles) stash(buf ^ 1);
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

  // ---- epilogue: out = O / l, rounded to bf16 ----
#pragma unroll
  for (int sb = 0; sb < kSub; ++sb) {
    if (!row_ok[sb]) continue;
    const float l_tot = lacc[sb][0];
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + t_row[sb]) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < kNDT; ++dt) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t o = {(__bf16)(acc[sb][dt][0] * inv), (__bf16)(acc[sb][dt][1] * inv),
                    (__bf16)(acc[sb][dt][2] * inv), (__bf16)(acc[sb][dt][3] * inv)};
      *reinterpret_cast<bf16x4_t*>(orow + 16 * dt + 4 * g) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Bidirectional launches without a window: every query of a sequence sees
// all of its keys, so a workgroup's key range is the whole sequence and the
// matrix work per staged K/V tile is the largest. This kernel takes 32
// queries per wave on v_mfma_f32_32x32x16_bf16 (half the MFMA and LDS-read
// instructions per flop of the 16x16x32 shape, and a quarter fewer LDS reads
// per score) and 128 queries per workgroup (each staged tile feeds twice as
// many queries). Measured on ModernBERT-shaped layers it is 6-9% faster than
// the kernel above for these launches, and slower for windowed ones (a longer
// band per workgroup, fewer resident waves), which stay on the kernel above.
// With CAUSAL (head_dim 64) it also takes causal launches without a window:
// the workgroup stages keys up to its last row, each wave stops after the
// tile holding its own last row and masks only the tiles crossing its
// diagonal; a materialised bias is read by the coalesced walk below only on
// tiles every row of the wave sees whole, and per entry, clamped to the row's
// own diagonal, on the others. A ModernBERT-shaped causal layer runs 8-12%
// faster than on the kernel above, with no bias, a T5 bias or a materialised
// one.
//
// Operand layout (32x32x16, lane l, j = l % 32, hh = l / 32; A[i][k] comes
// from lane i + 32 (k/8) element k%8, B[k][j] from lane j + 32 (k/8) element
// k%8, and D[i][j] lands in lane j + 32 ((i/4)%2), register 4 (i/8) + i%4):
// * S^T = K Q^T over 16-dim steps: lane l feeds K[key j][16 st + 8 hh + e]
//   and Q[query j][same dims] (16 contiguous bytes each) and ends holding
//   S^T[key 8u + 4hh + r][query j] in register 4u + r (u, r = 0..3): 16 scores
//   of one query, the other 16 in lane l ^ 32.
// * O^T = V^T P^T over 16-key steps ks: element e of the lane's B operand is
//   key 16 ks + 8 (e/4) + 4 hh + e%4, so the P operand is the lane's own
//   registers 8 ks .. 8 ks + 7. The V^T operand comes from the transposing LDS
//   read: lane jj = l % 16 of 16-lane group G points at key 16 ks + 4 hh +
//   jj/4, dims 32 dt + 16 (G%2) + 4 (jj%4) .. +3, and receives keys +0..3 of
//   dim 32 dt + j; a second read 8 rows further supplies the other 4 keys.
//   V rows are padded to D + 32 bf16, so the 4 rows each half-wave touches
//   start 16 banks apart.
// * Row sums: each lane adds its 16 rounded weights with v_dot2_f32_bf16
//   against (1, 1) (exact products, fp32 sums); the two halves of a query
//   are added once, at the end. out = sum(P~ V) / sum(P~) as above.
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kQT32 = 128;                    // queries per workgroup
constexpr int kThreads32 = 64 * (kQT32 / 32);  // one wave per 32 queries

__device__ __forceinline__ float16_t mfma32_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                 float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Bias-free launches at head_dim 64 (the encoder workload's full-attention
// layers) are held to 96 VGPRs, 5 waves per SIMD instead of 4, with no spill:
// 3.8% faster on the ModernBERT-shaped layers. The bias variants would spill
// at that bound and keep the default.
template <int D, int BIAS>
constexpr int min_waves32() { return D == 64 && BIAS == 0 ? 5 : 1; }

template <int D, int BIAS, bool CAUSAL>
__global__ void __launch_bounds__(kThreads32, (min_waves32<D, BIAS>()))
pa_prefill_bf16_32(PrefillArgs a) {
  constexpr int kThreads = kThreads32;
  constexpr int kKRow = D + 8;                 // K row stride in LDS (bf16)
  constexpr int kVRow = D + 32;                // V row stride in LDS (bf16)
  constexpr int kSteps = D / 16;               // 16-dim steps of S^T
  constexpr int kNDT = D / 32;                 // 32-dim output slices
  constexpr int kKLoads = kKT * D / 8 / kThreads;        // 16-byte K loads per thread
  static_assert(kKLoads >= 1, "tile shape");
  static_assert(D == 64 || D == 128, "head_dim");

  const int H = a.num_heads;
  int b, h, tile, L, q0, nq;
  if (!prefill_work_of(blockIdx.x, a, b, h, tile, L, q0, nq)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int j = lane & 31;
  const int hh = lane >> 5;
  const int jj = lane & 15;
  const int g1 = (lane >> 4) & 1;

  const int t_first = tile * kQT32;
  if (t_first >= nq) return;
  const int pos0 = L - nq;
  const int w_first = t_first + wave * 32;
  const bool wave_active = w_first < nq;   // uniform over the wave

  const float cs = a.scale_log2 == 0.0f ? 1.0f : fabsf(a.scale_log2);
  const float bmul = a.scale_log2 == 0.0f ? 0.0f : (a.scale_log2 < 0.0f ? -1.0f : 1.0f);

  // the lane's query row and its position; keys j >= L of the last tile are
  // masked: with d = p - j for key j = c0 + 8u + 4hh + r, d = dq - c0 - 8u - r
  // and j < L iff d > p - L
  const int t_row = w_first + j;
  const bool row_ok = t_row < nq;
  const int p_row = pos0 + t_row;
  const int dq = p_row - 4 * hh;
  const int dlo = p_row - L;
  // causal: the wave's rows sit at positions pw0 .. pw0 + 31 and see keys
  // j <= p (all of them inside the sequence); the workgroup stages keys up to
  // its last row, and a wave skips the tiles past its own last row
  const int pw0 = pos0 + w_first;

  bf16x8_t qv[kSteps];
  {
    const int tq = row_ok ? t_row : t_first;
    const bool qzero = !row_ok || bmul == 0.0f;
    const uint32_t qsign = bmul < 0.0f ? 0x80008000u : 0u;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + 8 * hh);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      uint4 v = qrow[2 * st];
      v = qzero ? make_uint4(0u, 0u, 0u, 0u)
                : make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      qv[st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kKT * kVRow];
  // T5 bias of relative position r = j - p at rel_lds[r + md + 3] for r in
  // [-md - 3, md + 3]; distances past md repeat the end buckets, so a lane's
  // four consecutive keys clamp their first distance once and read four
  // neighbouring entries
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 7 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md + 6; i += kThreads)
      rel_lds[i] = bmul == 0.0f ? 0.0f
                                : rel_bias(min(max(i - 3 - rel_md, -rel_md), rel_md), a.rel,
                                           head_row) * bmul;
  }

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int kend = CAUSAL ? min(L, pos0 + t_first + kQT32) : L;
  const int ntiles = (kend + kKT - 1) / kKT;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;

  // staging as in the kernel above: each wave's 16-byte pieces of one load
  // lie in one cache block; rows at or past L come from an in-pool block,
  // and V there is zeroed
  int tb[2];
  auto load_table = [&](int tk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = tk * (kKT / kBlockSize) + i;
      tb[i] = blk < nblk_seq ? table[blk] : 0;
    }
  };
  typedef uint32_t st_t __attribute__((ext_vector_type(4 * kKLoads)));
  st_t kst, vst;
  auto fetch = [&](int tk) {
    const int base = tk * kKT;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      const int sel = (i * kThreads + wave * 64) / (D / 8) / kBlockSize;
      const int64_t blk = ((int64_t)tb[sel] * H + h) * (kBlockSize * D);
      const uint32_t off = (uint32_t)((r % kBlockSize) * D + col);
      const uint4 kv = *reinterpret_cast<const uint4*>(kc + blk + off);
      const uint4 vv = *reinterpret_cast<const uint4*>(vc + blk + off);
      kst[4 * i] = kv.x;
      kst[4 * i + 1] = kv.y;
      kst[4 * i + 2] = kv.z;
      kst[4 * i + 3] = kv.w;
      vst[4 * i] = vv.x;
      vst[4 * i + 1] = vv.y;
      vst[4 * i + 2] = vv.z;
      vst[4 * i + 3] = vv.w;
    }
    if (base + kKT > L) {   // uniform: only the sequence's last tile
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {
        const int r = (i * kThreads + tid) / (D / 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) vst[4 * i + w] = base + r < L ? vst[4 * i + w] : 0u;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][r * kKRow + col]) =
          make_uint4(kst[4 * i], kst[4 * i + 1], kst[4 * i + 2], kst[4 * i + 3]);
      *reinterpret_cast<uint4*>(&v_lds[buf][r * kVRow + col]) =
          make_uint4(vst[4 * i], vst[4 * i + 1], vst[4 * i + 2], vst[4 * i + 3]);
    }
  };

  float16_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  float lsum = 0.0f;                      // this lane's half of the row sum
  float m_ref = -INFINITY, neg_m = 0.0f;  // running reference (base 2), -m_ref once finite
  const float* bias_row = nullptr;
  // causal: a row reads entries of keys j <= p_bias only (rows past the
  // query set read the last query's row, which sees every key below L)
  const int p_bias = row_ok ? p_row : L - 1;
  if (BIAS == 1) {
    const int tb_row = row_ok ? t_row : (CAUSAL ? nq - 1 : t_first);
    bias_row = a.bias_start
                   ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                   : a.attn_bias +
                         (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) * a.max_seq_len;
  }
  // a lane's bias entries of a tile are 4 runs of 4 contiguous keys: 16-byte
  // loads on tiles that lie wholly inside the sequence, if every lane's row
  // is 16-byte aligned (uniform)
  const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  // Bias entries of tiles lying wholly inside the sequence (causal: and
  // wholly at or before the wave's first row, so that every row of the wave
  // sees every key of the tile) are read with whole 128-byte row segments
  // per 8 lanes: load q of a tile takes rows lane/8 + 8q of the wave's 32 (a
  // row past the last query repeats the last query's row), 16 bytes per
  // lane, one tile ahead, as non-temporal loads (each entry is read once,
  // and whole lines at a time); the wave then passes them through its own
  // LDS block (rows padded to 36 floats, so the reads of 16 lanes cover all
  // banks once) to the lanes that own the rows. Reading a lane's own 4 runs
  // of 4 entries directly would touch 32 rows in every load instruction, 32
  // bytes each. The block is the wave's alone and its LDS operations
  // complete in order, so no barrier is involved.
  constexpr int kBRow = 36;
  __shared__ __attribute__((aligned(16))) float b_lds[BIAS == 1 ? (kQT32 / 32) * 32 * kBRow : 4];
  float* bw = &b_lds[BIAS == 1 ? wave * 32 * kBRow : 0];
  const float* bbase = nullptr;   // the bias row of the wave's first query
  int boff[4] = {0, 0, 0, 0};     // element offsets of the lane's 4 load rows
  bool bias_vec = false;          // uniform: every row 16-byte aligned
  if (BIAS == 1 && wave_active) {
    const int64_t pitch = a.bias_start ? L : a.max_seq_len;
    bbase = a.bias_start
                ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + w_first) * L
                : a.attn_bias +
                      (((int64_t)b * H + h) * a.max_seq_len + pos0 + w_first) * a.max_seq_len;
    // (32-bit row offsets: rows of up to 2^26 entries)
    bias_vec = (reinterpret_cast<uintptr_t>(bbase) & 15) == 0 && (pitch & 3) == 0 &&
               pitch < (1 << 26);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = min(w_first + (lane >> 3) + 8 * q, nq - 1) - w_first;
      boff[q] = (int)(rr * pitch) + 4 * (lane & 7);
    }
  }
  float4_t bnext[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bnext[q] = float4_t{0, 0, 0, 0};
  if (BIAS == 1 && bias_vec && kKT <= L && (!CAUSAL || kKT - 1 <= pw0)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bnext[q] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(bbase + boff[q]));
  }

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

  auto tile_step = [&](int tk, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int c0 = tk * kKT;
    if (wave_active && (!CAUSAL || c0 <= pw0 + 31)) {
      const bool bias_whole = bias_vec && c0 + kKT <= L && (!CAUSAL || c0 + kKT - 1 <= pw0);
      // ---- S^T for the tile's 32 keys ----
      float16_t s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const uint4 kv =
            *reinterpret_cast<const uint4*>(&k_lds[buf][j * kKRow + 16 * st + 8 * hh]);
        s = mfma32_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[st], s);
      }
      // ---- bias (unscaled scores) and the tail mask. Every row of these
      // launches sees all L keys, so every bias entry read is a visible one
      // (keys past L of the last tile re-read entry L - 1, then are masked) ----
      if constexpr (BIAS == 1) {
        if (bias_whole) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4_t*>(&bw[((lane >> 3) + 8 * q) * kBRow + 4 * (lane & 7)]) =
                bnext[q];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float4_t bv =
                *reinterpret_cast<const float4_t*>(&bw[j * kBRow + 8 * u + 4 * hh]);
#pragma unroll
            for (int r = 0; r < 4; ++r) s[4 * u + r] = fmaf(bv[r], bmul, s[4 * u + r]);
          }
          // the next tile's entries, a whole tile of work ahead of their use
          if (c0 + 2 * kKT <= L && (!CAUSAL || c0 + 2 * kKT - 1 <= pw0)) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              bnext[q] = __builtin_nontemporal_load(
                  reinterpret_cast<const float4_t*>(bbase + boff[q] + c0 + kKT));
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s[4 * u + r] =
                  fmaf(bias_row[min(c0 + 8 * u + 4 * hh + r, CAUSAL ? p_bias : L - 1)], bmul,
                       s[4 * u + r]);
        }
      }
      if constexpr (BIAS == 2) {
        // the tile's relative positions j - p run from c0 - pw0 - 31 to
        // c0 + 31 - pw0; all at or beyond the maximum distance on one side
        // (uniform), they share that side's end bucket (at head_dim 64: at
        // 128 the branch would cost a resident wave)
        if (D == 64 && (c0 + kKT - 1 - pw0 <= -rel_md || c0 - pw0 - 31 >= rel_md)) {
          const float bend = rel_lds[c0 < pw0 ? 3 : 2 * rel_md + 3];
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] += bend;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e0 = min(max(c0 + 8 * u + 4 * hh - p_row, -rel_md - 3), rel_md) + rel_md + 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[4 * u + r] += rel_lds[e0 + r];
          }
        }
      }
      if constexpr (CAUSAL) {
        if (c0 + kKT - 1 > pw0) {   // uniform: tiles crossing the wave's diagonal
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s[4 * u + r] = dq - c0 - 8 * u - r >= 0 ? s[4 * u + r] : -INFINITY;
        }
      } else if (c0 + kKT > L) {   // uniform: only the last tile
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[4 * u + r] = dq - c0 - 8 * u - r > dlo ? s[4 * u + r] : -INFINITY;
      }
      // ---- online softmax, lazily moved reference (base-2 units) ----
      float mt = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = vmax(mt, s[i]);
      {
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1])) * cs;
      }
      const bool move = mt > m_ref + 8.0f;   // the same in lanes l and l ^ 32
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;
        m_ref = move ? mt : m_ref;
        neg_m = move ? -mt : neg_m;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;
      }
      bf16x8_t pw[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pw[ks][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 * ks + e], cs, neg_m));
        const uint4 pu = __builtin_bit_cast(uint4, pw[ks]);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.x), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.y), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.z), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.w), one2, lsum,
                                               false);
      }
      // ---- O^T += V^T P^T over the tile's two 16-key steps ----
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) {
          const uint16_t* p = &v_lds[buf][(16 * ks + 4 * hh + (jj >> 2)) * kVRow + 32 * dt +
                                          16 * g1 + 4 * (jj & 3)];
          const uint2 lo = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * kVRow)));
          acc[dt] = mfma32_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                pw[ks], acc[dt]);
        }
      }
    }
    if (tk + 1 < ntiles) stash(buf ^ 1);
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

  // ---- epilogue: out = O / l, rounded to bf16 (the swap runs in every lane) ----
  const auto xl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                   false, false);
  const float l_tot = __uint_as_float(xl[0]) + __uint_as_float(xl[1]);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + t_row) * H + h) * D;
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t o = {(__bf16)(acc[dt][4 * u] * inv), (__bf16)(acc[dt][4 * u + 1] * inv),
                    (__bf16)(acc[dt][4 * u + 2] * inv), (__bf16)(acc[dt][4 * u + 3] * inv)};
      *reinterpret_cast<bf16x4_t*>(orow + 32 * dt + 8 * u + 4 * hh) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// The same launches at head_dim 64, software-pipelined. Each wave's tile
// work is a chain (S^T products, then the softmax, then the P.V products),
// and in the kernel above the matrix cores sit idle while a wave computes its
// weights unless another resident wave happens to be multiplying. Here each
// step issues the S^T products of the next tile right after the current
// tile's row maximum, so they run on the matrix cores while the same wave
// computes the current weights; then the P.V products of the current tile.
// K of a tile is therefore staged two steps before its P.V step and V one
// step before, still with one barrier per step: entering step k, S_k is in
// registers, K of tile k+1 and V of tile k are in LDS, and the loads of K of
// tile k+2 and V of tile k+1 are in flight; step k stores those into the K
// buffer that tile k left and the V buffer that tile k-1 left, then issues
// the loads of V of tile k+2 and K of tile k+3. Operand layouts, softmax and
// rounding are those of the kernel above, so the two give identical results.
#ifndef PA_PREFILL_BF16_PIPE
#define PA_PREFILL_BF16_PIPE 0
#endif

template <int D, int BIAS>
__global__ void __launch_bounds__(kThreads32, 4)
pa_prefill_bf16_32p(PrefillArgs a) {
  constexpr int kThreads = kThreads32;
  constexpr int kKRow = D + 8;                 // K row stride in LDS (bf16)
  constexpr int kVRow = D + 32;                // V row stride in LDS (bf16)
  constexpr int kSteps = D / 16;               // 16-dim steps of S^T
  constexpr int kNDT = D / 32;                 // 32-dim output slices
  constexpr int kKLoads = kKT * D / 8 / kThreads;        // 16-byte K loads per thread
  static_assert(kKLoads >= 1, "tile shape");

  const int H = a.num_heads;
  int b, h, tile, L, q0, nq;
  if (!prefill_work_of(blockIdx.x, a, b, h, tile, L, q0, nq)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int j = lane & 31;
  const int hh = lane >> 5;
  const int jj = lane & 15;
  const int g1 = (lane >> 4) & 1;

  const int t_first = tile * kQT32;
  if (t_first >= nq) return;
  const int pos0 = L - nq;
  const int w_first = t_first + wave * 32;
  const bool wave_active = w_first < nq;   // uniform over the wave

  const float cs = a.scale_log2 == 0.0f ? 1.0f : fabsf(a.scale_log2);
  const float bmul = a.scale_log2 == 0.0f ? 0.0f : (a.scale_log2 < 0.0f ? -1.0f : 1.0f);

  const int t_row = w_first + j;
  const bool row_ok = t_row < nq;
  const int p_row = pos0 + t_row;
  const int dq = p_row - 4 * hh;
  const int dlo = p_row - L;

  bf16x8_t qv[kSteps];
  {
    const int tq = row_ok ? t_row : t_first;
    const bool qzero = !row_ok || bmul == 0.0f;
    const uint32_t qsign = bmul < 0.0f ? 0x80008000u : 0u;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * H + h) * D + 8 * hh);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      uint4 v = qrow[2 * st];
      v = qzero ? make_uint4(0u, 0u, 0u, 0u)
                : make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      qv[st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kKT * kVRow];
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 1 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md; i += kThreads)
      rel_lds[i] = bmul == 0.0f ? 0.0f : rel_bias(i - rel_md, a.rel, head_row) * bmul;
  }

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int ntiles = (L + kKT - 1) / kKT;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;

  // staging as in the kernel above; K and V of a tile are loaded at
  // different steps, so each has its own block-table entries
  int tbk[2], tbv[2];
  auto load_table = [&](int (&tb)[2], int tk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = tk * (kKT / kBlockSize) + i;
      tb[i] = blk < nblk_seq ? table[blk] : 0;
    }
  };
  typedef uint32_t st_t __attribute__((ext_vector_type(4 * kKLoads)));
  st_t kst, vst;
  auto fetch = [&](st_t& dst, const uint16_t* src, const int (&tb)[2]) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      const int sel = (i * kThreads + wave * 64) / (D / 8) / kBlockSize;
      const int64_t blk = ((int64_t)tb[sel] * H + h) * (kBlockSize * D);
      const uint32_t off = (uint32_t)((r % kBlockSize) * D + col);
      const uint4 x = *reinterpret_cast<const uint4*>(src + blk + off);
      dst[4 * i] = x.x;
      dst[4 * i + 1] = x.y;
      dst[4 * i + 2] = x.z;
      dst[4 * i + 3] = x.w;
    }
  };
  auto stash_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][r * kKRow + col]) =
          make_uint4(kst[4 * i], kst[4 * i + 1], kst[4 * i + 2], kst[4 * i + 3]);
    }
  };
  // V rows at or past L come from an in-pool block and are zeroed here, a
  // step after their loads were issued
  auto stash_v = [&](int buf, int tk) {
    const int base = tk * kKT;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int e = i * kThreads + tid;
      const int r = e / (D / 8), col = (e % (D / 8)) * 8;
      uint4 x = make_uint4(vst[4 * i], vst[4 * i + 1], vst[4 * i + 2], vst[4 * i + 3]);
      if (base + kKT > L && base + r >= L) x = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&v_lds[buf][r * kVRow + col]) = x;
    }
  };

  auto qk = [&](auto kb_c, float16_t& s) {
    constexpr int kb = decltype(kb_c)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const uint4 kv = *reinterpret_cast<const uint4*>(&k_lds[kb][j * kKRow + 16 * st + 8 * hh]);
      s = mfma32_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[st], s);
    }
  };

  float16_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  float lsum = 0.0f;
  float m_ref = -INFINITY, neg_m = 0.0f;
  const float* bias_row = nullptr;
  if (BIAS == 1) {
    const int tb_row = row_ok ? t_row : t_first;
    bias_row = a.bias_start
                   ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                   : a.attn_bias +
                         (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) * a.max_seq_len;
  }
  const bool bias_vec =
      BIAS == 1 &&
      __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(bias_row) & 15) != 0) == 0;
  const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  float4_t bnext[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bnext[u] = float4_t{0, 0, 0, 0};
  if (BIAS == 1 && bias_vec && wave_active && kKT <= L) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      bnext[u] = *reinterpret_cast<const float4_t*>(bias_row + 8 * u + 4 * hh);
  }

  // start-up: K and V of tile 0 and K of tile 1 to LDS, the S^T products of
  // tile 0, then the loads of V of tile 1 and K of tile 2 in flight
  float16_t s_cur;
#pragma unroll
  for (int i = 0; i < 16; ++i) s_cur[i] = 0.0f;
  if (ntiles > 0) {
    int tb1[2] = {0, 0};
    load_table(tbk, 0);
    if (ntiles > 1) load_table(tb1, 1);
    fetch(kst, kc, tbk);
    fetch(vst, vc, tbk);
    st_t k1 = kst;
    if (ntiles > 1) fetch(k1, kc, tb1);
    stash_k(0);
    stash_v(0, 0);
    if (ntiles > 1) {
      kst = k1;
      stash_k(1);
    }
    tbk[0] = tb1[0];
    tbk[1] = tb1[1];
  }
  __syncthreads();
  // entering step k, tbv holds the table entries of tile k+2 and tbk those
  // of tile k+3
  if (ntiles > 0) {
    if (wave_active) qk(IntC<0>{}, s_cur);
    if (ntiles > 1) {
      tbv[0] = tbk[0];
      tbv[1] = tbk[1];   // tile 1
      fetch(vst, vc, tbv);
      if (ntiles > 2) {
        load_table(tbk, 2);
        fetch(kst, kc, tbk);
        tbv[0] = tbk[0];
        tbv[1] = tbk[1];   // tile 2
      }
      if (ntiles > 3) load_table(tbk, 3);
    }
  }
  __syncthreads();   // every wave has read K of tile 0 before tile 2 replaces it

  auto tile_step = [&](int tk, auto buf_c, auto next_c) {
    constexpr int buf = decltype(buf_c)::value;   // tk & 1
    constexpr bool NEXT = decltype(next_c)::value;
    const int c0 = tk * kKT;
    if (wave_active) {
      // ---- bias (unscaled scores) and the tail mask, as above ----
      if constexpr (BIAS == 1) {
        if (bias_vec && c0 + kKT <= L) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s_cur[4 * u + r] = fmaf(bnext[u][r], bmul, s_cur[4 * u + r]);
          if (c0 + 2 * kKT <= L) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              bnext[u] =
                  *reinterpret_cast<const float4_t*>(bias_row + c0 + kKT + 8 * u + 4 * hh);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s_cur[4 * u + r] =
                  fmaf(bias_row[min(c0 + 8 * u + 4 * hh + r, L - 1)], bmul, s_cur[4 * u + r]);
        }
      }
      if constexpr (BIAS == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j0 = c0 + 8 * u + 4 * hh;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s_cur[4 * u + r] += rel_lds[min(max(j0 + r - p_row, -rel_md), rel_md) + rel_md];
        }
      }
      if (c0 + kKT > L) {   // uniform: only the last tile
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s_cur[4 * u + r] = dq - c0 - 8 * u - r > dlo ? s_cur[4 * u + r] : -INFINITY;
      }
      // ---- row maximum and the lazily moved reference (base 2) ----
      float mt = s_cur[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = vmax(mt, s_cur[i]);
      {
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1])) * cs;
      }
      const bool move = mt > m_ref + 8.0f;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;
        m_ref = move ? mt : m_ref;
        neg_m = move ? -mt : neg_m;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;
      }
      // ---- the next tile's products, independent of the weights below ----
      float16_t s_next;
      if constexpr (NEXT) qk(IntC<buf ^ 1>{}, s_next);
      bf16x8_t pw[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pw[ks][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * ks + e], cs, neg_m));
        const uint4 pu = __builtin_bit_cast(uint4, pw[ks]);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.x), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.y), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.z), one2, lsum,
                                               false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.w), one2, lsum,
                                               false);
      }
      // ---- O^T += V^T P^T over the tile's two 16-key steps ----
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) {
          const uint16_t* p = &v_lds[buf][(16 * ks + 4 * hh + (jj >> 2)) * kVRow + 32 * dt +
                                          16 * g1 + 4 * (jj & 3)];
          const uint2 lo = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * kVRow)));
          acc[dt] = mfma32_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                pw[ks], acc[dt]);
        }
      }
      if constexpr (NEXT) s_cur = s_next;
    }
    if constexpr (NEXT) {
      if (tk + 2 < ntiles) stash_k(buf);
      stash_v(buf ^ 1, tk + 1);
      if (tk + 2 < ntiles) {
        fetch(vst, vc, tbv);   // V of tile k+2
        if (tk + 3 < ntiles) {
          fetch(kst, kc, tbk);   // K of tile k+3
          tbv[0] = tbk[0];
          tbv[1] = tbk[1];
          if (tk + 4 < ntiles) load_table(tbk, tk + 4);
        }
      }
      __syncthreads();
    }
  };
  int tk = 0;
  for (; tk + 2 < ntiles; tk += 2) {
    tile_step(tk, IntC<0>{}, IntC<true>{});
    tile_step(tk + 1, IntC<1>{}, IntC<true>{});
  }
  if (tk + 1 < ntiles) {
    tile_step(tk, IntC<0>{}, IntC<true>{});
    tile_step(tk + 1, IntC<1>{}, IntC<false>{});
  } else if (tk < ntiles) {
    tile_step(tk, IntC<0>{}, IntC<false>{});
  }

  // ---- epilogue: out = O / l, rounded to bf16 (the swap runs in every lane) ----
  const auto xl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                   false, false);
  const float l_tot = __uint_as_float(xl[0]) + __uint_as_float(xl[1]);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + t_row) * H + h) * D;
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t o = {(__bf16)(acc[dt][4 * u] * inv), (__bf16)(acc[dt][4 * u + 1] * inv),
                    (__bf16)(acc[dt][4 * u + 2] * inv), (__bf16)(acc[dt][4 * u + 3] * inv)};
      *reinterpret_cast<bf16x4_t*>(orow + 32 * dt + 8 * u + 4 * hh) = o;
    }
  }
}

// Bidirectional launches without a window or chunks take the
// 32-query-per-wave kernel, and so do causal ones without a window or chunks
// at head_dim 64 (switch below); other causal, windowed and chunked ones the
// 16-query-per-wave kernel.
#ifndef PA_PREFILL_BF16_CAUSAL32
#define PA_PREFILL_BF16_CAUSAL32 1
#endif

template <int D, int BIAS>
constexpr bool causal_on_32() { return PA_PREFILL_BF16_CAUSAL32 && D == 64; }

bool wide_tiles(const PrefillArgs& a, int D) {
  if (a.window > 0 || a.chunk > 0) return false;
  return !a.causal || (PA_PREFILL_BF16_CAUSAL32 && D == 64);
}

template <int D, int BIAS>
void launch_bias(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(Cfg<D>::kThreads);
  const bool banded = a.window > 0 || a.chunk > 0;
  if (a.causal) {
    if (banded)
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, true, true>), grid, block, 0, stream, a);
    else if constexpr (causal_on_32<D, BIAS>())
      hipLaunchKernelGGL((pa_prefill_bf16_32<D, BIAS, true>), grid, dim3(kThreads32), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, true, false>), grid, block, 0, stream, a);
  } else if (banded) {
    hipLaunchKernelGGL((pa_prefill_bf16<D, BIAS, false, true>), grid, block, 0, stream, a);
  } else {
    if constexpr (PA_PREFILL_BF16_PIPE && D == 64 && BIAS == 0)
      hipLaunchKernelGGL((pa_prefill_bf16_32p<64, 0>), grid, dim3(kThreads32), 0, stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_bf16_32<D, BIAS, false>), grid, dim3(kThreads32), 0, stream,
                         a);
  }
}

template <int D>
hipError_t launch_d(PrefillArgs a, hipStream_t stream) {
  const int bias = a.rel.table ? 2 : (a.attn_bias ? 1 : 0);
  // queries per workgroup
  const int qt = wide_tiles(a, D) ? kQT32 : kQT;
  a.num_qtiles = (a.max_seq_len + qt - 1) / qt;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  const int64_t nwg = (pairs + kXcds - 1) / kXcds * kXcds * a.num_qtiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  if (bias == 2)
    launch_bias<D, 2>(a, grid, stream);
  else if (bias == 1)
    launch_bias<D, 1>(a, grid, stream);
  else
    launch_bias<D, 0>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace pa
