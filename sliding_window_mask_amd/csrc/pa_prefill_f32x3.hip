// fp32 prefill attention on the bf16 matrix cores, for bidirectional launches
// without a window or chunks at head_dim 64 (gfx950).
//
// Computes the same rows as the fp32 prefill kernel -- every query of a
// sequence attends to all L keys, softmax((q K^T + A) * scale) V ("[Kernel]
// [Model] PagedAttention: Support custom attention bias for T5 model (1/2)",
// PR description) -- with fp32 inputs, outputs and accuracy, but on
// v_mfma_f32_16x16x32_bf16 instead of v_mfma_f32_16x16x4_f32.
//
// Every fp32 operand x is split exactly into three bf16 parts, x = x0 + x1 +
// x2: x0 keeps the top 8 significand bits of x (bit truncation), x1 the next
// 8 of the exact remainder x - x0, x2 the rest (x - x0 - x1, at most 8 bits),
// so each part is a bf16 value and the sum is exact. A product a.b is then
// the sum of the nine products a_i b_j; the six with i + j <= 2 are computed
// (each bf16 x bf16 product is exact in fp32, and the matrix cores accumulate
// in fp32), the three dropped ones are below 2^-16 |a_1 b_1| ~ 2^-24 |a b|,
// i.e. at the level of fp32 rounding. Six bf16 MFMAs of 16x16x32 do the
// work of eight 16x16x4 fp32 ones in about a third of the matrix-core time
// (the bf16 peak is 16 times the fp32 one).
//
// Work decomposition: one workgroup of 8 wave64s per (128-query tile, head,
// sequence), numbered and ordered as in the other prefill kernels (XCD-aware,
// longest sequences first for batches of up to 63). Keys are walked in 32-key
// tiles through double-buffered LDS: the workgroup loads a tile's fp32 K and
// V rows (16 bytes per thread each), splits them and stores the three bf16
// planes of each. The loop is software-pipelined: each step issues the S^T
// products of the next tile before the softmax of the current one, so the
// matrix cores have independent work while the wave computes and splits the
// weights. K of a tile is therefore staged two steps before its P.V step and
// V one step before, and one barrier per step still suffices.
//
// Operand layouts (16x16x32, lane l, g = l / 16, c = l % 16), as in the bf16
// prefill kernel: S^T = K Q^T over two 32-dim steps st, lane l feeding
// K[key c][16 g + 8 st + e] and Q[query c][same dims] (e = 0..7); it ends
// holding S^T[key 4g + r][query c] for each 16-key chunk. O^T = V^T P^T over
// the tile's 32 keys: the P operand is the lane's own 8 weights (keys 4g+e of
// chunk 0, then of chunk 1) and the V^T operand comes from two transposing
// LDS reads (ds_read_b64_tr_b16) per plane and 16-dim output slice. Scores
// are kept in base 2 (q is multiplied by scale * log2(e) in fp32 before it is
// split) and the softmax, with its lazily moved reference, is the fp32
// kernel's.
#include "pa_internal.h"

namespace pa {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 64;                  // head_dim of this kernel
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 16 * kWaves;        // queries per workgroup
constexpr int kKT = 32;                 // keys per tile
constexpr int kKRow = kD + 8;           // K plane row stride in LDS (bf16)
constexpr int kVRow = kD + 16;          // V plane row stride in LDS (bf16)
constexpr int kNDT = kD / 16;           // 16-dim output slices

__device__ __forceinline__ float4_t mfma(const bf16x8_t& a, const bf16x8_t& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float vmax(float x, float y) {
  return __builtin_elementwise_maximum(x, y);
}

// x = p0 + p1 + p2 exactly, each part a bf16 value (its fp32 bit pattern has
// zero low 16 bits); returned as those upper 16-bit halves
__device__ __forceinline__ void split3(float x, uint32_t& h0, uint32_t& h1, uint32_t& h2) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t t0 = u & 0xffff0000u;
  const float r = x - __uint_as_float(t0);           // exact
  const uint32_t t1 = __float_as_uint(r) & 0xffff0000u;
  const float r2 = r - __uint_as_float(t1);          // exact, at most 8 significant bits
  h0 = t0 >> 16;
  h1 = t1 >> 16;
  h2 = __float_as_uint(r2) >> 16;
}

// four floats -> three planes of four bf16 (8 bytes each)
__device__ __forceinline__ void split4(const float4_t& v, uint2& p0, uint2& p1, uint2& p2) {
  uint32_t a0, a1, a2, b0, b1, b2, c0, c1, c2, d0, d1, d2;
  split3(v[0], a0, a1, a2);
  split3(v[1], b0, b1, b2);
  split3(v[2], c0, c1, c2);
  split3(v[3], d0, d1, d2);
  p0 = make_uint2(a0 | (b0 << 16), c0 | (d0 << 16));
  p1 = make_uint2(a1 | (b1 << 16), c1 | (d1 << 16));
  p2 = make_uint2(a2 | (b2 << 16), c2 | (d2 << 16));
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// BIAS: 0 none, 1 materialised (padded or ragged) fp32 bias, 2 T5 relative
// bias from a bucket table (a.rel).
template <int BIAS>
__global__ void __launch_bounds__(kThreads, 2)
pa_prefill_f32x3(PrefillArgs a) {
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
  const int pos0 = L - nq;
  const int w_first = t_first + wave * 16;
  const bool wave_active = w_first < nq;       // uniform over the wave

  // the lane's query row; keys j >= L of the last tile are masked: with
  // d = p - j for key j = c0 + 4g + r, d = dq - c0 - r and j < L iff d > p - L
  const int t_row = w_first + c;
  const bool row_ok = t_row < nq;
  const int p_row = pos0 + t_row;
  const int dq = p_row - 4 * g;
  const int dlo = p_row - L;
  const int pr0 = pos0 + w_first;   // position of the wave's first row
  const float cs = a.scale_log2;

  // q * scale * log2(e) in fp32, split into three bf16 planes: dims
  // 16 g + 8 st .. + 7 of the lane's query for the two steps st
  // (loaded here, split once the first tiles' loads are in flight)
  float4_t qx[4];
  {
    const int tq = row_ok ? t_row : t_first;
    const float* qrow = static_cast<const float*>(a.q) + ((int64_t)(q0 + tq) * H + h) * kD + 16 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) qx[i] = *reinterpret_cast<const float4_t*>(qrow + 4 * i);
  }
  bf16x8_t qp[3][2];
  auto split_q = [&]() {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float4_t x0 = qx[2 * st], x1 = qx[2 * st + 1];
      if (!row_ok) x0 = x1 = float4_t{0, 0, 0, 0};
      uint2 a0, a1, a2, b0, b1, b2;
      split4(x0 * cs, a0, a1, a2);
      split4(x1 * cs, b0, b1, b2);
      qp[0][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, b0.x, b0.y));
      qp[1][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a1.x, a1.y, b1.x, b1.y));
      qp[2][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a2.x, a2.y, b2.x, b2.y));
    }
  };

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][3][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][3][kKT * kVRow];
  // T5 bias of relative position r = j - p at rel_lds[r + md + 3] for r in
  // [-md - 3, md + 3] (longer distances share the end buckets, so the three
  // entries past each end repeat them: a lane's four consecutive keys clamp
  // their first distance once and read four neighbouring entries),
  // multiplied by scale * log2(e) as a materialised bias entry is; gfx950
  // gives a workgroup up to 160 KiB of LDS, and two of these workgroups
  // (65 KiB each) fit a CU
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 7 : 1];
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md + 6; i += kThreads)
      rel_lds[i] = rel_bias(min(max(i - 3 - rel_md, -rel_md), rel_md), a.rel, head_row) * cs;
  }

  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int ntiles = (L + kKT - 1) / kKT;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;

  // staging: thread t loads dims 4 (t % 16) .. + 3 of tile row t / 16 (a
  // wave's 64 threads cover 4 rows of one cache block, so the address is a
  // uniform block base plus a fixed per-lane offset); rows at or past L come
  // from an in-pool block (K there only feeds masked scores; V is zeroed)
  const int srow = tid >> 4;
  const int scol = (tid & 15) * 4;
  // K and V of a tile are staged at different times (K two tiles ahead of
  // its P.V step, V one), so each has its own block-table entries
  int tbk[2], tbv[2];
  auto load_table = [&](int (&tb)[2], int tk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = tk * (kKT / kBlockSize) + i;
      tb[i] = blk < nblk_seq ? table[blk] : 0;
    }
  };
  const uint32_t soff = (uint32_t)((srow % kBlockSize) * kD + scol);
  float4_t kst, vst;
  auto fetch_k = [&]() {
    kst = *reinterpret_cast<const float4_t*>(
        kc + ((int64_t)tbk[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
  };
  auto fetch_v = [&]() {
    vst = *reinterpret_cast<const float4_t*>(
        vc + ((int64_t)tbv[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
  };
  auto stash_k = [&](int buf) {
    uint2 k0, k1, k2;
    split4(kst, k0, k1, k2);
    *reinterpret_cast<uint2*>(&k_lds[buf][0][srow * kKRow + scol]) = k0;
    *reinterpret_cast<uint2*>(&k_lds[buf][1][srow * kKRow + scol]) = k1;
    *reinterpret_cast<uint2*>(&k_lds[buf][2][srow * kKRow + scol]) = k2;
  };
  // V rows at or past L are zeroed here, a tile after their loads were
  // issued (a select right after the loads would wait for them at once)
  auto stash_v = [&](int buf, int tk) {
    uint2 v0, v1, v2;
    if (tk * kKT + kKT > L && tk * kKT + srow >= L) vst = float4_t{0, 0, 0, 0};
    split4(vst, v0, v1, v2);
    *reinterpret_cast<uint2*>(&v_lds[buf][0][srow * kVRow + scol]) = v0;
    *reinterpret_cast<uint2*>(&v_lds[buf][1][srow * kVRow + scol]) = v1;
    *reinterpret_cast<uint2*>(&v_lds[buf][2][srow * kVRow + scol]) = v2;
  };

  float4_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) acc[dt] = float4_t{0, 0, 0, 0};
  float m_ref = -INFINITY, neg_m = 0.0f, l_run = 0.0f;
  const float* bias_row = nullptr;
  if (BIAS == 1) {
    const int tb_row = row_ok ? t_row : t_first;   // every row sees every key
    bias_row = a.bias_start
                   ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                   : a.attn_bias +
                         (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) * a.max_seq_len;
  }
  // a lane's 4 bias entries of a chunk are contiguous: one 16-byte load on
  // chunks inside the sequence, when every lane's row is 16-byte aligned
  const bool bias_vec =
      BIAS == 1 &&
      __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(bias_row) & 15) != 0) == 0;

  // ---- S^T = K Q^T of one tile: K_i Q_j for i + j <= 2, two 32-dim steps ----
  auto qk = [&](auto kb_c, float4_t (&s)[2]) {
    constexpr int kb = decltype(kb_c)::value;
    s[0] = s[1] = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int o = (ch * 16 + c) * kKRow + 16 * g + 8 * st;
        const bf16x8_t k0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][0][o]));
        const bf16x8_t k1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][1][o]));
        const bf16x8_t k2 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][2][o]));
        s[ch] = mfma(k2, qp[0][st], s[ch]);
        s[ch] = mfma(k1, qp[1][st], s[ch]);
        s[ch] = mfma(k0, qp[2][st], s[ch]);
        s[ch] = mfma(k1, qp[0][st], s[ch]);
        s[ch] = mfma(k0, qp[1][st], s[ch]);
        s[ch] = mfma(k0, qp[0][st], s[ch]);
      }
    }
  };

  // a lane's 4 bias entries of each 16-key chunk of a tile, loaded a step
  // ahead (whole chunks, when the rows are 16-byte aligned), non-temporal:
  // each entry is read once
  float4_t bcur[2];
  auto load_bias = [&](int tk) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int c0 = tk * kKT + ch * 16;
      bcur[ch] = float4_t{0, 0, 0, 0};
      if (bias_vec && c0 + 16 <= L)
        bcur[ch] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(bias_row + c0 + 4 * g));
    }
  };

  // Pipeline (one barrier per tile): entering step k, the scores S_k are in
  // registers, K of tile k+1 and V of tile k are in LDS, and the loads of K
  // of tile k+2 and V of tile k+1 are in flight. Step k issues the products
  // of S_{k+1} before the softmax of tile k, so the matrix cores work on
  // them while the wave computes the weights, then P.V of tile k; meanwhile
  // K of tile k+2 goes to the K buffer that tile k left and V of tile k+1 to
  // the V buffer that tile k-1 left.
  float4_t s_cur[2];
  s_cur[0] = s_cur[1] = float4_t{0, 0, 0, 0};
  // start-up: the table entries of tiles 0 and 1, then K and V of tile 0
  // and K of tile 1, all in flight together
  if (ntiles > 0) {
    int tb1[2] = {0, 0};
    load_table(tbk, 0);
    if (ntiles > 1) load_table(tb1, 1);
    tbv[0] = tbk[0]; tbv[1] = tbk[1];
    fetch_k();
    fetch_v();
    float4_t k1 = kst;
    if (ntiles > 1) {
      tbk[0] = tb1[0]; tbk[1] = tb1[1];
      k1 = *reinterpret_cast<const float4_t*>(
          kc + ((int64_t)tbk[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
    }
    split_q();
    stash_k(0);
    stash_v(0, 0);
    if (ntiles > 1) {
      kst = k1;
      stash_k(1);
    }
  } else {
    split_q();
  }
  __syncthreads();
  // entering step k, tbv holds the table entries of tile k+2 and tbk those
  // of tile k+3
  if (ntiles > 0) {
    if (wave_active) {
      qk(IntC<0>{}, s_cur);
      if constexpr (BIAS == 1) load_bias(0);
    }
    if (ntiles > 1) {
      tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile 1
      fetch_v();
      if (ntiles > 2) {
        load_table(tbk, 2);
        fetch_k();
        tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile 2
      }
      if (ntiles > 3) load_table(tbk, 3);
    }
  }
  __syncthreads();   // every wave has read K of tile 0 before tile 2 replaces it

  // One step. NEXT: a tile follows (its S^T products are issued here);
  // LAST: the final tile, the only one that can reach past the sequence end.
  auto tile_step = [&](int tk, auto buf_c, auto next_c, auto last_c) {
    constexpr int buf = decltype(buf_c)::value;   // tk & 1
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    const int base = tk * kKT;
    if (wave_active) {
      float4_t* s = s_cur;
      // ---- bias (added as a * scale * log2(e)) and the tail mask ----
      if constexpr (BIAS == 1) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int c0 = base + ch * 16;
          const int j0 = c0 + 4 * g;
          if (bias_vec && (!LAST || c0 + 16 <= L)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + bcur[ch][r] * cs;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = -INFINITY;
              if (j0 + r < L) x = s[ch][r] + bias_row[j0 + r] * cs;
              s[ch][r] = x;
            }
          }
        }
        if constexpr (NEXT) load_bias(tk + 1);   // in flight until the next step
      }
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int c0 = base + ch * 16;
        const int j0 = c0 + 4 * g;
        if constexpr (BIAS == 2) {
          // the chunk's relative positions j - p run from c0 - pr0 - 15 to
          // c0 + 15 - pr0 (pr0: the wave's first row); all at or beyond the
          // maximum distance on one side (uniform), they share that side's
          // end bucket
          if (c0 + 15 - pr0 <= -rel_md || c0 - pr0 - 15 >= rel_md) {
            const float bend = rel_lds[c0 < pr0 ? 3 : 2 * rel_md + 3];
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + bend;
          } else {
            const int e0 = min(max(j0 - p_row, -rel_md - 3), rel_md) + rel_md + 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + rel_lds[e0 + r];
          }
        }
        if (LAST && c0 + 16 > L) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[ch][r] = dq - c0 - r > dlo ? s[ch][r] : -INFINITY;
        }
      }
      // ---- online softmax with a lazily moved reference (base 2) ----
      float mt = vmax(vmax(vmax(s[0][0], s[0][1]), vmax(s[0][2], s[0][3])),
                      vmax(vmax(s[1][0], s[1][1]), vmax(s[1][2], s[1][3])));
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = vmax(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                          __float_as_uint(mt), false, false);
        mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      const bool move = mt > m_ref + 8.0f;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;
        m_ref = move ? mt : m_ref;
        neg_m = move ? -mt : neg_m;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;
      }
      // the next tile's products, independent of the weights computed below
      float4_t s_next[2];
      if constexpr (NEXT) qk(IntC<buf ^ 1>{}, s_next);
      // weights, split into three bf16 planes (keys 4g + e of chunk 0, then 1)
      uint32_t w0[4], w1[4], w2[4];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(s[ch][r] + neg_m);
          l_run += pr[r];
        }
        uint2 a0, a1, a2;
        split4(float4_t{pr[0], pr[1], pr[2], pr[3]}, a0, a1, a2);
        w0[2 * ch] = a0.x; w0[2 * ch + 1] = a0.y;
        w1[2 * ch] = a1.x; w1[2 * ch + 1] = a1.y;
        w2[2 * ch] = a2.x; w2[2 * ch + 1] = a2.y;
      }
      const bf16x8_t p0 = __builtin_bit_cast(bf16x8_t, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      const bf16x8_t p1 = __builtin_bit_cast(bf16x8_t, make_uint4(w1[0], w1[1], w1[2], w1[3]));
      const bf16x8_t p2 = __builtin_bit_cast(bf16x8_t, make_uint4(w2[0], w2[1], w2[2], w2[3]));
      // ---- O^T += V^T P^T: V_j P_i for i + j <= 2, per 16-dim slice ----
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
        bf16x8_t vv[3];
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
          const uint16_t* pp = &v_lds[buf][pl][(4 * g + (c >> 2)) * kVRow + 16 * dt + 4 * (c & 3)];
          const uint2 lo = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)pp));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(pp + 16 * kVRow)));
          vv[pl] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
        acc[dt] = mfma(vv[2], p0, acc[dt]);
        acc[dt] = mfma(vv[1], p1, acc[dt]);
        acc[dt] = mfma(vv[0], p2, acc[dt]);
        acc[dt] = mfma(vv[1], p0, acc[dt]);
        acc[dt] = mfma(vv[0], p1, acc[dt]);
        acc[dt] = mfma(vv[0], p0, acc[dt]);
      }
      if constexpr (NEXT) {
        s_cur[0] = s_next[0];
        s_cur[1] = s_next[1];
      }
    }
    if constexpr (NEXT) {
      // staging: K of tile k+2 into the K buffer of tile k (read at step
      // k-1), V of tile k+1 into the V buffer of tile k-1 (read at step k-1);
      // then the loads of V of tile k+2 and K of tile k+3
      if (tk + 2 < ntiles) stash_k(buf);
      stash_v(buf ^ 1, tk + 1);
      if (tk + 2 < ntiles) {
        fetch_v();
        if (tk + 3 < ntiles) {
          fetch_k();
          tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile k+3
          if (tk + 4 < ntiles) load_table(tbk, tk + 4);
        }
      }
      __syncthreads();
    }
  };
  int tk = 0;
  for (; tk + 2 < ntiles; tk += 2) {
    tile_step(tk, IntC<0>{}, IntC<true>{}, IntC<false>{});
    tile_step(tk + 1, IntC<1>{}, IntC<true>{}, IntC<false>{});
  }
  if (tk + 1 < ntiles) {
    tile_step(tk, IntC<0>{}, IntC<true>{}, IntC<false>{});
    tile_step(tk + 1, IntC<1>{}, IntC<false>{}, IntC<true>{});
  } else if (tk < ntiles) {
    tile_step(tk, IntC<0>{}, IntC<false>{}, IntC<true>{});
  }

  // ---- epilogue: out = O / l (lanes c, c+16, c+32, c+48 share a query) ----
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* orow = static_cast<float*>(a.out) + ((int64_t)(q0 + t_row) * H + h) * kD;
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
    *reinterpret_cast<float4_t*>(orow + 16 * dt + 4 * g) = acc[dt] * inv;
}

// ---------------------------------------------------------------------------
// Causal, windowed and chunked launches on the same split operands (BAND 0:
// causal without a window, 1: window, 2: chunks). A workgroup walks only the
// key tiles its rows may see ([lo, hi) of its positions, from the 16-key block
// holding lo), each wave computes only the tiles its own 16 rows may see, and
// a 16-key chunk that some row of a wave sees only in part is masked per
// element; chunks inside every row's range take the unmasked path. The tile
// loop is pipelined as in the kernel above.
#ifndef PA_X3_BAND_PIPE
#define PA_X3_BAND_PIPE 1
#endif

template <int BIAS, bool CAUSAL, int BAND>
__global__ void __launch_bounds__(kThreads, 4)   // 4 waves per SIMD: two workgroups per CU
pa_prefill_f32x3_band(PrefillArgs a) {
  const int H = a.num_heads;
  int b, h, tile, L, q0, nq;
  if (!prefill_work_of(blockIdx.x, a, b, h, tile, L, q0, nq)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int c = lane & 15;
  const int g = lane >> 4;
  const int window = BAND == 1 ? a.window : 0;
  const int chunk = BAND == 2 ? a.chunk : 0;
  // The tile loop is pipelined as in the kernel above: the S^T products of
  // tile k+1 are issued at step k (K of tile k+1 is in LDS then, and the
  // buffer of tile k is refilled during step k). With kPipe they go before
  // the softmax of tile k, overlapping it; with a materialised bias they go
  // after its P.V, and the next tile's bias entries are requested with them,
  // which keeps those variants within 128 VGPRs (four waves per SIMD)
  // without spilling.
  constexpr bool kPipe = BIAS != 1 && PA_X3_BAND_PIPE;

  const int t_first = tile * kQT;
  if (t_first >= nq) return;
  const int pos0 = L - nq;
  const int w_first = t_first + wave * 16;
  const bool wave_active = w_first < nq;       // uniform over the wave

  // the lane's query row: key j (d = p - j) is visible iff dlo < d < dhi;
  // for key j = c0 + 4g + r, d = dq - c0 - r. Rows past the query set see no
  // key (and so read no bias entry).
  const int t_row = w_first + c;
  const bool row_ok = t_row < nq;
  const int p_row = pos0 + t_row;
  const int dq = p_row - 4 * g;
  const int pr0 = pos0 + w_first;   // position of the wave's first row
  int dlo, dhi;
  if constexpr (BAND == 0) {
    dlo = max(p_row - L, -1);
    dhi = 0x7fffffff;
  } else {
    prefill_row_bounds(p_row, L, window, chunk, CAUSAL, dlo, dhi);
  }
  if (!row_ok) dlo = 0x7fffffff;
  // with a window or chunks, the keys [bjlo, bjhi] the row sees (empty for
  // rows past the query set): chunks some row sees only in part read their
  // bias entries with the key clamped into this range, so that they are
  // requested a step ahead with the whole chunks and still only visible
  // entries are read (causal launches read them when they are used: the
  // registers held across the step would cost spills there)
  constexpr bool kEarly = BIAS == 1 && BAND != 0;
  int bjlo = 0, bjhi = -1;
  if (kEarly && row_ok) {
    bjhi = p_row - dlo - 1;
    bjlo = max(p_row - dhi + 1, 0);
  }
  const float cs = a.scale_log2;

  // keys [lo, hi) the workgroup's rows may see, walked in 32-key tiles from
  // the 16-key block holding lo
  int lo, hi;
  prefill_key_range(pos0 + t_first, pos0 + min(t_first + kQT, nq) - 1, L, window, chunk, CAUSAL,
                    lo, hi);
  const int kstart = lo & ~(kBlockSize - 1);
  const int ntiles = hi > kstart ? (hi - kstart + kKT - 1) / kKT : 0;
  const int nblk = (hi + kBlockSize - 1) / kBlockSize;   // blocks backing keys below hi
  // the wave's keys [wlo, whi), its tiles wt0 .. wt1, and the keys [cwlo,
  // cwhi) every one of its rows sees (uniform)
  int wlo = 0, whi = 0, wt0 = 1, wt1 = 0, cwlo = 0, cwhi = 0;
  if (wave_active) {
    const int pw0 = pos0 + w_first, pw1 = pos0 + min(w_first + 16, nq) - 1;
    prefill_key_range(pw0, pw1, L, window, chunk, CAUSAL, wlo, whi);
    if (whi > wlo) {
      wt0 = (wlo - kstart) / kKT;
      wt1 = (whi - 1 - kstart) / kKT;
    }
    if constexpr (BAND == 0) {
      cwlo = 0;
      cwhi = L;
    } else {
      prefill_common_keys(pw0, pw1, window, chunk, cwlo, cwhi);
      cwhi = min(cwhi, L);
    }
    if (CAUSAL) cwhi = min(cwhi, pw0 + 1);
  }
  auto chunk_whole = [&](int c0) { return c0 >= cwlo && c0 + 16 <= cwhi; };
  auto chunk_live = [&](int c0) { return c0 < whi && c0 + 16 > wlo; };

  // q * scale * log2(e) in fp32, split into three bf16 planes
  // (loaded here, split once the first tiles' loads are in flight)
  float4_t qx[4];
  {
    const int tq = row_ok ? t_row : t_first;
    const float* qrow = static_cast<const float*>(a.q) + ((int64_t)(q0 + tq) * H + h) * kD + 16 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) qx[i] = *reinterpret_cast<const float4_t*>(qrow + 4 * i);
  }
  bf16x8_t qp[3][2];
  auto split_q = [&]() {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float4_t x0 = qx[2 * st], x1 = qx[2 * st + 1];
      if (!row_ok) x0 = x1 = float4_t{0, 0, 0, 0};
      uint2 a0, a1, a2, b0, b1, b2;
      split4(x0 * cs, a0, a1, a2);
      split4(x1 * cs, b0, b1, b2);
      qp[0][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, b0.x, b0.y));
      qp[1][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a1.x, a1.y, b1.x, b1.y));
      qp[2][st] = __builtin_bit_cast(bf16x8_t, make_uint4(a2.x, a2.y, b2.x, b2.y));
    }
  };

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][3][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][3][kKT * kVRow];
  __shared__ float rel_lds[BIAS == 2 ? 2 * kMaxRelDistance + 7 : 1];   // as above
  const int rel_md = BIAS == 2 ? a.rel.max_distance : 0;
  if constexpr (BIAS == 2) {
    const float* head_row = a.rel.table + (int64_t)h * a.rel.num_buckets;
    for (int i = tid; i <= 2 * rel_md + 6; i += kThreads)
      rel_lds[i] = rel_bias(min(max(i - 3 - rel_md, -rel_md), rel_md), a.rel, head_row) * cs;
  }

  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  // staging as in the kernel above; blocks at or past hi come from an
  // in-pool block (K there only feeds masked scores; V is zeroed), so no
  // table entry backing only keys the workgroup cannot see is read
  const int srow = tid >> 4;
  const int scol = (tid & 15) * 4;
  int tbk[2], tbv[2];
  auto load_table = [&](int (&tb)[2], int tk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = kstart / kBlockSize + tk * (kKT / kBlockSize) + i;
      tb[i] = blk < nblk ? table[blk] : 0;
    }
  };
  const uint32_t soff = (uint32_t)((srow % kBlockSize) * kD + scol);
  float4_t kst, vst;
  auto fetch_k = [&]() {
    kst = *reinterpret_cast<const float4_t*>(
        kc + ((int64_t)tbk[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
  };
  auto fetch_v = [&]() {
    vst = *reinterpret_cast<const float4_t*>(
        vc + ((int64_t)tbv[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
  };
  auto stash_k = [&](int buf) {
    uint2 k0, k1, k2;
    split4(kst, k0, k1, k2);
    *reinterpret_cast<uint2*>(&k_lds[buf][0][srow * kKRow + scol]) = k0;
    *reinterpret_cast<uint2*>(&k_lds[buf][1][srow * kKRow + scol]) = k1;
    *reinterpret_cast<uint2*>(&k_lds[buf][2][srow * kKRow + scol]) = k2;
  };
  auto stash_v = [&](int buf, int tk) {
    const int base = kstart + tk * kKT;
    if (base + kKT > hi && base + srow >= hi) vst = float4_t{0, 0, 0, 0};
    uint2 v0, v1, v2;
    split4(vst, v0, v1, v2);
    *reinterpret_cast<uint2*>(&v_lds[buf][0][srow * kVRow + scol]) = v0;
    *reinterpret_cast<uint2*>(&v_lds[buf][1][srow * kVRow + scol]) = v1;
    *reinterpret_cast<uint2*>(&v_lds[buf][2][srow * kVRow + scol]) = v2;
  };

  float4_t acc[kNDT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt) acc[dt] = float4_t{0, 0, 0, 0};
  float m_ref = -INFINITY, neg_m = 0.0f, l_run = 0.0f;
  const float* bias_row = nullptr;
  if (BIAS == 1) {
    // rows past the query set take the wave's first row: they read entries
    // only on chunks every row of the wave sees
    const int tb_row = row_ok ? t_row : w_first;
    bias_row = a.bias_start
                   ? a.attn_bias + a.bias_start[b] + ((int64_t)h * nq + tb_row) * L
                   : a.attn_bias +
                         (((int64_t)b * H + h) * a.max_seq_len + pos0 + tb_row) * a.max_seq_len;
  }
  const bool bias_vec =
      BIAS == 1 &&
      __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(bias_row) & 15) != 0) == 0;
  // a lane's 4 bias entries of each chunk of a tile: chunks inside every
  // row's range in one 16-byte non-temporal load when the rows are 16-byte
  // aligned, others (with a window or chunks) entry by entry with the key
  // clamped into the row's range
  float4_t bcur[2];
  auto load_bias = [&](int tk) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int c0 = kstart + tk * kKT + ch * 16;
      const int j0 = c0 + 4 * g;
      bcur[ch] = float4_t{0, 0, 0, 0};
      if (bias_vec && chunk_whole(c0)) {
        bcur[ch] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(bias_row + j0));
      } else if (kEarly && chunk_live(c0) && bjlo <= bjhi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bcur[ch][r] = bias_row[min(max(j0 + r, bjlo), bjhi)];
      }
    }
  };

  auto qk = [&](auto kb_c, float4_t (&s)[2]) {
    constexpr int kb = decltype(kb_c)::value;
    s[0] = s[1] = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int o = (ch * 16 + c) * kKRow + 16 * g + 8 * st;
        const bf16x8_t k0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][0][o]));
        const bf16x8_t k1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][1][o]));
        const bf16x8_t k2 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[kb][2][o]));
        s[ch] = mfma(k2, qp[0][st], s[ch]);
        s[ch] = mfma(k1, qp[1][st], s[ch]);
        s[ch] = mfma(k0, qp[2][st], s[ch]);
        s[ch] = mfma(k1, qp[0][st], s[ch]);
        s[ch] = mfma(k0, qp[1][st], s[ch]);
        s[ch] = mfma(k0, qp[0][st], s[ch]);
      }
    }
  };

  float4_t s_cur[2];
  s_cur[0] = s_cur[1] = float4_t{0, 0, 0, 0};
  // start-up: the table entries of tiles 0 and 1, then K and V of tile 0
  // and K of tile 1, all in flight together
  if (ntiles > 0) {
    int tb1[2] = {0, 0};
    load_table(tbk, 0);
    if (ntiles > 1) load_table(tb1, 1);
    tbv[0] = tbk[0]; tbv[1] = tbk[1];
    fetch_k();
    fetch_v();
    float4_t k1 = kst;
    if (ntiles > 1) {
      tbk[0] = tb1[0]; tbk[1] = tb1[1];
      k1 = *reinterpret_cast<const float4_t*>(
          kc + ((int64_t)tbk[srow / kBlockSize] * H + h) * (kBlockSize * kD) + soff);
    }
    split_q();
    stash_k(0);
    stash_v(0, 0);
    if (ntiles > 1) {
      kst = k1;
      stash_k(1);
    }
  } else {
    split_q();
  }
  __syncthreads();
  if (ntiles > 0) {
    if (wave_active && wt0 == 0) {
      qk(IntC<0>{}, s_cur);
      if constexpr (BIAS == 1) load_bias(0);
    }
    if (ntiles > 1) {
      tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile 1
      fetch_v();
      if (ntiles > 2) {
        load_table(tbk, 2);
        fetch_k();
        tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile 2
      }
      if (ntiles > 3) load_table(tbk, 3);
    }
  }
  __syncthreads();

  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  // softmax and P.V of tile tk (in the wave's range); NEXT: tile tk + 1 is in
  // the wave's range too, and its products are issued here
  auto body = [&](int tk, auto buf_c, auto next_c) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int base = kstart + tk * kKT;
    float4_t* s = s_cur;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int c0 = base + ch * 16;
      const int j0 = c0 + 4 * g;
      if constexpr (BIAS == 2) {
        // as in the kernel above: one end bucket for a chunk wholly at or
        // beyond the maximum distance from every row of the wave
        if (c0 + 15 - pr0 <= -rel_md || c0 - pr0 - 15 >= rel_md) {
          const float bend = rel_lds[c0 < pr0 ? 3 : 2 * rel_md + 3];
#pragma unroll
          for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + bend;
        } else {
          const int e0 = min(max(j0 - p_row, -rel_md - 3), rel_md) + rel_md + 3;
#pragma unroll
          for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + rel_lds[e0 + r];
        }
      }
      if (chunk_whole(c0)) {   // uniform
        if constexpr (BIAS == 1) {
          if (kEarly || bias_vec) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + bcur[ch][r] * cs;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ch][r] = s[ch][r] + bias_row[j0 + r] * cs;
          }
        }
      } else if (chunk_live(c0)) {
        const int d0 = dq - c0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = d0 - r;
          float x = -INFINITY;
          if (d > dlo && d < dhi) {
            x = s[ch][r];
            if constexpr (BIAS == 1) x = x + (kEarly ? bcur[ch][r] : bias_row[j0 + r]) * cs;
          }
          s[ch][r] = x;
        }
      } else {
        s[ch] = float4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
    float mt = vmax(vmax(vmax(s[0][0], s[0][1]), vmax(s[0][2], s[0][3])),
                    vmax(vmax(s[1][0], s[1][1]), vmax(s[1][2], s[1][3])));
    {
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt),
                                                        __float_as_uint(mt), false, false);
      mt = vmax(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                        __float_as_uint(mt), false, false);
      mt = vmax(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    const bool move = mt > m_ref + 8.0f;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.0f;
      m_ref = move ? mt : m_ref;
      neg_m = move ? -mt : neg_m;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) acc[dt] *= alpha;
    }
    float4_t s_next[2];
    if constexpr (NEXT && kPipe) qk(IntC<buf ^ 1>{}, s_next);
    uint32_t w0[4], w1[4], w2[4];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(s[ch][r] + neg_m);
        l_run += pr[r];
      }
      uint2 a0, a1, a2;
      split4(float4_t{pr[0], pr[1], pr[2], pr[3]}, a0, a1, a2);
      w0[2 * ch] = a0.x; w0[2 * ch + 1] = a0.y;
      w1[2 * ch] = a1.x; w1[2 * ch + 1] = a1.y;
      w2[2 * ch] = a2.x; w2[2 * ch + 1] = a2.y;
    }
    const bf16x8_t p0 = __builtin_bit_cast(bf16x8_t, make_uint4(w0[0], w0[1], w0[2], w0[3]));
    const bf16x8_t p1 = __builtin_bit_cast(bf16x8_t, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    const bf16x8_t p2 = __builtin_bit_cast(bf16x8_t, make_uint4(w2[0], w2[1], w2[2], w2[3]));
#pragma unroll
    for (int dt = 0; dt < kNDT; ++dt) {
      bf16x8_t vv[3];
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint16_t* pp = &v_lds[buf][pl][(4 * g + (c >> 2)) * kVRow + 16 * dt + 4 * (c & 3)];
        const uint2 lo2 = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)pp));
        const uint2 hi2 = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(pp + 16 * kVRow)));
        vv[pl] = __builtin_bit_cast(bf16x8_t, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
      }
      acc[dt] = mfma(vv[2], p0, acc[dt]);
      acc[dt] = mfma(vv[1], p1, acc[dt]);
      acc[dt] = mfma(vv[0], p2, acc[dt]);
      acc[dt] = mfma(vv[1], p0, acc[dt]);
      acc[dt] = mfma(vv[0], p1, acc[dt]);
      acc[dt] = mfma(vv[0], p0, acc[dt]);
    }
    if constexpr (NEXT) {
      if constexpr (kPipe) {
        s_cur[0] = s_next[0];
        s_cur[1] = s_next[1];
      } else {
        qk(IntC<buf ^ 1>{}, s_cur);
        if constexpr (BIAS == 1) load_bias(tk + 1);   // in flight until the next step
      }
    }
  };
  auto tile_step = [&](int tk, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;   // tk & 1
    const bool cur = wave_active && tk >= wt0 && tk <= wt1;            // uniform
    const bool nxt = wave_active && tk + 1 >= wt0 && tk + 1 <= wt1;    // uniform
    if (cur) {
      if (nxt)
        body(tk, buf_c, IntC<1>{});
      else
        body(tk, buf_c, IntC<0>{});
    } else if (nxt) {   // the wave's first tile follows
      qk(IntC<buf ^ 1>{}, s_cur);
      if constexpr (BIAS == 1) load_bias(tk + 1);
    }
    if (tk + 1 < ntiles) {
      // staging as in the kernel above
      if (tk + 2 < ntiles) stash_k(buf);
      stash_v(buf ^ 1, tk + 1);
      if (tk + 2 < ntiles) {
        fetch_v();
        if (tk + 3 < ntiles) {
          fetch_k();
          tbv[0] = tbk[0]; tbv[1] = tbk[1];   // tile k+3
          if (tk + 4 < ntiles) load_table(tbk, tk + 4);
        }
      }
      __syncthreads();
    }
  };
  for (int tk = 0; tk < ntiles; tk += 2) {
    tile_step(tk, IntC<0>{});
    if (tk + 1 < ntiles) tile_step(tk + 1, IntC<1>{});
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* orow = static_cast<float*>(a.out) + ((int64_t)(q0 + t_row) * H + h) * kD;
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
    *reinterpret_cast<float4_t*>(orow + 16 * dt + 4 * g) = acc[dt] * inv;
}

template <int BIAS>
void launch_band(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  if (a.window > 0) {
    if (a.causal)
      hipLaunchKernelGGL((pa_prefill_f32x3_band<BIAS, true, 1>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_f32x3_band<BIAS, false, 1>), grid, block, 0, stream, a);
  } else if (a.chunk > 0) {
    if (a.causal)
      hipLaunchKernelGGL((pa_prefill_f32x3_band<BIAS, true, 2>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_f32x3_band<BIAS, false, 2>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((pa_prefill_f32x3_band<BIAS, true, 0>), grid, block, 0, stream, a);
  }
}

}  // namespace

// Launches at head_dim 64, with a materialised bias, an in-kernel T5 bias or
// none: bidirectional ones without a window or chunks take the first kernel,
// causal, windowed and chunked ones the banded one.
hipError_t launch_prefill_f32x3(PrefillArgs a, hipStream_t stream) {
  a.num_qtiles = (a.max_seq_len + kQT - 1) / kQT;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  const int64_t nwg = (pairs + kXcds - 1) / kXcds * kXcds * a.num_qtiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg), block(kThreads);
  if (a.causal || a.window > 0 || a.chunk > 0) {
    if (a.rel.table)
      launch_band<2>(a, grid, stream);
    else if (a.attn_bias)
      launch_band<1>(a, grid, stream);
    else
      launch_band<0>(a, grid, stream);
  } else if (a.rel.table)
    hipLaunchKernelGGL((pa_prefill_f32x3<2>), grid, block, 0, stream, a);
  else if (a.attn_bias)
    hipLaunchKernelGGL((pa_prefill_f32x3<1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_f32x3<0>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
