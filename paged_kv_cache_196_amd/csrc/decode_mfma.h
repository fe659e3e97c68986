// decode_mfma.h — decode engine on the gfx950 matrix cores (fp16 / bf16).
//
// The driver (pa_device.h) streams 16-token sub-tiles of each piece (tokens
// of one (sequence b, KV head)); this engine loads a sub-tile and folds it
// into a wave's online-softmax state.
//
// Per sub-tile the query group of the KV head (G heads, padded to 16 MFMA
// columns) meets the 16 keys as a dense tile:
//   S^T[16 tok][16 heads]  = K[16 tok][128] . Q^T[128][16 heads]
//       4 x v_mfma_f32_16x16x32_{bf16,f16}; A = K rows straight from the
//       token-major K tile, B = the query group (loaded once per piece).
//   O^T[128 dims][16 heads] += V^T[128][16 tok] . P^T[16 tok][16 heads]
//       8 dim tiles x v_mfma_f32_16x16x32_{bf16,f16}; A = the V group of
//       the sub-tile, stored transposed ([128][16]) and read as-is, B = P^T,
//       which is exactly the C-layout of S^T, so the probabilities never
//       leave their registers.
// P is fed as hi + lo halves (p = hi + lo, both in the input type), so
// the weighted sum keeps ~16 mantissa bits instead of the 8 (bf16) or 11
// (fp16) one rounding would leave; this keeps the result within the fp32
// accumulation budget.  Both halves go through one 32-deep product per dim
// tile (each lane's 4 tokens appear twice along K: once against hi, once
// against lo), at the instruction rate of one 16-deep product.
//
// MFMA operand layouts used (wave64, 16x16 tiles; lane = 16*grp + col):
//   A (16 x K): lane holds row `col`, K elements grp*k..grp*k+k-1 (k = K/4)
//   B (K x 16): lane holds column `col`, the same K elements
//   C/D (16 x 16): lane holds column `col`, rows 4*grp .. 4*grp+3
// Only the pairing of A and B K-elements matters for a product, and both
// operands are built with the same (grp, element) -> (dim or token) map.
//
// Softmax statistics follow "39 · PagedAttention", §2 (one softmax over all
// scores) in its online form: a running max m per head, the running sum l
// and the accumulator rescaled by 2^(m_old - m_new) when the max grows.
#pragma once

#include "pa_device.h"

namespace pa {

// kWide: the LDS of the shared-prefix kernel (room for the prefix items'
// 32-column merges, shared_prefix.h); the arithmetic is the same.
template <class T, int B, int G, bool kWide = false>
struct MfmaEngine {
  static_assert(T::kEsize == 2, "matrix-core path takes fp16 / bf16");
  static_assert((G >= 1 && G <= 16) || G == 32 || G == 64,
                "query group padded to 16 MFMA columns, or split into column tiles of 16");
  static_assert(B % kSub == 0, "block size must be a multiple of 16");

  using Smem = MergeSmem<T, G, kWide>;
  static constexpr int NT = kTilesPerWave<G>;  // 16-column tiles each sub-tile is scored against
  using Op8 = typename std::conditional<T::kCode == BF16::kCode, bf16x8, f16x8>::type;
  using Op4 = typename std::conditional<T::kCode == BF16::kCode, bf16x4, f16x4>::type;
  using Elem = typename std::conditional<T::kCode == BF16::kCode, __bf16, _Float16>::type;
  static constexpr int kTileBytes = B * kD * 2;

  struct Tile {
    uint4 k[4];  // K rows: token `col`, dims 32x + 8grp .. +8   (x = 0..3)
    uint2 v[8];  // V^T: dim 16x + col, tokens 4grp .. 4grp+3   (x = 0..7)
  };
  struct Query {
    uint4 op[NT][4];  // B operand of column tile t: head `col` of t, dims 32x + 8grp .. +8
  };
  struct State {
    f32x4 acc[NT][8];  // O^T tile x of column tile t: dims 16x + 4grp .. +4 of its head `col`
    float m[NT];       // running max of that head (base-2 units)
    float lsum[NT];    // this lane's share of the running sum of 2^(s - m)
  };

  static __device__ __forceinline__ f32x4 mma_qk(const uint4& k, const uint4& q, f32x4 c) {
    const Op8 a = __builtin_bit_cast(Op8, k);
    const Op8 b = __builtin_bit_cast(Op8, q);
    if constexpr (T::kCode == BF16::kCode)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }

  // One 32-deep product c += A . B (A: 16 rows x 32, B: 32 x 16 columns,
  // each lane holding its 8 K elements as 16-byte words).
  static __device__ __forceinline__ f32x4 mma_32(const uint4& a, const uint4& b, f32x4 c) {
    if constexpr (T::kCode == BF16::kCode)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(Op8, a),
                                                     __builtin_bit_cast(Op8, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(Op8, a),
                                                    __builtin_bit_cast(Op8, b), c, 0, 0, 0);
  }

  // Two floats rounded to the input type and packed (first in the low half).
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    typedef Elem pair __attribute__((ext_vector_type(2)));
    const pair v = {(Elem)x, (Elem)y};
    return __builtin_bit_cast(uint32_t, v);
  }

  // c += V^T . (P_hi + P_lo)^T for one 16-dim tile in a single 32-deep
  // product: the lane's 8 K elements are its 4 tokens twice, paired with
  // the hi probabilities in the first four and the lo ones in the last four
  // (A = the V chunk repeated, B = phi then plo).
  static __device__ __forceinline__ f32x4 mma_pv2(const uint2& v, const Op4& phi, const Op4& plo,
                                                  f32x4 c) {
    const Op8 a = __builtin_bit_cast(Op8, make_uint4(v.x, v.y, v.x, v.y));
    const uint2 h = __builtin_bit_cast(uint2, phi), l = __builtin_bit_cast(uint2, plo);
    const Op8 b = __builtin_bit_cast(Op8, make_uint4(h.x, h.y, l.x, l.y));
    if constexpr (T::kCode == BF16::kCode)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }

  static __device__ __forceinline__ void reset(State& st) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int x = 0; x < 8; ++x) st.acc[t][x] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m[t] = -INFINITY;
      st.lsum[t] = 0.f;
    }
  }

  // Query group of piece p from its LDS staging (zero columns >= G); a
  // wave of column group c takes heads 32c + 16t + col of its tiles t.
  static __device__ __forceinline__ void load_query(const Smem& sm, int p, Query& q) {
    const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
    const int base = kColGroups<G> > 1 ? (int)(threadIdx.x >> 6) / kColWaves<G> * 32 : 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int head = base + 16 * t + col;
      const int c0 = (head * kD + 8 * grp) * 2 / 16;  // 16-byte chunk of dims 8grp.. of the head
#pragma unroll
      for (int x = 0; x < 4; ++x)
        q.op[t][x] = head < G ? sm.q[p][c0 + 4 * x] : make_uint4(0, 0, 0, 0);
    }
  }

  // The sub-tile starting at slot s16 of physical block `phys`, KV head kvh.
  template <int kPolicy>
  static __device__ __forceinline__ void load_tile(const Args& a, int kvh, int s16, int phys,
                                                   int bytes, Tile& t) {
    const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
    const int64_t tile = ((int64_t)phys * a.Hp + pool_head(a, kvh)) * kTileBytes;
    const auto rk = tile_rsrc(a.kp, tile, bytes);
    const auto rv = tile_rsrc(a.vp, tile, bytes);
    const int koff = (col * kD + 8 * grp) * 2;    // this lane's K bytes inside a sub-tile
    const int voff = (col * kSub + 4 * grp) * 2;  // this lane's V^T bytes inside a group
#pragma unroll
    for (int x = 0; x < 4; ++x) t.k[x] = tile_load16<kPolicy>(rk, koff + 64 * x, s16 * kD * 2);
#pragma unroll
    for (int x = 0; x < 8; ++x) t.v[x] = tile_load8<kPolicy>(rv, voff + 32 * x * kSub, s16 * kD * 2);
  }

  // Fold a sub-tile whose first `valid` tokens (1 .. 16) are attended into
  // the wave state.
  static __device__ __forceinline__ void compute(const Args& a, Smem&, const Query& q, State& st,
                                                 Tile& t, int valid) {
    const int lane = threadIdx.x & 63, grp = lane >> 4;
    Op4 phi[NT], plo[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 4; ++x) s = mma_qk(t.k[x], q.op[ct][x], s);
      float xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = (4 * grp + r < valid) ? s[r] * a.scale_log2 : -INFINITY;
      float bm = fmaxf(fmaxf(xr[0], xr[1]), fmaxf(xr[2], xr[3]));
      bm = max_xor16(bm);
      bm = max_xor32(bm);
      const float mn = fmaxf(st.m[ct], bm);
      if (wave_any(mn > st.m[ct])) {
        // The max grew somewhere in the wave: rescale sums and accumulators
        // (alpha = 1 in lanes whose max did not move).
        const float alpha = fast_exp2(st.m[ct] - mn);
        st.lsum[ct] *= alpha;
#pragma unroll
        for (int x = 0; x < 8; ++x) st.acc[ct][x] *= alpha;
        st.m[ct] = mn;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(xr[r] - st.m[ct]);
      st.lsum[ct] += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        phi[ct][r] = (Elem)p[r];
        plo[ct][r] = (Elem)(p[r] - (float)phi[ct][r]);
      }
    }
    if (valid < kSub) {
      // Slots past the sequence end may hold anything (NaN included):
      // zero them so that 0 * slot cannot poison the product.
      const int nv = valid - 4 * grp;  // valid tokens among this lane's 4
      const uint32_t lo_mask = (nv >= 1 ? 0x0000ffffu : 0u) | (nv >= 2 ? 0xffff0000u : 0u);
      const uint32_t hi_mask = (nv >= 3 ? 0x0000ffffu : 0u) | (nv >= 4 ? 0xffff0000u : 0u);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        t.v[x].x &= lo_mask;
        t.v[x].y &= hi_mask;
      }
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        st.acc[ct][x] = mma_pv2(t.v[x], phi[ct], plo[ct], st.acc[ct][x]);
      }
    }
  }

  // Wave partial of column tile `t` -> LDS (lsum summed over the 4 row
  // groups of each column); a column-split group writes the tile's 16
  // heads at columns 0..15, one tile per merge round.
  static __device__ __forceinline__ void to_lds(Smem& sm, const State& st, int wave, int t = 0) {
    const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
    float lsum = sum_xor16(st.lsum[t]);
    lsum = sum_xor32(lsum);
    if (col < G) {
#pragma unroll
      for (int x = 0; x < 8; ++x)
        *reinterpret_cast<f32x4*>(&sm.o[wave][col][16 * x + 4 * grp]) = st.acc[t][x];
      if (grp == 0) {
        sm.m[wave][col] = st.m[t];
        sm.l[wave][col] = lsum;
      }
    }
  }
};

}  // namespace pa
