// decode_valu.h — decode engine on the vector ALU (fp32 / fp16 / bf16).
//
// Same driver as the matrix-core engine (pa_device.h streams 16-token
// sub-tiles of each piece); this engine loads a sub-tile and folds it into a
// wave's online-softmax state with fp32 arithmetic.
//
// Scores.  The K sub-tile (16 token rows, token-major) is read as 16-byte
// chunks, one per lane per load: a token row spans RL lanes (RL = 16 for
// 16-bit types, 32 for fp32), so one load covers 64/RL tokens.  Each lane
// dots its chunk with the matching chunk of a query head (packed dot2
// instructions with fp32 accumulation for 16-bit types, fp32 FMAs for
// fp32); the RL partial sums of a row are then summed by DPP row moves (and
// one cross-row exchange for fp32), leaving the token's score in all RL
// lanes.  The heads of the group are taken one after another, so only one
// head's scores are live at a time.
//
// Weighted values.  The V group of the sub-tile is stored transposed
// (its 16 tokens of one value dimension contiguous): each 16-byte chunk
// holds E consecutive tokens of one dimension.  The probabilities of the
// sub-tile go through a 16-float per-wave LDS line per head; each lane
// converts its V chunks once, then for each head reads the E probabilities
// it needs and accumulates o[dim] += sum_e p_e v_e for its dimensions; the
// RV lanes sharing a dimension are summed once at the end of the piece.
//
// Register budget: two sub-tiles in flight, the accumulators of the group,
// one head's query chunk, scores and probabilities, and the converted V
// chunks (the query group stays in LDS) fit the 256 VGPRs a wave has at
// two waves per SIMD, with nothing spilled to scratch, for groups of up to
// 4 heads (16-bit types) or 1 head (fp32); larger groups run as several
// virtual groups of the largest built size (the K/V tiles are then read
// once per virtual group).
//
// Online softmax as in the matrix-core engine ("39 · PagedAttention", §2,
// one softmax over all scores, kept as a running max and rescaled sums).
#pragma once

#include "pa_device.h"

namespace pa {

template <class T, int B, int G>
struct ValuEngine {
  static_assert(G >= 1 && G <= (T::kEsize == 4 ? 1 : 4), "group sizes whose state fits the registers without spilling");
  static_assert(B % kSub == 0, "block size must be a multiple of 16");
  static constexpr int E = 16 / T::kEsize;  // elements per 16-byte chunk
  static constexpr int RL = kD / E;         // lanes per K row
  static constexpr int NK = kSub * RL / 64; // K loads per lane per sub-tile
  static constexpr int TPL = 64 / RL;       // tokens per K load
  static constexpr int RV = kSub / E;       // lanes per V dimension row
  static constexpr int NV = kD * RV / 64;   // V loads per lane per sub-tile
  static constexpr int DPL = 64 / RV;       // dimensions per V load
  static constexpr int kTileBytes = B * kD * T::kEsize;

  struct Smem : MergeSmem<T, G> {
    float p[kWaves][G][kSub];  // per-wave probability line of the current sub-tile
  };
  struct Tile {
    uint4 k[NK];
    uint4 v[NV];
  };
  struct Query {
    int p;  // the piece whose staged query group (LDS) the sub-tiles are scored against
  };
  struct State {
    float acc[NV][G];
    float m[G], lsum[G];
  };

  static __device__ __forceinline__ float row_sum(float x) {
    x = row16_sum(x);
    if constexpr (RL == 32) x = sum_xor16(x);
    return x;
  }

  static __device__ __forceinline__ void reset(State& st) {
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int g = 0; g < G; ++g) st.acc[n][g] = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      st.m[g] = -INFINITY;
      st.lsum[g] = 0.f;
    }
  }

  static __device__ __forceinline__ void load_query(const Smem&, int p, Query& q) { q.p = p; }

  // Dot product of a query chunk and a K chunk (E elements), fp32 result.
  static __device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k) {
    if constexpr (T::kCode == F32::kCode) {
      float d = __uint_as_float(q.x) * __uint_as_float(k.x);
      d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
      d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
      return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
    } else if constexpr (T::kCode == BF16::kCode) {
      typedef __bf16 pair __attribute__((ext_vector_type(2)));
      float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pair, q.x),
                                                __builtin_bit_cast(pair, k.x), 0.f, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pair, q.y), __builtin_bit_cast(pair, k.y), d,
                                          false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pair, q.z), __builtin_bit_cast(pair, k.z), d,
                                          false);
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pair, q.w), __builtin_bit_cast(pair, k.w),
                                             d, false);
    } else {
      typedef _Float16 pair __attribute__((ext_vector_type(2)));
      float d = __builtin_amdgcn_fdot2(__builtin_bit_cast(pair, q.x), __builtin_bit_cast(pair, k.x), 0.f,
                                       false);
      d = __builtin_amdgcn_fdot2(__builtin_bit_cast(pair, q.y), __builtin_bit_cast(pair, k.y), d, false);
      d = __builtin_amdgcn_fdot2(__builtin_bit_cast(pair, q.z), __builtin_bit_cast(pair, k.z), d, false);
      return __builtin_amdgcn_fdot2(__builtin_bit_cast(pair, q.w), __builtin_bit_cast(pair, k.w), d, false);
    }
  }

  // The sub-tile starting at slot s16 of physical block `phys`, KV head kvh.
  template <int kPolicy>
  static __device__ __forceinline__ void load_tile(const Args& a, int kvh, int s16, int phys,
                                                   int bytes, Tile& t) {
    const int lane = threadIdx.x & 63, rlane = lane % RL, vlane = lane % RV;
    const int64_t tile = ((int64_t)phys * a.Hp + pool_head(a, kvh)) * kTileBytes;
    const auto rk = tile_rsrc(a.kp, tile, bytes);
    const auto rv = tile_rsrc(a.vp, tile, bytes);
    const int koff = ((lane / RL) * kD + rlane * E) * T::kEsize;    // K bytes of load 0
    const int voff = ((lane / RV) * kSub + vlane * E) * T::kEsize;  // V bytes of load 0
#pragma unroll
    for (int n = 0; n < NK; ++n)
      t.k[n] = tile_load16<kPolicy>(rk, koff + n * TPL * kD * T::kEsize, s16 * kD * T::kEsize);
#pragma unroll
    for (int n = 0; n < NV; ++n)
      t.v[n] = tile_load16<kPolicy>(rv, voff + n * DPL * kSub * T::kEsize, s16 * kD * T::kEsize);
  }

  // Fold a sub-tile whose first `valid` tokens (1 .. 16) are attended into
  // the wave state.
  static __device__ __forceinline__ void compute(const Args& a, Smem& sm, const Query& q, State& st,
                                                 Tile& t, int valid) {
    const int lane = threadIdx.x & 63, rlane = lane % RL, vlane = lane % RV;
    const int wave = uniform(threadIdx.x >> 6);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 qc = sm.q[q.p][g * kD / E + rlane];  // this lane's chunk of head g
      float x[NK];
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        const float d = row_sum(chunk_dot(qc, t.k[n]));
        x[n] = n * TPL + lane / RL < valid ? d * a.scale_log2 : -INFINITY;
      }
      float bm = x[0];
#pragma unroll
      for (int n = 1; n < NK; ++n) bm = fmaxf(bm, x[n]);
      if constexpr (RL == 16) bm = max_xor16(bm);
      bm = max_xor32(bm);
      const float mn = fmaxf(st.m[g], bm);
      const float alpha = fast_exp2(st.m[g] - mn);
      st.m[g] = mn;
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        x[n] = fast_exp2(x[n] - mn);
        ps += x[n];
      }
      st.lsum[g] = st.lsum[g] * alpha + ps;
#pragma unroll
      for (int n = 0; n < NV; ++n) st.acc[n][g] *= alpha;
      // this head's probabilities to the wave's LDS line: one lane per token row writes
      if (rlane == 0) {
#pragma unroll
        for (int n = 0; n < NK; ++n) sm.p[wave][g][n * TPL + lane / RL] = x[n];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float vf[NV][E];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      chunk_to_float<T>(t.v[n], vf[n]);
      if (valid < kSub) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[n][e] = (vlane * E + e < valid) ? vf[n][e] : 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pw[E];
#pragma unroll
      for (int e = 0; e < E; ++e) pw[e] = sm.p[wave][g][vlane * E + e];
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[n][g] = fmaf(pw[e], vf[n][e], st.acc[n][g]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Wave partial -> LDS: sum over the RV lanes of a dimension row and over
  // the token rows.
  static __device__ __forceinline__ void to_lds(Smem& sm, const State& st, int wave) {
    const int lane = threadIdx.x & 63, vlane = lane % RV;
    float acc[NV][G], lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        acc[n][g] = st.acc[n][g] + dpp<kQuadXor1>(st.acc[n][g]);
        if constexpr (RV == 4) acc[n][g] += dpp<kQuadXor2>(acc[n][g]);
      }
      lsum[g] = st.lsum[g];
      if constexpr (RL == 16) lsum[g] = sum_xor16(lsum[g]);
      lsum[g] = sum_xor32(lsum[g]);
    }
    if (vlane == 0) {
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int g = 0; g < G; ++g) sm.o[wave][g][n * DPL + lane / RV] = acc[n][g];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sm.m[wave][g] = st.m[g];
        sm.l[wave][g] = lsum[g];
      }
    }
  }
};

}  // namespace pa
