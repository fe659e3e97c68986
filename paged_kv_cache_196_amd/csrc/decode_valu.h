// decode_valu.h — decode engine on the vector ALU (fp32 / fp16 / bf16).
//
// Same driver as the matrix-core engine (pa_device.h streams 16-token
// sub-tiles of each piece); this engine loads a sub-tile and folds it into a
// wave's online-softmax state with fp32 FMAs.
//
// Scores.  The K sub-tile (16 token rows, token-major) is read as 16-byte
// chunks, one per lane per load: a token row spans RL lanes (RL = 16 for
// 16-bit types, 32 for fp32), so one load covers 64/RL tokens.  Each lane
// dots its chunk with the matching slice of every query head of the group;
// the RL partial sums of a row are then summed by DPP row moves (and one
// cross-row exchange for fp32), leaving the token's score in all RL lanes.
//
// Weighted values.  The V group of the sub-tile is stored transposed
// (its 16 tokens of one value dimension contiguous): each 16-byte chunk
// holds E consecutive tokens of one dimension.  The probabilities of the sub-tile go through a 16-float
// per-wave LDS line so every lane can read the E it needs; each lane then
// accumulates o[dim] += sum_e p_e v_e for its dimensions, and the RV lanes
// sharing a dimension are summed once at the end of the piece.
//
// Online softmax as in the matrix-core engine ("39 · PagedAttention", §2,
// one softmax over all scores, kept as a running max and rescaled sums).
#pragma once

#include "pa_device.h"

namespace pa {

template <class T, int B, int G>
struct ValuEngine {
  static_assert(G >= 1 && G <= 8, "vector path holds the whole group in registers");
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
    float f[G][E];  // this lane's slice of every query head of the group
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

  static __device__ __forceinline__ void load_query(const Smem& sm, int p, Query& q) {
    const int rlane = (threadIdx.x & 63) % RL;
#pragma unroll
    for (int g = 0; g < G; ++g) chunk_to_float<T>(sm.q[p][g * kD / E + rlane], q.f[g]);
  }

  // The sub-tile starting at slot s16 of physical block `phys`, KV head kvh.
  template <int kPolicy>
  static __device__ __forceinline__ void load_tile(const Args& a, int kvh, int s16, int phys,
                                                   int bytes, Tile& t) {
    const int lane = threadIdx.x & 63, rlane = lane % RL, vlane = lane % RV;
    const int64_t tile = ((int64_t)phys * a.Hkv + kvh) * kTileBytes;
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
    float x[NK][G];
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      float kf[E];
      chunk_to_float<T>(t.k[n], kf);
      const bool ok = n * TPL + lane / RL < valid;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(q.f[g][e], kf[e], d);
        d = row_sum(d);
        x[n][g] = ok ? d * a.scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = x[0][g];
#pragma unroll
      for (int n = 1; n < NK; ++n) bm = fmaxf(bm, x[n][g]);
      if constexpr (RL == 16) bm = max_xor16(bm);
      bm = max_xor32(bm);
      const float mn = fmaxf(st.m[g], bm);
      const float alpha = fast_exp2(st.m[g] - mn);
      st.m[g] = mn;
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        x[n][g] = fast_exp2(x[n][g] - mn);
        ps += x[n][g];
      }
      st.lsum[g] = st.lsum[g] * alpha + ps;
#pragma unroll
      for (int n = 0; n < NV; ++n) st.acc[n][g] *= alpha;
    }
    // Probabilities to the wave's LDS line: one lane per token row writes.
    if (rlane == 0) {
#pragma unroll
      for (int n = 0; n < NK; ++n)
#pragma unroll
        for (int g = 0; g < G; ++g) sm.p[wave][g][n * TPL + lane / RL] = x[n][g];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pw[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) pw[g][e] = sm.p[wave][g][vlane * E + e];
    const bool tail = valid < kSub;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      float vf[E];
      chunk_to_float<T>(t.v[n], vf);
      if (tail) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = (vlane * E + e < valid) ? vf[e] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[n][g] = fmaf(pw[g][e], vf[e], st.acc[n][g]);
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
