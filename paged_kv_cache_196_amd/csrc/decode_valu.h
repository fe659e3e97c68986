// decode_valu.h — decode engine on the vector ALU (fp32 / fp16 / bf16).
//
// Same work split as the matrix-core engine: a piece is logical blocks
// [j0, j1) of one (sequence b, KV head), streamed in 16-token sub-tiles,
// wave w taking sub-tiles w, w+4, ...  Products are fp32 FMAs.
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

  static constexpr int kDepth = 2;  // sub-tiles in flight per wave

  struct Smem : MergeSmem<G> {
    float p[kWaves][G][kSub];
  };

  struct Tile {
    uint4 k[NK];
    uint4 v[NV];
  };

  static __device__ __forceinline__ float row_sum(float x) {
    x = row16_sum(x);
    if constexpr (RL == 32) x = sum_xor16(x);
    return x;
  }

  static __device__ void piece(const Args& a, Smem& sm, const Piece& pc) {
    const int b = pc.b, kvh = pc.kvh, j0 = pc.j0, j1 = pc.j1, L = pc.L;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int rlane = lane % RL;  // position inside a K row
    const int vlane = lane % RV;  // position inside a V dimension row

    // This lane's slice of every query head of the group.
    float qf[G][E];
    {
      const char* qb = static_cast<const char*>(a.q);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t off = (((int64_t)b * a.Hq + (int64_t)kvh * G + g) * kD + rlane * E) * T::kEsize;
        const uint4 c = *reinterpret_cast<const uint4*>(qb + off);
        chunk_to_float<T>(c, qf[g]);
      }
    }

    const int tok_begin = j0 * B;
    const int tok_end = min(j1 * B, L);
    const int nsub = (tok_end - tok_begin + kSub - 1) / kSub;
    const const_i32_ptr row = as_constant(a.bt + (int64_t)b * a.mbs);

    auto phys_of = [&](int i) { return row[(tok_begin + kSub * i) / B]; };
    constexpr int kTileBytes = B * kD * T::kEsize;
    const int koff = ((lane / RL) * kD + rlane * E) * T::kEsize;  // K bytes of load 0
    const int voff = ((lane / RV) * kSub + vlane * E) * T::kEsize;  // V bytes of load 0
    auto load = [&](int i, int phys, Tile& t) {
      const int s16 = (tok_begin + kSub * i) % B;
      const int64_t tile = ((int64_t)phys * a.Hkv + kvh) * kTileBytes;
      const auto rk = tile_rsrc(a.kp, tile, kTileBytes);
      const auto rv = tile_rsrc(a.vp, tile, kTileBytes);
#pragma unroll
      for (int n = 0; n < NK; ++n)
        t.k[n] = tile_load16(rk, koff + n * TPL * kD * T::kEsize, s16 * kD * T::kEsize);
#pragma unroll
      for (int n = 0; n < NV; ++n)
        t.v[n] = tile_load16(rv, voff + n * DPL * kSub * T::kEsize, s16 * kD * T::kEsize);
    };

    float acc[NV][G];
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int g = 0; g < G; ++g) acc[n][g] = 0.f;
    float m[G], lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      lsum[g] = 0.f;
    }

    auto compute = [&](Tile& t, int i) {
      const int valid = tok_end - (tok_begin + kSub * i);  // >= 1
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
          for (int e = 0; e < E; ++e) d = fmaf(qf[g][e], kf[e], d);
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
        const float mn = fmaxf(m[g], bm);
        const float alpha = fast_exp2(m[g] - mn);
        m[g] = mn;
        float ps = 0.f;
#pragma unroll
        for (int n = 0; n < NK; ++n) {
          x[n][g] = fast_exp2(x[n][g] - mn);
          ps += x[n][g];
        }
        lsum[g] = lsum[g] * alpha + ps;
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[n][g] *= alpha;
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
          for (int e = 0; e < E; ++e) acc[n][g] = fmaf(pw[g][e], vf[e], acc[n][g]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if (wave < nsub)
      stream_subtiles<kDepth, Tile>(
          wave, wave + kWaves * ((nsub - 1 - wave) / kWaves), phys_of, load, compute, [&](int i) {
            set_priority_for_progress(pc.done_before + (kSub * i) / B, pc.chunk_len);
          });

    // Sum over the RV lanes of a dimension row and over the token rows.
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        acc[n][g] += dpp<kQuadXor1>(acc[n][g]);
        if constexpr (RV == 4) acc[n][g] += dpp<kQuadXor2>(acc[n][g]);
      }
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
        sm.m[wave][g] = m[g];
        sm.l[wave][g] = lsum[g];
      }
    }
    __syncthreads();
    emit_piece<T, G>(a, sm, pc);
    __syncthreads();
  }
};

}  // namespace pa
