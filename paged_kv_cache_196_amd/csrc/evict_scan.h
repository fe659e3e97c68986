// evict_scan.h — gfx950 kernels for block-wise eviction scoring over the
// paged cache ("PagedEviction: Structured Block-wise KV Cache Pruning for
// Efficient Large Language Model Inference", the review's "Core claim" and
// "What carries the argument").
//
// A token's importance is the ratio of its value norm to its key norm,
// S_t = ||V_t||_2 / ||K_t||_2, read straight from the cached rows (no
// attention scores); a block's score is the mean of S_t over its tokens;
// during decode, when a sequence's most recent block has just filled
// (L % B == 0), the block with the lowest score is the one to evict.  The
// norms run over the token's whole key (value) row of the layer: every KV
// head, head_dim elements each.
//
// block_score_kernel: one wave per (sequence, full logical block).  It reads
// the block's K and V tiles of every KV head (each one contiguous burst,
// 16 bytes per lane per load, streaming cache policy: read once), squares
// and sums in fp32:
//   K tile rows are token-major, so a load's 16-byte chunks of one row sit
//   in consecutive lanes and a DPP row reduction (plus one xor-16 step for
//   fp32 rows) gives the row's sum of squares;
//   V groups are transposed (16 tokens of one dimension contiguous), so a
//   lane's chunk holds E consecutive tokens of one dimension; lanes with the
//   same token slots are summed with xor butterflies.
// Lane t < 16 then gathers token t's two sums of every 16-token sub-tile,
// forms sqrt(vv) / sqrt(kk), and a row reduction gives the block mean.
//
// evict_choice_kernel: one wave per sequence, arg-min over its block scores
// (lowest score, then lowest block index).
#pragma once

#include "kernel_args.h"
#include "pa_device.h"

namespace pa {


// Sum of squares of the elements of one 16-byte chunk.
template <class T>
__device__ __forceinline__ float chunk_sumsq(const uint4& c) {
  float f[16 / T::kEsize];
  chunk_to_float<T>(c, f);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16 / T::kEsize; ++e) s += f[e] * f[e];
  return s;
}

// Grid: (ceil(mbs / kAuxWaves), S) workgroups of kAuxThreads; wave -> block
// j = blockIdx.x * kAuxWaves + wave of sequence blockIdx.y.  Entries of blocks
// that are not full (j >= L / B) are set to NaN.
template <class T, int B>
__global__ __launch_bounds__(kAuxThreads) void block_score_kernel(ScoreArgs a) {
  constexpr int E = 16 / T::kEsize;         // elements per 16-byte chunk
  constexpr int CPR = kD * T::kEsize / 16;  // chunks per key row: 16 or 32
  constexpr int TPL = 64 / CPR;             // key rows per wave load: 4 or 2
  constexpr int NL = kSub / TPL;            // wave loads per 16-token sub-tile (K and V alike)
  constexpr int NS = B / kSub;              // sub-tiles per block
  constexpr int VR = kSub / E;              // lanes whose V chunks hold different tokens
  constexpr int64_t kSubBytes = (int64_t)kSub * kD * T::kEsize;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int j = uniform(blockIdx.x * kAuxWaves + (threadIdx.x >> 6));
  if (j >= a.mbs) return;
  const int L = as_constant(a.lens)[b];
  float* out = a.scores + (int64_t)b * a.mbs + j;
  if (j >= L / B) {
    if (lane == 0) *out = __builtin_nanf("");
    return;
  }
  const int phys = as_constant(a.bt + (int64_t)b * a.mbs)[j];
  float kk[NS][NL], vv[NS][E];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int n = 0; n < NL; ++n) kk[s][n] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) vv[s][e] = 0.f;
  }
  for (int h = 0; h < a.Hkv; ++h) {
    // each tile is read once: streaming-policy buffer loads, resource = the tile
    const int64_t tile = ((int64_t)phys * a.Hkv + uniform(h)) * B * kD * T::kEsize;  // bytes
    const auto rk = tile_rsrc(a.kp, tile, B * kD * T::kEsize);
    const auto rv = tile_rsrc(a.vp, tile, B * kD * T::kEsize);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 kc[NL], vc[NL];
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        kc[n] = tile_load16<kStreamPolicy>(rk, s * (int)kSubBytes + (lane + 64 * n) * 16, 0);
        vc[n] = tile_load16<kStreamPolicy>(rv, s * (int)kSubBytes + (lane + 64 * n) * 16, 0);
      }
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        kk[s][n] += chunk_sumsq<T>(kc[n]);  // row lane / CPR + n * TPL
        float f[E];
        chunk_to_float<T>(vc[n], f);        // tokens (lane * E) % 16 .. + E, one dimension
#pragma unroll
        for (int e = 0; e < E; ++e) vv[s][e] += f[e] * f[e];
      }
    }
  }
  // Whole-row sums: K over the CPR lanes of a row, V over the lanes that
  // hold the same token slots (lane % VR).
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      float x = row16_sum(kk[s][n]);
      if constexpr (CPR == 32) x += xor_lanes(x, 16);
      kk[s][n] = x;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = vv[s][e];
#pragma unroll
      for (int m = VR; m < 64; m <<= 1) x += xor_lanes(x, m);
      vv[s][e] = x;
    }
  }
  // Lane t (< 16) takes token t of every sub-tile: its key sum sits in lane
  // (t % TPL) * CPR as kk[s][t / TPL], its value sum in lane t / E as vv[s][t % E].
  const int t = lane & 15;
  float ratio_sum = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float ksum = 0.f, vsum = 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const float x = __shfl(kk[s][n], (t % TPL) * CPR);
      if (n == t / TPL) ksum = x;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = __shfl(vv[s][e], t / E);
      if (e == t % E) vsum = x;
    }
    ratio_sum += __builtin_sqrtf(vsum) / __builtin_sqrtf(ksum);
  }
  // lanes 16..63 repeat lanes 0..15; row 0 holds the 16 distinct tokens
  const float total = row16_sum(ratio_sum);
  if (lane == 0) *out = total / (float)B;
}

// Grid: ceil(S / kAuxWaves) workgroups; wave -> sequence.  evict[b] = arg-min
// of scores[b][0 .. L/B) when L > 0 and L % B == 0, else -1.
__global__ __launch_bounds__(kAuxThreads) void evict_choice_kernel(ScoreArgs a, int B) {
  const int lane = threadIdx.x & 63;
  const int b = uniform(blockIdx.x * kAuxWaves + (threadIdx.x >> 6));
  if (b >= a.S) return;
  const int L = as_constant(a.lens)[b];
  if (L <= 0 || L % B != 0) {
    if (lane == 0) a.evict[b] = -1;
    return;
  }
  const int n = L / B;
  const float* sc = a.scores + (int64_t)b * a.mbs;
  float best = INFINITY;
  int arg = 0x7fffffff;
  for (int j = lane; j < n; j += 64) {
    const float x = sc[j];
    if (x < best) {  // first j of the lane's strided run wins ties
      best = x;
      arg = j;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float ob = xor_lanes(best, m);
    const int oa = __shfl_xor(arg, m);
    if (ob < best || (ob == best && oa < arg)) {
      best = ob;
      arg = oa;
    }
  }
  if (lane == 0) a.evict[b] = arg == 0x7fffffff ? 0 : arg;
}

}  // namespace pa
