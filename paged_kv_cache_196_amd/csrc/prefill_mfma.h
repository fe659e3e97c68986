// prefill_mfma.h — causal paged prefill on the gfx950 matrix cores
// (fp16 / bf16).
//
// Prefill scores many query positions of a request against its cache, whose
// length differs from the number of queries ("FlashAttention vs
// PagedAttention", "How prefill and decode change the diagnosis"); every
// query reads exactly its own sequence's pages through the block table, and
// masking a query to its own keys leaves exact attention unchanged ("Paging
// the KV cache with a fused mask", "What carries the argument" and its list
// of assumptions).
//
// Convention: sequence b contributes n_b = q_start[b+1] - q_start[b] query
// rows, its newest n_b tokens, already written to the cache; row i sits at
// position p = L_b - n_b + i and attends tokens 0 .. p.  n_b = L_b is a whole
// prompt, 1 < n_b < L_b a chunk of one (chunked prefill).
//
// Work item: one wave per (sequence b, KV head, kPrefillTiles column tiles).
// A column tile holds R = 16 / G consecutive query rows times the G query
// heads of the KV head: 16 MFMA columns, column c = (row c / G, head c % G),
// each with its own causal limit.  The wave walks 16-token sub-tiles from
// token 0 up to its largest position; every loaded sub-tile serves all of
// its column tiles:
//   S^T[16 tok][16 cols] = K[16][128] . Q^T[128][16]   4 x mfma 16x16x32
//   O^T[128][16 cols]   += V^T[128][16] . P^T[16][16]  8 dim tiles x mfma 16x16x32 (hi + lo P)
// (operand layouts and the hi + lo split of P as in the decode engine), with
// a running max and sum per column.  The waves of one (b, KV head) read the
// same K/V tiles, through L2 (cached load policy).  Waves with later rows
// (longer) are issued first, across the whole batch.
#pragma once

#include "decode_mfma.h"
#include "kernel_args.h"
#include "pa_device.h"

namespace pa {


// Grid: ceil(tiles * S * Hkv / kAuxWaves) workgroups of kAuxThreads; `tiles`
// counts groups of kPrefillTiles column tiles.  Items run (column group,
// sequence, KV head) with the column group slowest and reversed, so the
// longest rows of the whole batch are issued first and the shortest last.
template <class T, int B, int G>
__global__ __launch_bounds__(kAuxThreads) void prefill_kernel(PrefillArgs a) {
  using M = MfmaEngine<T, B, G>;
  using Op4 = typename M::Op4;
  using Elem = typename M::Elem;
  constexpr int NT = kPrefillTiles;
  constexpr int R = kSub / G;  // query rows per column tile
  constexpr int kTileBytes = B * kD * 2;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int item = uniform(blockIdx.x * kAuxWaves + (threadIdx.x >> 6));
  if (item >= a.tiles * a.S * a.Hkv) return;
  const int ct0 = (a.tiles - 1 - item / (a.S * a.Hkv)) * NT;  // longest rows of the whole batch first
  const int b = (item / a.Hkv) % a.S;
  const int kvh = item % a.Hkv;
  const int q0 = as_constant(a.qs)[b];
  const int n = as_constant(a.qs)[b + 1] - q0;
  const int L = as_constant(a.lens)[b];
  if (n <= 0 || n > L || ct0 * R >= n) return;
  const int head = kvh * G + col % G;
  const int last = L - n + min(n, (ct0 + NT) * R) - 1;  // largest position among the wave's rows

  int row[NT], pos[NT];
  uint4 qop[NT][4];  // query operand of tile t: column col, dims 32x + 8grp .. +8
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    row[t] = (ct0 + t) * R + col / G;
    const bool live = row[t] < n;
    pos[t] = live ? L - n + row[t] : 0;  // padding columns attend token 0 with a zero query
    // padding columns address row 0 of the sequence, which exists, and load nothing
    const int qrow = q0 + (live ? row[t] : 0);
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        static_cast<const char*>(a.q) + (((int64_t)qrow * a.Hq + head) * kD + 8 * grp) * 2);
#pragma unroll
    for (int x = 0; x < 4; ++x) qop[t][x] = live ? qsrc[4 * x] : make_uint4(0, 0, 0, 0);
  }

  f32x4 acc[NT][8];
  float m[NT], lsum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[t][x] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    lsum[t] = 0.f;
  }

  const const_i32_ptr row_bt = as_constant(a.bt + (int64_t)b * a.mbs);
  const int koff = (col * kD + 8 * grp) * 2;
  const int voff = (col * kSub + 4 * grp) * 2;
  const int nsub = last / kSub + 1;
  for (int j = 0; j < nsub; ++j) {
    const int tok0 = j * kSub;
    const int phys = row_bt[tok0 / B];
    const int64_t tile = ((int64_t)phys * a.Hp + pool_head(a, kvh)) * kTileBytes;
    const auto rk = tile_rsrc(a.kp, tile, kTileBytes);
    const auto rv = tile_rsrc(a.vp, tile, kTileBytes);
    const int soff = (tok0 % B) * kD * 2;
    uint4 k[4];
    uint2 v[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) k[x] = tile_load16<kCachedPolicy>(rk, koff + 64 * x, soff);
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = tile_load8<kCachedPolicy>(rv, voff + 32 * x * kSub, soff);
    const int valid = last - tok0 + 1;  // tokens of this sub-tile that any column attends
    if (valid < kSub) {
      // Slots past the wave's last position may lie past the sequence end
      // and hold anything (NaN included): zero them so 0 * slot stays 0.
      const int nv = valid - 4 * grp;
      const uint32_t lo_mask = (nv >= 1 ? 0x0000ffffu : 0u) | (nv >= 2 ? 0xffff0000u : 0u);
      const uint32_t hi_mask = (nv >= 3 ? 0x0000ffffu : 0u) | (nv >= 4 ? 0xffff0000u : 0u);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        v[x].x &= lo_mask;
        v[x].y &= hi_mask;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 4; ++x) s = M::mma_qk(k[x], qop[t][x], s);
      float xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xr[r] = (tok0 + 4 * grp + r <= pos[t]) ? s[r] * a.scale_log2 : -INFINITY;
      float bm = fmaxf(fmaxf(xr[0], xr[1]), fmaxf(xr[2], xr[3]));
      bm = max_xor16(bm);
      bm = max_xor32(bm);
      // Token 0 is in sub-tile 0 and every column attends it, so m is
      // finite from the first sub-tile on.
      const float mn = fmaxf(m[t], bm);
      if (wave_any(mn > m[t])) {
        // some column's max grew: rescale (alpha = 1 where it did not)
        const float alpha = fast_exp2(m[t] - mn);
        lsum[t] *= alpha;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[t][x] *= alpha;
        m[t] = mn;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(xr[r] - m[t]);
      lsum[t] += (p[0] + p[1]) + (p[2] + p[3]);
      Op4 phi, plo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        phi[r] = (Elem)p[r];
        plo[r] = (Elem)(p[r] - (float)phi[r]);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        acc[t][x] = M::mma_pv2(v[x], phi, plo, acc[t][x]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float l = sum_xor16(lsum[t]);
    l = sum_xor32(l);
    if (row[t] < n) {
      const float inv = 1.f / l;
      const int64_t base = ((int64_t)(q0 + row[t]) * a.Hq + head) * kD + 4 * grp;
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_out<T>(a.out, base + 16 * x + r, acc[t][x][r] * inv, a.out_f32);
    }
  }
}

}  // namespace pa
