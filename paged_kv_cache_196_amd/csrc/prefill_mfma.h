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
// Work item: one workgroup of kWaves waves per (sequence b, KV head, block
// of rows); wave w takes kPrefillTiles column tiles of the block.  A column
// tile holds R = 16 / G consecutive query rows times the G query heads of
// the KV head: 16 MFMA columns, column c = (row c / G, head c % G), each
// with its own causal limit.  The workgroup walks the keys in 64-token
// steps of four 16-token K/V sub-tiles from token 0 up to its largest
// position; each sub-tile is read from memory once per workgroup (one
// 16-byte K and one V load per thread, one step ahead), staged in a
// double-buffered LDS stage and read from there by every wave that still
// has rows attending it:
//   S^T[16 tok][16 cols] = K[16][128] . Q^T[128][16]        4 x mfma 16x16x32 per sub-tile
//   O^T[128][16 cols]   += V^T[128][32] . P^T[32][16]        8 dim tiles x mfma 16x16x32 per
//                                                            sub-tile pair (fp16 V and P; see
//                                                            the weighted-value modes below)
// (operand layouts as in the decode engine), with a running max and sum per
// column.  Workgroups run longest rows first across the batch, and the
// blocks of one (sequence, KV head) go to one XCD (workgroup i runs on XCD
// i mod 8), so they share its L2.  Finished tiles leave through LDS as
// whole 16-byte chunks (prefill_store_tiles).
#pragma once

#include "decode_mfma.h"
#include "kernel_args.h"
#include "pa_device.h"

#include <type_traits>

namespace pa {


constexpr int kPrefillStepSub = 4;           // 16-token sub-tiles per step (one softmax update)
constexpr int kPrefillKRow = kD * 2 + 16;     // LDS bytes per K row (padded: rows 4 banks apart)
constexpr int kPrefillKBytes = kSub * kPrefillKRow;
// A pair of sub-tiles (2h, 2h + 1) in LDS: the K rows of both, then their
// V^T as 16-byte entries in the order [dim / 16][token quarter][dim % 16],
// entry = 4 tokens of one dim from sub-tile 2h, then the same 4 tokens'
// places in 2h + 1: exactly the A operand of one 32-deep weighted-value
// product, so a lane reads it with one 16-byte load, and the 16 lanes of
// one LDS cycle (one token quarter, 16 dims) read 256 contiguous bytes.
constexpr int kPrefillVPair = 2 * kSub * kD * 2;
constexpr int kPrefillPair = 2 * kPrefillKBytes + kPrefillVPair;
static_assert(kPrefillThreads * 16 == kSub * kD * 2, "one K and one V chunk per thread per sub-tile");

// Reference-max slack of the prefill's lazy rescaling (log2 units).
constexpr float kPrefillSlack = 8.f;
static_assert(kPrefillStepSub % 2 == 0, "weighted values take sub-tiles in pairs");

// Zero the V^T entries of tokens past the valid ones in the 8 dim tiles
// of a pair entry: nv0 / nv1 = valid tokens among this lane's 4 of
// sub-tile 2h (halves x, y) / of 2h + 1 (halves z, w).
__device__ __forceinline__ void v_tail_mask(uint4 (&v)[8], int nv0, int nv1) {
  const uint32_t m0 = (nv0 >= 1 ? 0x0000ffffu : 0u) | (nv0 >= 2 ? 0xffff0000u : 0u);
  const uint32_t m1 = (nv0 >= 3 ? 0x0000ffffu : 0u) | (nv0 >= 4 ? 0xffff0000u : 0u);
  const uint32_t m2 = (nv1 >= 1 ? 0x0000ffffu : 0u) | (nv1 >= 2 ? 0xffff0000u : 0u);
  const uint32_t m3 = (nv1 >= 3 ? 0x0000ffffu : 0u) | (nv1 >= 4 ? 0xffff0000u : 0u);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    v[x].x &= m0;
    v[x].y &= m1;
    v[x].z &= m2;
    v[x].w &= m3;
  }
}

// How the weighted values take V and P.  P rounded to bf16 alone (8 bits)
// is not enough: the worst error in a CPU simulation of 2048-token causal
// prompts (N(0,1) data, K scaled up to 2x) reached 2.4-3.9e-3, over the
// 2e-3 bar, even with the sum taken over the rounded P.  P rounded to fp16
// alone (11 bits), with the sum over the same rounded values, gave 7.2e-4
// on fp16 data and 7.4e-4 on bf16 data.  So:
//  kPvF16   fp16 inputs: V as stored, P rounded to fp16, one product per
//           pair of sub-tiles;
//  kPvConv  bf16 inputs: V converted to fp16 as it is staged (exact for
//           every bf16 value of magnitude in [2^-17, 2^16); smaller ones
//           move by less than 2^-24), then as kPvF16.  A workgroup that
//           stages a V value of magnitude 2^16 or more (beyond fp16) reruns
//           with kPvSplit;
//  kPvSplit bf16: V as stored, P as hi + lo (two products per pair).
constexpr int kPvF16 = 0, kPvConv = 1, kPvSplit = 2;
constexpr float kPvConvLimit = 65536.f;  // smallest bf16 magnitude fp16 cannot hold

// Two bf16 values (low half first) as two fp16 values, and the larger
// magnitude folded into vmax (NaN ignored).  Round toward zero: every value
// the conversion must keep is representable, so the mode does not matter.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float& vmax) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  vmax = fmaxf(fmaxf(vmax, fabsf(lo)), fabsf(hi));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// bf16: probabilities p0, p1 as hi and lo pairs, p ~= hi + lo: hi is p with
// its low 16 bits cut off (the upper halves of both, one byte permute), lo
// the exact remainder rounded to bf16; p <= 2^8 here and |lo| < 2^-7 p, so
// the pair keeps about 16 bits.
__device__ __forceinline__ void split_pair_bf16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 pair __attribute__((ext_vector_type(2)));
  const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
  hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
  const pair r = {(__bf16)(p0 - __uint_as_float(b0 & 0xffff0000u)),
                  (__bf16)(p1 - __uint_as_float(b1 & 0xffff0000u))};
  lo = __builtin_bit_cast(uint32_t, r);
}

// A wave's finished column tiles to out, through LDS: the scattered
// per-lane elements (4 consecutive dims of one column per 16-byte chunk)
// are written to the wave's LDS region `buf` as [column][dim] rows, then
// read back as 16-byte chunks in output order, so every global store is a
// whole 16-byte chunk and consecutive lanes write consecutive chunks (the
// G heads of a row are contiguous).  buf: kPrefillOutBytes bytes, 16-byte
// aligned, private to the wave; every wave of the workgroup calls this
// (it holds workgroup barriers).  inv[t] = 1 / l of the lane's column.
constexpr int kPrefillOutRow = kD * 4 + 16;  // fp32 row, padded: rows 4 banks apart
constexpr int kPrefillOutBytes = kSub * kPrefillOutRow;

template <class T, int G, int NT>
__device__ __forceinline__ void prefill_store_tiles(const PrefillArgs& a, unsigned char* buf,
                                                    const f32x4 (&acc)[NT][8], const float (&inv)[NT],
                                                    int ct0, int n, int q0, int kvh) {
  constexpr int R = kSub / G;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int esz = a.out_f32 ? 4 : 2;
  const int row_bytes = kD * esz;              // one column's output
  const int stride = row_bytes + 16;           // its padded LDS row
  const int cpc = row_bytes / 16;              // 16-byte chunks per column
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const f32x4 v = acc[t][x] * inv[t];
      unsigned char* dst = buf + col * stride + (16 * x + 4 * grp) * esz;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
        typedef typename std::conditional<T::kCode == BF16::kCode, __bf16, _Float16>::type E;
        typedef E e4 __attribute__((ext_vector_type(4)));
        const e4 h = {(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, h);
      }
    }
    __syncthreads();
    for (int id = lane; id < kSub * cpc; id += 64) {
      const int c = id / cpc, k = id % cpc;
      const int r = (ct0 + t) * R + c / G;
      if (r < n) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + c * stride + k * 16);
        const int64_t o = ((int64_t)(q0 + r) * a.Hq + kvh * G + c % G) * row_bytes + k * 16;
        // written once and not read again here: streaming stores (same-box
        // A/B on the 8 x 2048 prompt batch: 393 -> 386 us per call)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<char*>(a.out) + o));
      }
    }
    __syncthreads();
  }
}

// Rows of one workgroup's block for group size G.
template <int G>
constexpr int prefill_rows_per_block() {
  return kPrefillWaves * kPrefillTiles * (kSub / G);
}

// Grid: 8 * ceil(S * Hkv / 8) * tiles workgroups of kPrefillThreads, `tiles` the
// row blocks of the longest query set.  Workgroup i runs on XCD x = i % 8
// and takes the (sequence, KV head) pairs x, x + 8, ... (pair = b * Hkv +
// kvh) in two halves, within a half with its row block slowest and
// reversed, so each XCD works the longest rows of half its pairs first.
//
// The keys go by steps of kPrefillStepSub sub-tiles (64 tokens): the step's
// scores of every column tile first (independent 4-deep products per
// sub-tile), one softmax update per column tile for the whole step, then
// the weighted values (8-deep chains per dim tile across the step), so the
// matrix cores see long runs of independent products between the
// reductions.
template <class T, int B, int G>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a) {
  using M = MfmaEngine<T, B, G>;
  using Op4 = typename M::Op4;
  using Elem = typename M::Elem;
  constexpr int NT = kPrefillTiles;
  constexpr int KB = kPrefillStepSub;
  constexpr int R = kSub / G;  // query rows per column tile
  constexpr int kRowsBlock = prefill_rows_per_block<G>();
  constexpr int kTileBytes = B * kD * 2;
  constexpr int kStep = KB * kSub;  // tokens per step
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  __shared__ __align__(16) unsigned char stage[2][KB / 2][kPrefillPair];

  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int P = a.S * a.Hkv;
  const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
  const int px = (P - xcd + 7) / 8;  // pairs of this XCD
  if (k >= px * a.tiles) return;
  // The XCD's pairs in two halves, each with its row blocks longest
  // first: the K/V its workgroups stream at a time is half as large, so
  // more of it stays in the XCD's L2.
  const int hp = (px + 1) / 2, h1 = k >= hp * a.tiles ? 1 : 0;
  const int kk = h1 ? k - hp * a.tiles : k, pn = h1 ? px - hp : hp;
  const int rb = a.tiles - 1 - kk / pn;
  const int pair = xcd + 8 * (h1 * hp + kk % pn);
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int q0 = as_constant(a.qs)[b];
  const int n = as_constant(a.qs)[b + 1] - q0;
  const int L = as_constant(a.lens)[b];
  if (n <= 0 || n > L || rb * kRowsBlock >= n) return;  // uniform over the workgroup
  const int head = kvh * G + col % G;
  const int ct0 = (rb * kPrefillWaves + wave) * NT;  // this wave's first column tile
  // largest position among the wave's rows (-1: none) and the workgroup's
  const int last = ct0 * R < n ? L - n + min(n, (ct0 + NT) * R) - 1 : -1;
  const int last_blk = L - n + min(n, (rb + 1) * kRowsBlock) - 1;

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

  // Scores are scaled by c2 = |scale log2 e|; a negative scale flips the
  // query's sign bits instead (the products then come out negated exactly).
  const float c2 = fabsf(a.scale_log2);
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        qop[t][x].x ^= 0x80008000u; qop[t][x].y ^= 0x80008000u; qop[t][x].z ^= 0x80008000u; qop[t][x].w ^= 0x80008000u;
      }
  }
  f32x4 acc[NT][8];
  float m[NT], lsum[NT];

  // This thread's 2 x 16 bytes of every sub-tile: K chunk c (token c / 16,
  // dims 8 (c % 16) ..), c = threadIdx.x, and the V^T chunk of dim vdim,
  // tokens 8 vh .. + 8 (token quarters 2 vh and 2 vh + 1), with 16
  // consecutive lanes on 16 consecutive dims of one quarter (their LDS
  // stores hit distinct banks); where they go in the pair's stage.
  const int c16 = threadIdx.x;
  const int vdim = c16 % 16 + 16 * (c16 / 32), vh = (c16 / 16) % 2;
  const int v_src = (vdim * 2 + vh) * 16;
  const int k_off = c16 / 16 * kPrefillKRow + c16 % 16 * 16;
  const int v_off = 2 * kPrefillKBytes + (vdim / 16 * 64 + 2 * vh * 16 + vdim % 16) * 16;
  const int kvp = pool_head(a, kvh);
  const int last_sub = last_blk / kSub;
  const int nstep = last_blk / kStep + 1;
  // Every load is issued, so the wait before the LDS stores is the same on
  // every path: past the last sub-tile the resource has zero bytes (nothing
  // is read, zeros come back) and the table entry is clamped to a live one.
  uint4 gk[KB], gv[KB];  // step j + 1 while step j is computed
  // Table entries of the step a load call fetches are read by the call
  // before it, as vector loads: they retire in order with the K/V loads
  // that the LDS stores wait for anyway, so no barrier or load waits on a
  // table read (a scalar read would be waited for at the next barrier).
  const __amdgpu_buffer_rsrc_t tab_rsrc = tile_rsrc(a.bt, (int64_t)b * a.mbs * 4, a.mbs * 4);
  uint32_t tab[KB];
  auto gtab = [&](int j) {
#pragma unroll
    for (int u = 0; u < KB; ++u)
      tab[u] = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, 0, min(j * KB + u, last_sub) * kSub / B * 4,
                                                    kCachedPolicy);
  };
  auto gload = [&](int j) {
    int phys[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) phys[u] = uniform((int)tab[u]);
    gtab(j + 1);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int sub = j * KB + u;
      const bool live = sub <= last_sub;
      const int64_t tile = ((int64_t)phys[u] * a.Hp + kvp) * kTileBytes;
      const int bytes = uniform(live ? kTileBytes : 0);
      const int soff = ((live ? sub : last_sub) * kSub % B) * kD * 2;
      gk[u] = tile_load16<kCachedPolicy>(tile_rsrc(a.kp, tile, bytes), c16 * 16, soff);
      gv[u] = tile_load16<kCachedPolicy>(tile_rsrc(a.vp, tile, bytes), v_src, soff);
    }
  };
  __shared__ int v_overflow;  // kPvConv: some staged V value is beyond fp16

  // One pass over the keys with the weighted values in mode kMode; for
  // kPvConv, whether the workgroup staged a V value fp16 cannot hold (the
  // pass is then void and reruns with kPvSplit).
  auto run = [&](auto mode) -> bool {
    constexpr int kMode = decltype(mode)::value;
    constexpr bool kSplit = kMode == kPvSplit;
    using MP = MfmaEngine<typename std::conditional<kSplit, T, F16>::type, B, G>;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[t][x] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[t] = -INFINITY;
      lsum[t] = 0.f;
    }
    float vmax = 0.f;
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        unsigned char* dst = &stage[buf][u / 2][0];
        uint4 v = gv[u];
        if constexpr (kMode == kPvConv) {
          v.x = bf16x2_to_f16x2(v.x, vmax);
          v.y = bf16x2_to_f16x2(v.y, vmax);
          v.z = bf16x2_to_f16x2(v.z, vmax);
          v.w = bf16x2_to_f16x2(v.w, vmax);
        }
        *reinterpret_cast<uint4*>(dst + (u % 2) * kPrefillKBytes + k_off) = gk[u];
        *reinterpret_cast<uint2*>(dst + v_off + (u % 2) * 8) = make_uint2(v.x, v.y);
        // the next token quarter
        *reinterpret_cast<uint2*>(dst + v_off + 16 * 16 + (u % 2) * 8) = make_uint2(v.z, v.w);
      }
    };

    // Step j is in LDS buffer j & 1 and step j + 1 in flight in gk / gv.
    // Steps wholly at or below the wave's first row need no causal mask
    // (every live column attends all their tokens; padding columns are never
    // stored) and run without any mask code or branch; the steps from the
    // diagonal on run with it.  The rescale decision is taken once per step
    // for both column tiles, so the exponentials, the splits and the
    // weighted-value products of a step form one straight run in which one
    // tile's products overlap the other tile's vector work.
    auto step = [&](const int j, auto masked) {
      constexpr bool kMasked = decltype(masked)::value;
      const int ts = j * kStep;
      if (!kMasked || ts <= last) {
        // Every sub-tile of the step is scored, also those past the wave's
        // last position (zeros or stale tokens in LDS; the causal mask
        // removes them), so the products need no branches or zero fills.
        f32x4 s[NT][KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const unsigned char* su = &stage[j & 1][u / 2][0] + (u % 2) * kPrefillKBytes;
          uint4 kr[4];
#pragma unroll
          for (int x = 0; x < 4; ++x)
            kr[x] = *reinterpret_cast<const uint4*>(su + col * kPrefillKRow + (32 * x + 8 * grp) * 2);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s[t][u] = M::mma_qk(kr[0], qop[t][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int x = 1; x < 4; ++x) s[t][u] = M::mma_qk(kr[x], qop[t][x], s[t][u]);
          }
        }
        // Scores in base-2 units, x = s * c2; p = 2^(x - m).  Steps without
        // the mask keep the raw scores: the max is taken on them and scaled
        // once (c2 > 0, and rounding is monotonic, so this is the max of the
        // scaled scores), and each exponent is one fused s * c2 - m, which
        // leaves the largest p within 2^-24 |m| of 1 (1 exactly once rounded
        // to fp16 while |m| < 2^12).  Masked steps and the hi + lo mode scale
        // first, as the mask and the split need.
        float xr[NT][KB][4], bm[NT];
        bool up = false;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) xr[t][u][r] = (kMasked || kSplit) ? s[t][u][r] * c2 : s[t][u][r];
          if constexpr (kMasked) {
            const int d = pos[t] - ts - 4 * grp;  // token ts + 4 grp + i is masked when i > d
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (u * kSub + r > d) xr[t][u][r] = -INFINITY;
          }
          bm[t] = -INFINITY;
#pragma unroll
          for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) bm[t] = fmaxf(bm[t], xr[t][u][r]);
          bm[t] = max_xor16(bm[t]);
          bm[t] = max_xor32(bm[t]);
          if constexpr (!kMasked && !kSplit) bm[t] *= c2;
          up = up || bm[t] > m[t] + kPrefillSlack;
        }
        // Lazy rescaling: the reference max moves only when some column's
        // scores exceed it by more than 2^kPrefillSlack, so most steps skip
        // the rescale; the probabilities then stay below 2^kPrefillSlack, and
        // the result o / l does not depend on the reference.  Token 0 is in
        // step 0 and every column attends it, so m is finite from the first
        // step on (a tile whose columns did not move gets alpha = 1).
        if (wave_any(up)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float mn = fmaxf(m[t], bm[t]);
            const float alpha = fast_exp2(m[t] - mn);
            lsum[t] *= alpha;
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[t][x] *= alpha;
            m[t] = mn;
          }
        }
        // Probabilities as the B operands of the weighted-value products:
        // for sub-tile pair h (sub-tiles 2h, 2h + 1) the values of both (4
        // tokens each, packed): fp16, or (kPvSplit) the bf16 hi halves and,
        // separately, the lo halves.
        uint4 bh[NT][KB / 2], bl[NT][KB / 2];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float ps = 0.f;
          uint32_t hw[KB][2], lw[KB][2];
#pragma unroll
          for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const float p0 = (kMasked || kSplit) ? fast_exp2(xr[t][u][r] - m[t]) : fast_exp2(fmaf(xr[t][u][r], c2, -m[t]));
              const float p1 = (kMasked || kSplit) ? fast_exp2(xr[t][u][r + 1] - m[t]) : fast_exp2(fmaf(xr[t][u][r + 1], c2, -m[t]));
              if constexpr (kSplit) {
                ps += p0 + p1;
                split_pair_bf16(p0, p1, hw[u][r / 2], lw[u][r / 2]);
              } else {
                // P rounded once; the sum is over the same rounded values
                const half2_t h = {(_Float16)p0, (_Float16)p1};
                hw[u][r / 2] = __builtin_bit_cast(uint32_t, h);
                ps = __builtin_amdgcn_fdot2(h, half2_t{(_Float16)1.f, (_Float16)1.f}, ps, false);
              }
            }
          lsum[t] += ps;
#pragma unroll
          for (int h = 0; h < KB / 2; ++h) {
            bh[t][h] = make_uint4(hw[2 * h][0], hw[2 * h][1], hw[2 * h + 1][0], hw[2 * h + 1][1]);
            if constexpr (kSplit)
              bl[t][h] = make_uint4(lw[2 * h][0], lw[2 * h][1], lw[2 * h + 1][0], lw[2 * h + 1][1]);
          }
        }
        // Weighted values, two sub-tiles per 32-deep product: A = this
        // lane's 4 tokens of sub-tile 2h and of 2h + 1 (one dim, one 16-byte
        // LDS entry), against the probabilities (kPvSplit: the hi ones, then
        // the lo ones).
#pragma unroll
        for (int h = 0; h < KB / 2; ++h) {
          const int tok0 = ts + 2 * h * kSub, tok1 = tok0 + kSub;
          if constexpr (kMasked) {
            if (tok0 > last) continue;
          }
          const unsigned char* sv = &stage[j & 1][h][0] + 2 * kPrefillKBytes;
          uint4 va[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) va[x] = *reinterpret_cast<const uint4*>(sv + (x * 64 + grp * 16 + col) * 16);
          if constexpr (kMasked) {
            // Slots past the wave's last position may lie past the sequence
            // end and hold anything (NaN included; sub-tile 2h + 1 may lie
            // wholly past it): zero them so 0 * slot stays 0.
            if (last - tok1 + 1 < kSub) v_tail_mask(va, last - tok0 + 1 - 4 * grp, last - tok1 + 1 - 4 * grp);
          }
#pragma unroll
          for (int x = 0; x < 8; ++x) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              acc[t][x] = MP::mma_32(va[x], bh[t][h], acc[t][x]);
              if constexpr (kSplit) acc[t][x] = MP::mma_32(va[x], bl[t][h], acc[t][x]);
            }
          }
        }
      }
      // step j + 1 to the other buffer (last read before the previous
      // barrier), then step j + 2 starts loading: it has one step of compute
      // to arrive
      if (j + 1 < nstep) stage_store((j + 1) & 1);
      gload(j + 2);
      __syncthreads();
    };

    if (kMode == kPvConv && threadIdx.x == 0) v_overflow = 0;
    gtab(0);
    gload(0);
    stage_store(0);
    gload(1);
    __syncthreads();
    // The first step crossing the wave's first row (0 for a wave without
    // rows: every step then only stages and waits).
    const int jd = last < 0 ? 0 : min(nstep, (L - n + ct0 * R + 1) / kStep);
    int j = 0;
    for (; j < jd; ++j) step(j, std::false_type{});
    for (; j < nstep; ++j) step(j, std::true_type{});
    if constexpr (kMode != kPvConv) {
      return false;
    } else {
      // every thread is past its last stage read (the step's barrier)
      if (vmax >= kPvConvLimit) v_overflow = 1;
      __syncthreads();
      return v_overflow != 0;
    }
  };
  if constexpr (T::kCode == BF16::kCode) {
    if (run(std::integral_constant<int, kPvConv>{})) run(std::integral_constant<int, kPvSplit>{});
  } else {
    run(std::integral_constant<int, kPvF16>{});
  }
  // Every wave is past its last stage read (the last step's barrier): the
  // stage now holds each wave's output tiles on their way out.  Waves
  // without rows take part in the barriers and store nothing.
  float inv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l = sum_xor32(sum_xor16(lsum[t]));
    inv[t] = last < 0 ? 0.f : 1.f / l;
  }
  static_assert(kPrefillWaves * kPrefillOutBytes <= sizeof(stage), "output tiles fit the stage");
  prefill_store_tiles<T, G, NT>(a, &stage[0][0][0] + wave * kPrefillOutBytes, acc, inv, ct0, n, q0, kvh);
}

}  // namespace pa
