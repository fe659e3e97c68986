// kv_write.h — gfx950 kernels that write the paged cache in the library's
// pool layout: appending one decode token per sequence, and the whole-block
// copy of copy-on-write sharing.
//
// Both are pure data movement and bound by memory traffic, not arithmetic.
//
// Append ("PagedAttention: The Cache Was Storing Nothing", §2.2: the block
// table maps a request's logical blocks to physical ones, and only its last
// block is ever partly filled).  The token at logical position t of
// sequence b lands in physical block block_tables[b][t / B], slot t % B,
// of every KV head.  In the K pool that slot is one contiguous head_dim
// row (the tile is token-major); in the V pool the tile is transposed
// inside each 16-token group, so the row's head_dim values lie 16 elements
// apart.  One wave handles one (sequence, KV head): the K row is one
// coalesced 256-byte (16-bit types) store, the V row 128 element stores
// into the 4 KiB group.
//
// Block copy (§2.3 of the same page: a shared block is copied only when a
// sequence diverges and writes into it).  A physical block of one pool is
// one contiguous num_kv_heads * B * head_dim * esize range, a multiple of
// 4 KiB; the copy moves it in 4 KiB chunks, 16 bytes per thread (the
// source with the non-temporal policy: it is read once), with four chunks'
// loads in flight per workgroup before their stores.
#pragma once

#include "kernel_args.h"
#include "pa_device.h"

namespace pa {


template <int kEsize>
struct Bits;
template <>
struct Bits<2> { using T = uint16_t; using Pair = uint32_t; };
template <>
struct Bits<4> { using T = uint32_t; using Pair = uint2; };

// Grid: ceil(S * Hkv / kAuxWaves) workgroups of kAuxThreads; wave = one
// (sequence, KV head).  Lane l moves dims 2l and 2l + 1.
template <int kEsize>
__global__ __launch_bounds__(kAuxThreads) void append_kernel(AppendArgs a) {
  using E = typename Bits<kEsize>::T;
  using E2 = typename Bits<kEsize>::Pair;
  static_assert(kD == 128, "two dims per lane");
  const int lane = threadIdx.x & 63;
  const int i = uniform(blockIdx.x * kAuxWaves + (threadIdx.x >> 6));
  if (i >= a.S * a.Hkv) return;
  const int b = i / a.Hkv, kvh = i % a.Hkv;
  const int t = as_constant(a.pos)[b];
  if (t < 0) return;
  const int phys = as_constant(a.bt + (int64_t)b * a.mbs)[t / a.B];
  const int slot = t % a.B;
  const int64_t tile = ((int64_t)phys * a.Hkv + kvh) * a.B * kD;  // element offset of the tile
  const int64_t row = ((int64_t)b * a.Hkv + kvh) * kD;            // element offset of the new rows
  const E2 k2 = reinterpret_cast<const E2*>(static_cast<const E*>(a.kn) + row)[lane];
  const E2 v2 = reinterpret_cast<const E2*>(static_cast<const E*>(a.vn) + row)[lane];
  // K: row `slot` of the token-major tile
  reinterpret_cast<E2*>(static_cast<E*>(a.kp) + tile + (int64_t)slot * kD)[lane] = k2;
  // V: element (slot, d) of the tile sits at ((slot/16)*kD + d)*16 + slot%16
  E* vt = static_cast<E*>(a.vp) + tile + (int64_t)(slot / kSub) * kD * kSub + slot % kSub;
  E lo, hi;
  if constexpr (kEsize == 2) {
    lo = (E)(v2 & 0xffffu);
    hi = (E)(v2 >> 16);
  } else {
    lo = v2.x;
    hi = v2.y;
  }
  vt[(2 * lane) * kSub] = lo;
  vt[(2 * lane + 1) * kSub] = hi;
}


// Work item w = ((pair * 2) + pool) * chunks + c.  Grid-stride over passes
// of kCopyUnroll consecutive items; item indices are wave-uniform, so the
// id lookups are scalar loads.
__global__ __launch_bounds__(kAuxThreads) void copy_blocks_kernel(CopyArgs a) {
  const int per_pair = 2 * a.chunks;
  for (int w0 = blockIdx.x * kCopyUnroll; w0 < a.total; w0 += gridDim.x * kCopyUnroll) {
    uint4 v[kCopyUnroll];
    uint4* to[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int w = uniform(w0 + u);
      to[u] = nullptr;
      if (w >= a.total) continue;
      const int pair = w / per_pair, rem = w % per_pair;
      char* pool = rem < a.chunks ? a.kp : a.vp;
      const int64_t c = rem % a.chunks;
      const int64_t s = as_constant(a.src)[pair], d = as_constant(a.dst)[pair];
      const auto src = tile_rsrc(pool, s * a.block_bytes + c * kChunkBytes, kChunkBytes);
      v[u] = tile_load16<kStreamPolicy>(src, threadIdx.x * 16, 0);
      to[u] = reinterpret_cast<uint4*>(pool + d * a.block_bytes + c * kChunkBytes + threadIdx.x * 16);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (to[u]) *to[u] = v[u];
  }
}

}  // namespace pa
