// shared_prefix.h — decode over a batch whose sequences share prefix blocks,
// reading every shared block once for the whole group.
//
// "PagedAttention: The Cache Was Storing Nothing", §2.3: sequences that
// start with the same prompt (parallel samples, beams, a common system
// prompt) point their tables at the same physical blocks.  Decode attends
// each of those blocks once per sequence; here the sequences of a prefix
// group are attended together on their shared blocks, so the group's query
// heads meet each shared K/V tile in one pass:
//
//   item = (sub-group of <= kWideCols / G members, KV head): the members'
//   G query heads each, as up to kWideCols = 32 MFMA columns (two 16-column
//   tiles), against the 16-token sub-tiles of the shared blocks.  Column
//   (member m, head g) attends token t of the shared blocks only while
//   t < min(L_m, shared * B): a member shorter than the shared prefix stops
//   inside it (its last shared block is partly its own).
//
// A member's attention is then the merge ("39 · PagedAttention", §3 merge
// equation) of its item part and its private part (the blocks after the
// shared ones, attended as usual), which the member-pair protocol of
// pa_device.h publishes, counts in and folds.  Sequences outside every
// group, and groups with one member or no shared block, run the ordinary
// path.
//
// Schedule.  Two unit spaces, each cut into nwg equal chunks: the items'
// blocks (sub-group-major, then KV head, then block) and the private
// blocks (sequence-major as in the ordinary decode, without the shared
// blocks).  Workgroup k streams its chunk of private units first and runs
// its chunk of item units last (after its chunk-end folds).  An item's
// fixed costs (staging the members' queries, merging the waves,
// publishing, folding) leave the memory system idle; run last, they fall
// where workgroups finish their streams at different times, while others
// still stream (measured on the serving batch: items first 267 us per
// call, items last on half the workgroups 264, on all 262; items placed
// at staggered points inside the streams 290).  Contributions count in on
// their pair's counter in any order.
#pragma once

#include "decode_mfma.h"
#include "pa_device.h"

#include <type_traits>

namespace pa {

// Exclusive prefix sum of count(i), i < n, into out[0..n] (out[n] = total),
// in passes of kThreads with a carry.  All threads call; wsum holds kWaves
// ints of LDS.
template <class F>
__device__ inline void block_scan(int n, F count, int* out, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    int x = i < n ? count(i) : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry, total = carry;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    if (i < n) out[i + 1] = before + x;
    carry = total;
    __syncthreads();
  }
  if (tid == 0) out[0] = 0;
  __syncthreads();
}

// Exclusive prefix sums of count1(i), i < n1, into out1[0..n1] and of
// count2(i), i < n2, into out2[0..n2], in one set of passes (the two take
// the barriers of one).  All threads call; wsum holds 2 * kWaves ints of
// LDS.
template <class F1, class F2>
__device__ inline void block_scan2(int n1, F1 count1, int* out1, int n2, F2 count2, int* out2,
                                   int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c1 = 0, c2 = 0;
  for (int base = 0; base < max(n1, n2); base += kThreads) {
    const int i = base + tid;
    int x = i < n1 ? count1(i) : 0, y = i < n2 ? count2(i) : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(x, off), v = __shfl_up(y, off);
      if (lane >= off) {
        x += u;
        y += v;
      }
    }
    if (lane == 63) {
      wsum[wave] = x;
      wsum[kWaves + wave] = y;
    }
    __syncthreads();
    int b1 = c1, t1 = c1, b2 = c2, t2 = c2;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) {
        b1 += wsum[w];
        b2 += wsum[kWaves + w];
      }
      t1 += wsum[w];
      t2 += wsum[kWaves + w];
    }
    if (i < n1) out1[i + 1] = b1 + x;
    if (i < n2) out2[i + 1] = b2 + y;
    c1 = t1;
    c2 = t2;
    __syncthreads();
  }
  if (tid == 0) {
    out1[0] = 0;
    out2[0] = 0;
  }
  __syncthreads();
}

// Virtual units charged per (sequence, KV head) in the private unit space.
// On the serving batch a workgroup's stream time measured linear in its
// chunk's 16-token blocks (~0.3 us each) and pieces (~2 us each: the merge
// across the waves, the publication and the fold at the chunk end); with
// the items last, charges of 4, 5, 6, 7, 8 and 10 blocks per piece
// measured 285, 264, 259.5, 260.3, 261.7 and 267 us per call.
constexpr int kPieceUnits = 6;

// Builds the shared-prefix schedule in dynamic LDS (SharedLayout, scalars
// in sm.ssc).  A group of M >= 2 members with shared > 0 blocks is cut into
// ceil(M / Mmax) sub-groups of near-equal size, Mmax = kWideCols / G.
// Group bounds are clamped to [0, S], so malformed groups cannot address
// outside the arrays (their results are undefined; pa_validate_shared_host
// rejects them).  The lengths and the group arrays are read from global
// memory in one pass.  All threads call; wsum holds 2 * kWaves ints.
template <int B, int G, class Smem>
__device__ inline void shared_prologue(const Args& a, Smem& sm, int* wsum) {
  constexpr int kMmax = kWideCols / G;
  const int S = a.S, ng = a.ngroups;
  const SharedLayout l = shared_layout(S, ng);
  for (int i = threadIdx.x; i < S || i <= ng; i += kThreads) {
    if (i < S) {
      l.lens[i] = a.lens[i];
      l.shb[i] = 0;
      l.seq_sg[i] = -1;
    }
    if (i <= ng && ng > 0) {
      l.gstart[i] = a.grp_start[i];
      l.gshared[i] = i < ng ? a.grp_shared[i] : 0;
    }
  }
  __syncthreads();
  auto range = [&](int g, int& st, int& en, int& sh) {
    st = min(max(l.gstart[g], 0), S);
    en = min(max(l.gstart[g + 1], st), S);
    sh = max(l.gshared[g], 0);
  };
  block_scan(ng, [&](int g) {
    int st, en, sh;
    range(g, st, en, sh);
    const int M = en - st;
    return (M >= 2 && sh > 0) ? (M + kMmax - 1) / kMmax : 0;
  }, l.gbase, wsum);
  for (int g = threadIdx.x; g < ng; g += kThreads) {
    int st, en, sh;
    range(g, st, en, sh);
    const int M = en - st, n = l.gbase[g + 1] - l.gbase[g];
    // tokens of the shared blocks, saturated (sh * B may exceed int)
    const int shtok = sh > (0x7fffffff / B) ? 0x7fffffff : sh * B;
    for (int i = 0; i < n; ++i) {
      const int s = l.gbase[g] + i;
      if (s >= S) break;  // only overlapping (invalid) groups get here
      const int f = st + (i * M) / n, e = st + ((i + 1) * M) / n;  // e - f <= kMmax
      int lmax = 0, ref = f;
      // the members' lengths first, all reads in flight at once
      int Ls[kMmax];
#pragma unroll
      for (int k = 0; k < kMmax; ++k) Ls[k] = f + k < e ? l.lens[f + k] : 0;
#pragma unroll
      for (int k = 0; k < kMmax; ++k) {
        const int b = f + k;
        if (b < e) {  // a guard rather than a break, so the loop unrolls
          const int lim = min(Ls[k], shtok);
          if (Ls[k] > 0) {
            l.shb[b] = blocks_of(lim, B);
            l.seq_sg[b] = s;
          }
          if (lim > lmax) {
            lmax = lim;
            ref = b;
          }
        }
      }
      l.sg_first[s] = f;
      l.sg_count[s] = e - f;
      l.sg_ref[s] = ref;
      l.sg_len[s] = lmax;
    }
  }
  __syncthreads();
  const int nsg = min(l.gbase[ng], S);
  block_scan2(S, [&](int b) {
    const int np = blocks_of(l.lens[b], B) - l.shb[b];
    return np > 0 ? np + kPieceUnits : 0;
  }, l.cum, nsg, [&](int s) { return blocks_of(l.sg_len[s], B); }, l.icum, wsum);
  if (threadIdx.x == 0) {
    sm.ssc.nsg = nsg;
    sm.ssc.B = B;
    sm.ssc.V = kPieceUnits;
    const int wi = l.icum[nsg] * a.Hkv, wp = l.cum[S] * a.Hkv;
    sm.ssc.cI = wi > 0 ? (wi + a.nwg - 1) / a.nwg : 1;
    sm.ssc.cP = wp > 0 ? (wp + a.nwg - 1) / a.nwg : 1;
  }
  __syncthreads();
}

// Sub-tiles in flight per wave in the item phase.  Two, as in the ordinary
// engine; three (the most that fit the registers) measured 1.5 us slower
// per call on the serving batch.
constexpr int kItemTiles = 2;

// One piece of an item: blocks [j0, j1) of sub-group sg's shared blocks,
// KV head kvh, all its members' query heads as up to kWideCols MFMA
// columns (two 16-column tiles when they need more than 16).  Each wave
// owns one column tile: with two tiles, waves 0-3 hold tile 0 and waves 4-7
// tile 1, and the two halves walk the same 16-token sub-tiles, kept within
// two passes of each other by barriers (the second read of a sub-tile is
// served by L2, so HBM sees it once);
// with one tile all eight waves share the sub-tiles.  kItemTiles sub-tiles
// are in flight per wave, and the wave partials of all columns merge in
// LDS in one pass.  A whole item's member parts go to the
// pair slots (or straight to `out` for a member without private blocks); a
// fragment cut by chunk boundaries goes to wide slot `slot` for the fold.
// All threads call.
template <class T, int B, int G, class Smem>
__device__ inline void item_piece(const Args& a, Smem& sm, const SharedInfo& si, int sg, int kvh,
                                  int j0, int j1, bool whole, int slot) {
  using M = MfmaEngine<T, B, G, true>;
  using Op4 = typename M::Op4;
  using Elem = typename M::Elem;
  using Tile = typename M::Tile;
  constexpr int kQC = kD * 2 / 16;  // 16-byte chunks per query head
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int b0 = si.sg_first[sg], nm = si.sg_count[sg], ref = si.sg_ref[sg];
  const int tb = j0 * B, te = min(j1 * B, si.sg_len[sg]);
  const int nsub = (te - tb + kSub - 1) / kSub;
  const int nct = nm * G > 16 ? 2 : 1;   // column tiles in use
  const int wpt = kWaves / nct;          // waves per column tile
  const int ct = uniform(wave / wpt);    // this wave's column tile
  const int c = 16 * ct + col;           // this lane's column

  // the list of contributions waiting for a count-in must have room for
  // this piece's members
  if (uniform(sm.dn) + nm > Smem::kDefers) flush_members<T, G, 1>(a, sm);

  // the wave's first two sub-tiles (default cache policy: the other column
  // tile's waves read the same sub-tiles)
  const int32_t* row = a.bt + (int64_t)ref * a.mbs;
  auto load = [&](int t, Tile& tile) {
    const bool live = t < nsub;
    const int tt = live ? t : nsub - 1;
    const int tok = uniform(tb + kSub * tt);
    const int phys = uniform(as_constant(row)[tok / B]);
    const int bytes = uniform(live ? B * kD * 2 : 0);
    M::template load_tile<kCachedPolicy>(a, kvh, tok % B, phys, bytes, tile);
  };
  Tile tl[kItemTiles];
  int t = wave % wpt;
#pragma unroll
  for (int k = 0; k < kItemTiles; ++k) load(t + k * wpt, tl[k]);
  // members' query heads (column c = member * G + head), zero past the
  // last, staged while the first sub-tiles are on their way
  uint4* wq = &sm.q[0][0];
  for (int x = threadIdx.x; x < kWideCols * kQC; x += kThreads) {
    const int cc = x / kQC, k = x % kQC, mi = cc / G, g = cc % G;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (mi < nm)
      v = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                         ((int64_t)(b0 + mi) * a.Hq + kvh * G + g) * kD * 2)[k];
    wq[x] = v;
  }
  __syncthreads();  // query heads staged

  // this lane's column: tokens end (0 for padding columns) and the B
  // operand of the score product
  int lim = 0;
  {
    const int mi = c / G;
    if (mi < nm) {
      const int b = b0 + mi;
      lim = min(si.lens[b], si.shb[b] * B);
    }
  }
  uint4 qop[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) qop[x] = wq[c * kQC + grp + 4 * x];
  f32x4 acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  // One sub-tile starting at token tok0 with `valid` tokens inside the
  // item (the rest are slack of the last shared block).  A column's running
  // max may stay -inf (a member whose shared part ends before this wave's
  // tokens, or a padding column): then its sums stay 0.
  auto compute = [&](Tile& tl, int tok0, int valid) {
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < 4; ++x) sc = M::mma_qk(tl.k[x], qop[x], sc);
    if (valid < kSub) {
      const int nv = valid - 4 * grp;
      const uint32_t lo_mask = (nv >= 1 ? 0x0000ffffu : 0u) | (nv >= 2 ? 0xffff0000u : 0u);
      const uint32_t hi_mask = (nv >= 3 ? 0x0000ffffu : 0u) | (nv >= 4 ? 0xffff0000u : 0u);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        tl.v[x].x &= lo_mask;
        tl.v[x].y &= hi_mask;
      }
    }
    float xr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      xr[r] = (tok0 + 4 * grp + r < lim) ? sc[r] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(xr[0], xr[1]), fmaxf(xr[2], xr[3]));
    bm = max_xor16(bm);
    bm = max_xor32(bm);
    const float mn = fmaxf(mrun, bm);
    if (wave_any(mn > mrun)) {
      const float alpha = mn > mrun ? fast_exp2(mrun - mn) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] *= alpha;
      mrun = mn;
    }
    const float mb = mrun == -INFINITY ? 0.f : mrun;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(xr[r] - mb);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    Op4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      phi[r] = (Elem)p[r];
      plo[r] = (Elem)(p[r] - (float)phi[r]);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      acc[x] = M::mma_pv2(tl.v[x], phi, plo, acc[x]);
    }
  };
  // every pass refills each tile register after its compute (an empty
  // load past the end), so the loads in flight are always in the order
  // they are consumed.  With two column tiles, waves w and w + 4 read the
  // same sub-tiles: every wave runs the same number of passes and a
  // barrier ends every second one (the merge below has its own), so the
  // two reads of a sub-tile are issued within two passes of each other and
  // the second finds it in L2.  Unsynchronised, about half of the shared
  // bytes were fetched from HBM twice (34 MB per call on the serving
  // batch); a barrier every pass removes all of it but costs more time
  // than it saves.
  const int passes = (nsub + kItemTiles * wpt - 1) / (kItemTiles * wpt);
  for (int pass = 0; pass < passes; ++pass) {
#pragma unroll
    for (int k = 0; k < kItemTiles; ++k) {
      const int tk = t + k * wpt;
      if (tk < nsub) compute(tl[k], tb + kSub * tk, min(kSub, te - (tb + kSub * tk)));
      load(tk + kItemTiles * wpt, tl[k]);
    }
    t += kItemTiles * wpt;
    if (nct == 2 && (pass & 1) && pass + 1 < passes) __syncthreads();
  }

  // wave partials -> LDS (wave w holds column tile w / wpt), then every
  // column merges the wpt waves of its tile
  {
    float l = sum_xor16(lsum);
    l = sum_xor32(l);
    if (grp == 0) {
      sm.m[wave][c] = mrun;
      sm.l[wave][c] = l;
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
      *reinterpret_cast<f32x4*>(&sm.o[wave][col][16 * x + 4 * grp]) = acc[x];
  }
  // A whole item whose member has every private contribution counted in
  // already is that pair's last contribution: the workgroup folds the pair
  // from the merged item part without publishing it or counting in (the
  // counter goes back to zero; nobody else touches it in this call).  The
  // fold takes the contributions in the same order and arithmetic as
  // fold_members, so the result does not depend on who folds.  Member
  // flags in sm.dlast, layouts in sm.dlay (both free between count-ins).
  if (whole && threadIdx.x < nm) {
    const int b = b0 + threadIdx.x, L = si.lens[b];
    int fast = 0;
    if (L > 0 && blocks_of(L, B) != si.shb[b]) {
      const int pair = b * a.Hkv + kvh;
      const MemberLayout m = member_layout(a, si, pair);
      if (counted(a.pcnt + pair) == m.nfr + m.npp - 1) {
        fast = 1;
        reset_count(a.pcnt + pair);
        acquire_counted();
        sm.dlay[threadIdx.x] = m;
      }
    }
    sm.dlast[threadIdx.x] = fast;
  }
  __syncthreads();
  constexpr int kOut = kWideCols * kD / kThreads;
  // item part of each of this thread's outputs that a fast member folds
  // below (pf = member + 1; 0: none)
  float po[kOut], pm[kOut], pl[kOut];
  int pf[kOut];
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    pf[r] = 0;
    po[r] = pl[r] = 0.f;
    pm[r] = -INFINITY;
    const int idx = threadIdx.x + r * kThreads;
    const int cc = idx / kD, d = idx % kD, cl = cc % 16, tile = cc / 16;
    const int mi = cc / G, g = cc % G;
    if (tile >= nct || mi >= nm) continue;
    const int w0 = tile * wpt;
    float Mx = sm.m[w0][cc];
    for (int w = w0 + 1; w < w0 + wpt; ++w) Mx = fmaxf(Mx, sm.m[w][cc]);
    float o = 0.f, l = 0.f;
    for (int w = w0; w < w0 + wpt; ++w) {
      const float f = rescale(sm.m[w][cc], Mx);
      o += f * sm.o[w][cl][d];
      l += f * sm.l[w][cc];
    }
    const int b = b0 + mi, L = si.lens[b];
    if (L == 0) continue;
    const int pair = b * a.Hkv + kvh;
    if (whole) {
      if (blocks_of(L, B) == si.shb[b]) {
        store_out<T>(a.out, ((int64_t)b * a.Hq + kvh * G + g) * kD + d, o / l, a.out_f32);
      } else if (sm.dlast[mi]) {
        pf[r] = mi + 1;
        po[r] = o;
        pm[r] = Mx;
        pl[r] = l;
      } else {
        st_agent(a.pair_o + ((int64_t)(2 * pair) * G + g) * kD + d, o);
        if (d == 0) {
          st_agent(a.pair_ml + ((int64_t)(2 * pair) * G + g) * 2, Mx);
          st_agent(a.pair_ml + ((int64_t)(2 * pair) * G + g) * 2 + 1, l);
        }
      }
    } else {
      st_agent(a.wide_o + ((int64_t)slot * kWideCols + cc) * kD + d, o);
      if (d == 0) {
        st_agent(a.wide_ml + ((int64_t)slot * kWideCols + cc) * 2, Mx);
        st_agent(a.wide_ml + ((int64_t)slot * kWideCols + cc) * 2 + 1, l);
      }
    }
  }
  // The fast members' folds: contributions two at a time (the item part
  // first), in the order and arithmetic of fold_members, for half of this
  // thread's outputs at a time with all their loads in flight together
  // (the whole set at once does not fit the registers).
  auto fold_fast = [&](auto half) {
    constexpr int kU = kOut / 2, r0 = decltype(half)::value * kU;
    int emax = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (pf[r0 + u]) emax = max(emax, sm.dlay[pf[r0 + u] - 1].nfr + sm.dlay[pf[r0 + u] - 1].npp);
    if (emax == 0) return;
    float fm[kU], fl[kU], fo[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      fm[u] = -INFINITY;
      fl[u] = fo[u] = 0.f;
    }
    for (int i0 = 0; i0 < emax; i0 += 2) {
      float vo[kU][2], vm[kU][2], vl[kU][2];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int r = r0 + u, idx = threadIdx.x + r * kThreads;
        const int g = (idx / kD) % G, d = idx % kD;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          vo[u][j] = 0.f;
          vm[u][j] = -INFINITY;
          vl[u][j] = 0.f;
          if (!pf[r]) continue;
          const MemberLayout& m = sm.dlay[pf[r] - 1];
          const int i = i0 + j;
          if (i == 0) {
            vo[u][j] = po[r];
            vm[u][j] = pm[r];
            vl[u][j] = pl[r];
          } else if (i < m.nfr + m.npp) {
            const float* co;
            const float* cml;
            member_contrib<G>(a, m, i, co, cml);
            vo[u][j] = ld_agent(co + g * kD + d);
            vm[u][j] = ld_agent(cml + g * 2);
            vl[u][j] = ld_agent(cml + g * 2 + 1);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float Mn = fmaxf(fm[u], fmaxf(vm[u][0], vm[u][1]));
        const float f0 = rescale(fm[u], Mn), f1 = rescale(vm[u][0], Mn), f2 = rescale(vm[u][1], Mn);
        fl[u] = fl[u] * f0 + f1 * vl[u][0] + f2 * vl[u][1];
        fo[u] = fo[u] * f0 + f1 * vo[u][0] + f2 * vo[u][1];
        fm[u] = Mn;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = r0 + u;
      if (!pf[r]) continue;
      const int idx = threadIdx.x + r * kThreads;
      const int cc = idx / kD, d = idx % kD, g = cc % G;
      const int b = b0 + pf[r] - 1;
      store_out<T>(a.out, ((int64_t)b * a.Hq + kvh * G + g) * kD + d, fo[u] / fl[u], a.out_f32);
    }
  };
  static_assert(kOut % 2 == 0, "outputs fold in two halves");
  fold_fast(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  fold_fast(std::integral_constant<int, 1>{});
  // list the members' contributions for the count-in (a whole item's
  // member without private blocks, or folded above, is already final)
  if (threadIdx.x < 64) {
    const int b = b0 + lane;
    bool add = lane < nm && si.lens[b] > 0;
    if (add && whole) add = blocks_of(si.lens[b], B) != si.shb[b] && !sm.dlast[lane];
    const uint64_t am = __builtin_amdgcn_ballot_w64(add);
    const int n0 = sm.dn;
    if (add) {
      const int i = n0 + __builtin_popcountll(am & ((uint64_t(1) << lane) - 1));
      sm.dpair[i] = b * a.Hkv + kvh;
      sm.dstage[i] = -1;
      sm.dpiece[i] = -1;
    }
    if (lane == 0) sm.dn = n0 + __builtin_popcountll(am);
  }
  __syncthreads();
}

// This workgroup's chunk of item units, then the count-in of their
// contributions.  All threads call.
template <class T, int B, int G, class Smem>
__device__ inline void run_items(const Args& a, Smem& sm, int chunk) {
  const SharedInfo si = shared_info(a, sm);
  const int wi = si.icum[si.nsg] * a.Hkv;
  const int s0 = chunk * si.cI, e0 = min(wi, s0 + si.cI);
  for (int f = s0; f < e0;) {
    const int sg = uniform(find_seq(si.icum, si.nsg, a.Hkv, f));
    const int nI = si.icum[sg + 1] - si.icum[sg];
    const int kvh = uniform((f - si.icum[sg] * a.Hkv) / nI);
    const int ustart = si.icum[sg] * a.Hkv + kvh * nI;
    const int j0 = f - ustart, pe = min(e0, ustart + nI), j1 = pe - ustart;
    item_piece<T, B, G>(a, sm, si, sg, kvh, j0, j1, j0 == 0 && j1 == nI,
                        2 * chunk + (f == s0 ? 0 : 1));
    f = pe;
  }
  if (uniform(sm.dn) > 0) flush_members<T, G, kMemberFoldU>(a, sm);
}

// The shared-prefix decode: prologue, this workgroup's private units with
// the ordinary streaming loop (member pieces publish instead of writing
// out), the chunk-end folds and count-in, then its item units and their
// count-in.
template <class T, int B, int G>
__device__ inline void run_decode_shared(const Args& a) {
  using Engine = MfmaEngine<T, B, G, true>;
  using Smem = typename Engine::Smem;
  __shared__ int wsum[2 * kWaves];
  __shared__ Smem sm;
  if (threadIdx.x == 0) {
    sm.fold_late = 0;
    sm.early_seen = -1;
    sm.dn = 0;
    sm.nstage = 0;
  }
  shared_prologue<B, G>(a, sm, wsum);
  const int chunk = chunk_of_wg(blockIdx.x, a.nwg);
  zero_empty_sequences<T>(a, chunk, shared_layout(a.S, a.ngroups).lens);
  const SharedInfo si = shared_info(a, sm);
  const int W = si.cum[a.S] * a.Hkv;
  const int c = si.cP;
  const int s = chunk * c;
  const int e = min(W, s + c);
  if (threadIdx.x == 0) sm.next_f = s;
  __syncthreads();
  while (true) {
    if (threadIdx.x < 64) list_batch<B, true>(a, sm, si.cum, si.lens, si.shb, s, e, chunk, c, si.V);
    __syncthreads();
    const int npl = sm.npl;
    if (npl == 0) break;
    stream_batch<T, B, G, Engine>(a, sm);
    __syncthreads();
    // the next batch adds at most kBatch member contributions
    static_assert(Smem::kBatch <= Smem::kDefers, "a batch of pieces must fit the count-in list");
    if (uniform(sm.dn) > Smem::kDefers - Smem::kBatch) flush_members<T, G, 1>(a, sm);
  }
  finish_chunk<T, G>(a, sm);
  // after the chunk-end folds: an item's merge reuses the LDS that holds
  // the own partial of a late split
  run_items<T, B, G>(a, sm, chunk);
}

}  // namespace pa
