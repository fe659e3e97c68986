"""Pins that tie the fp64 oracle to the pages and to mathematics.

Each pin takes a loaded oracle build (oracle.Oracle) and raises
AssertionError when that build disagrees with something fixed outside the
oracle: a worked example on the pages, a closed form, an invariant of
exact attention, a library routine (torch / numpy), or an independent
brute-force evaluation written here.  test_oracle.py runs every pin on the
real build; test_oracle_mutants.py runs them on builds with planted
mistakes and requires each mistake to be caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers
# Written independently of the oracle: numpy fancy indexing instead of the
# oracle's per-token loops.

def vgroup(B):
    """Tokens per transposed V group: 16 when B is a multiple of 16, else B."""
    return 16 if B % 16 == 0 else B


def scatter(Klog, Vlog, tables, lens, num_blocks, B, fill=np.nan):
    """Place logical fp64 K/V [S][Hkv][Lmax][D] into pools of the library
    layout: K [NB][Hkv][B][D], V [NB][Hkv][B/G][D][G]; untouched slots = fill."""
    S, H, _, D = Klog.shape
    Gv = vgroup(B)
    kp = np.full((num_blocks, H, B, D), fill)
    vp = np.full((num_blocks, H, B // Gv, D, Gv), fill)
    for b in range(S):
        t = np.arange(int(lens[b]))
        phys = np.asarray(tables[b])[t // B]
        slot = t % B
        for g in range(H):
            kp[phys, g, slot, :] = Klog[b, g, : t.size]
            vp[phys, g, slot // Gv, :, slot % Gv] = Vlog[b, g, : t.size]
    return kp, vp


def random_tables(rng, lens, B, num_blocks, max_blocks):
    ids = rng.permutation(num_blocks)
    bt = np.full((len(lens), max_blocks), -1, np.int32)
    k = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // B)
        bt[b, :n] = ids[k: k + n]
        k += n
    return bt


def numpy_reference(q, kp, vp, bt, lens, scale, Hkv, B):
    """Second, independent evaluation of the formula (fp64 numpy)."""
    S, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    for b in range(S):
        L = int(lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        phys, slot = bt[b, t // B], t % B
        Gv = vgroup(B)
        for h in range(Hq):
            K = kp[phys, h // G, slot, :]
            V = vp[phys, h // G, slot // Gv, :, slot % Gv]
            s = scale * (K @ q[b, h])
            w = np.exp(s - s.max())
            out[b, h] = (w / w.sum()) @ V
    return out


def sdpa(q, K, V, scale):
    """torch's scaled_dot_product_attention on CPU in fp64, one query."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).reshape(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, 0, 0].numpy()


def decode_f64(O, q, kp, vp, bt, lens, scale, Hkv, B):
    """Oracle on fp64 data stored as float32 (values chosen exactly
    representable in float32 by the callers)."""
    return O.paged_decode(np.asarray(q, np.float32), np.asarray(kp, np.float32),
                          np.asarray(vp, np.float32), bt, np.asarray(lens, np.int32), scale,
                          num_kv_heads=Hkv, block_size=B, dtype="f32")


def f32_normal(rng, shape, grid=None):
    """N(0,1) draws; with grid, rounded to multiples of 2**-grid."""
    x = rng.standard_normal(shape)
    if grid is not None:
        x = np.round(x * 2.0 ** grid) / 2.0 ** grid
    return x.astype(np.float32).astype(np.float64)


# ------------------------------------------------------------ conversions

def pin_f16_decode_all_patterns(O):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.to_f64(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decode_all_patterns(O):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_dtype_paths_agree(O):
    """f16 / bf16 storage gives the same result as f32 storage of the same
    (exactly representable) values."""
    rng = np.random.default_rng(11)
    S, Hq, Hkv, D, B = 3, 4, 2, 16, 4
    lens = [7, 1, 12]
    NB = 12
    bt = random_tables(rng, lens, B, NB, 4)
    Kl = rng.standard_normal((S, Hkv, 12, D))
    Vl = rng.standard_normal((S, Hkv, 12, D))
    q = rng.standard_normal((S, Hq, D))
    for dt, npdt in (("f16", np.float16), ("bf16", None)):
        def rnd(x):
            if npdt is not None:
                return x.astype(npdt)
            return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        def bits(x):
            r = rnd(x)
            return r if npdt is not None else r.view(torch.int16).numpy().view(np.uint16)
        def wide(x):
            r = rnd(x)
            return r.astype(np.float64) if npdt is not None else r.double().numpy()
        kp, vp = scatter(wide(Kl), wide(Vl), bt, lens, NB, B, fill=0.0)
        a = O.paged_decode(bits(q), bits(kp), bits(vp), bt, np.array(lens, np.int32), 0.25,
                           num_kv_heads=Hkv, block_size=B, dtype=dt)
        c = decode_f64(O, wide(q), kp, vp, bt, lens, 0.25, Hkv, B)
        assert np.array_equal(a, c), dt


# ------------------------------------------------ the pages' worked example

def pin_worked_example_walk(O):
    """Gather follows the block table exactly as the worked example walks it."""
    fx = _golden("worked_example_60tok.json")
    B, L, table = fx["block_size"], fx["num_tokens"], fx["block_table"]
    NB, D = 16, 2
    kp = np.full((NB, 1, B, D), np.nan, np.float32)
    vp = np.full((NB, 1, B // 16, D, 16), np.nan, np.float32)
    for p in range(NB):
        for s in range(B):
            kp[p, 0, s] = [p, s]          # K row encodes (physical block, slot)
            vp[p, 0, s // 16, :, s % 16] = [-p, -s]
    bt = np.array([table], np.int32)
    K, V = O.gather(kp, vp, bt, 0, 0, L, num_kv_heads=1, head_dim=D, block_size=B, dtype="f32")
    t = 0
    for step in fx["walk"]:
        for s in range(step["tokens"]):
            assert K[t, 0] == step["physical"] and K[t, 1] == s, (t, K[t])
            assert V[t, 0] == -step["physical"] and V[t, 1] == -s, (t, V[t])
            t += 1
    assert t == L == K.shape[0]


def pin_worked_example_paged_equals_contiguous(O):
    """Paged result == contiguous attention on the same logical K/V
    (bitwise, same summation order) and == torch SDPA (1e-12)."""
    fx = _golden("worked_example_60tok.json")
    B, L, table = fx["block_size"], fx["num_tokens"], fx["block_table"]
    rng = np.random.default_rng(60)
    D, NB = 128, 16
    Kl = f32_normal(rng, (1, 1, L, D))
    Vl = f32_normal(rng, (1, 1, L, D))
    q = f32_normal(rng, (1, 1, D))
    scale = float(np.float32(1 / math.sqrt(D)))
    kp, vp = scatter(Kl, Vl, [table], [L], NB, B)
    bt = np.array([table], np.int32)
    paged = decode_f64(O, q, kp, vp, bt, [L], scale, 1, B)[0, 0]
    contig = O.attention(q[0, 0], Kl[0, 0], Vl[0, 0], scale)
    assert np.array_equal(paged, contig)
    assert np.max(np.abs(paged - sdpa(q[0, 0], Kl[0, 0], Vl[0, 0], scale))) < 1e-12
    assert np.all(np.isfinite(paged))  # NaN in slots 12..15 of block 4 and unused blocks


# ------------------------------------------------------------ closed forms

def pin_single_token_returns_value_row(O):
    rng = np.random.default_rng(1)
    D, B, NB = 8, 4, 5
    Kl = f32_normal(rng, (1, 1, 1, D))
    Vl = f32_normal(rng, (1, 1, 1, D))
    q = f32_normal(rng, (1, 1, D))
    kp, vp = scatter(Kl, Vl, [[3]], [1], NB, B)
    out = decode_f64(O, q, kp, vp, np.array([[3]], np.int32), [1], 0.7, 1, B)
    assert np.array_equal(out[0, 0], Vl[0, 0, 0])


def pin_zero_query_gives_mean_of_exactly_L_values(O):
    """q = 0 -> every score 0 -> weights 1/L: the mean over exactly the
    attended tokens (a slack slot of the partial last block would shift it;
    here the slack holds NaN)."""
    rng = np.random.default_rng(2)
    D, B, NB, L = 16, 16, 9, 37
    bt = random_tables(rng, [L], B, NB, 3)
    Kl = f32_normal(rng, (1, 1, L, D))
    Vl = f32_normal(rng, (1, 1, L, D), grid=8)
    kp, vp = scatter(Kl, Vl, bt, [L], NB, B)
    out = decode_f64(O, np.zeros((1, 1, D)), kp, vp, bt, [L], 0.3, 1, B)[0, 0]
    assert np.max(np.abs(out - Vl[0, 0].mean(axis=0))) < 1e-13


def pin_dominant_score_selects_value_row(O):
    rng = np.random.default_rng(3)
    D, B, NB, L = 8, 4, 6, 19
    bt = random_tables(rng, [L], B, NB, 5)
    Kl = f32_normal(rng, (1, 1, L, D))
    Vl = f32_normal(rng, (1, 1, L, D))
    q = f32_normal(rng, (1, 1, D))
    s = Kl[0, 0] @ q[0, 0]
    kp, vp = scatter(Kl, Vl, bt, [L], NB, B)
    out = decode_f64(O, q, kp, vp, bt, [L], 1e6, 1, B)[0, 0]
    assert np.max(np.abs(out - Vl[0, 0, int(np.argmax(s))])) < 1e-12


def pin_two_tokens_by_hand(O):
    """D = 1, L = 2: out = (v0 e^s0 + v1 e^s1) / (e^s0 + e^s1), s_i = c q k_i."""
    q, k0, k1, v0, v1, c = 1.5, 0.25, -2.0, 3.0, -1.0, 0.5
    s0, s1 = c * q * k0, c * q * k1
    want = (v0 * math.exp(s0) + v1 * math.exp(s1)) / (math.exp(s0) + math.exp(s1))
    kp = np.full((3, 1, 2, 1), np.nan)
    vp = np.full((3, 1, 1, 1, 2), np.nan)
    kp[2, 0, 0, 0], kp[2, 0, 1, 0] = k0, k1
    vp[2, 0, 0, 0, 0], vp[2, 0, 0, 0, 1] = v0, v1
    out = decode_f64(O, [[[q]]], kp, vp, np.array([[2]], np.int32), [2], c, 1, 2)
    assert abs(out[0, 0, 0] - want) < 1e-15


def pin_empty_sequence_is_zero(O):
    kp = np.full((2, 1, 4, 3), np.nan)
    vp = np.full((2, 1, 1, 3, 4), np.nan)
    out = decode_f64(O, np.ones((1, 1, 3)), kp, vp, np.array([[-1]], np.int32), [0], 1.0, 1, 4)
    assert np.array_equal(out, np.zeros((1, 1, 3)))


def pin_table_out_of_range_is_an_error(O):
    kp = np.zeros((2, 1, 4, 3))
    vp = np.zeros((2, 1, 1, 3, 4))
    try:
        decode_f64(O, np.ones((1, 1, 3)), kp, vp, np.array([[2]], np.int32), [3], 1.0, 1, 4)
    except ValueError:
        return
    raise AssertionError("out-of-range table entry accepted")


# ------------------------------------------------------------- invariants

def _case(seed, S=3, Hq=4, Hkv=2, D=16, B=4, lens=(9, 16, 3), grid=None):
    rng = np.random.default_rng(seed)
    Lmax = max(lens)
    Kl = f32_normal(rng, (S, Hkv, Lmax, D), grid)
    Vl = f32_normal(rng, (S, Hkv, Lmax, D), grid)
    q = f32_normal(rng, (S, Hq, D), grid)
    return rng, Kl, Vl, q, list(lens)


def pin_block_permutation_invariance(O):
    rng, Kl, Vl, q, lens = _case(4)
    B, NB = 4, 14
    outs = []
    for _ in range(3):
        bt = random_tables(rng, lens, B, NB, 4)
        kp, vp = scatter(Kl, Vl, bt, lens, NB, B)
        outs.append(decode_f64(O, q, kp, vp, bt, lens, 0.25, 2, B))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def pin_block_size_invariance(O):
    rng, Kl, Vl, q, lens = _case(5, lens=(13, 32, 5))
    ref = None
    for B in (1, 2, 16, 32, 13):
        nbl = [-(-L // B) for L in lens]
        NB = sum(nbl) + 3
        bt = random_tables(rng, lens, B, NB, max(nbl))
        kp, vp = scatter(Kl, Vl, bt, lens, NB, B)
        out = decode_f64(O, q, kp, vp, bt, lens, 0.25, 2, B)
        if ref is None:
            ref = out
        assert np.array_equal(out, ref), B


def pin_key_shift_invariance(O):
    """Adding the same vector u to every key shifts every score by
    scale * q.u = 800 and must not change the output; e^800 overflows fp64,
    so skipping the max subtraction fails here."""
    rng = np.random.default_rng(6)
    D, B, NB, L = 8, 4, 7, 21
    bt = random_tables(rng, [L], B, NB, 6)
    Kl = f32_normal(rng, (1, 1, L, D), grid=10)
    Vl = f32_normal(rng, (1, 1, L, D))
    q = np.zeros((1, 1, D))
    q[0, 0, 3] = 2.0
    scale = 0.125
    Ks = Kl.copy()
    Ks[..., 3] += 800.0 / (scale * 2.0)  # exact in float32 on the 2**-10 grid
    kp, vp = scatter(Kl, Vl, bt, [L], NB, B)
    kps, _ = scatter(Ks, Vl, bt, [L], NB, B)
    a = decode_f64(O, q, kp, vp, bt, [L], scale, 1, B)
    b = decode_f64(O, q, kps, vp, bt, [L], scale, 1, B)
    assert np.all(np.isfinite(b))
    assert np.max(np.abs(a - b)) < 1e-12


def pin_output_in_convex_hull_of_values(O):
    rng, Kl, Vl, q, lens = _case(7)
    B, NB = 4, 12
    bt = random_tables(rng, lens, B, NB, 4)
    kp, vp = scatter(Kl, Vl, bt, lens, NB, B)
    out = decode_f64(O, q, kp, vp, bt, lens, 2.0, 2, B)
    for b, L in enumerate(lens):
        for h in range(4):
            V = Vl[b, h // 2, :L]
            assert np.all(out[b, h] >= V.min(axis=0) - 1e-14)
            assert np.all(out[b, h] <= V.max(axis=0) + 1e-14)


def pin_grouped_query_mapping(O):
    """Query head h reads KV head h // G (consecutive grouping); compared
    with torch SDPA on K/V repeated G times along the head axis."""
    rng = np.random.default_rng(8)
    S, Hq, Hkv, D, B = 2, 8, 2, 16, 4
    lens = [11, 6]
    NB = 10
    Kl = f32_normal(rng, (S, Hkv, 11, D))
    Vl = f32_normal(rng, (S, Hkv, 11, D))
    q = f32_normal(rng, (S, Hq, D))
    bt = random_tables(rng, lens, B, NB, 3)
    kp, vp = scatter(Kl, Vl, bt, lens, NB, B)
    out = decode_f64(O, q, kp, vp, bt, lens, 0.3, Hkv, B)
    for b, L in enumerate(lens):
        Kt = torch.from_numpy(Kl[b, :, :L]).repeat_interleave(Hq // Hkv, dim=0)
        Vt = torch.from_numpy(Vl[b, :, :L]).repeat_interleave(Hq // Hkv, dim=0)
        qt = torch.from_numpy(q[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=0.3)[:, 0]
        assert np.max(np.abs(out[b] - ref.numpy())) < 1e-12


def pin_attention_matches_library_sdpa(O):
    rng = np.random.default_rng(9)
    for L, D in ((1, 4), (5, 128), (300, 64), (64, 1)):
        q = rng.standard_normal(D)
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
        a = O.attention(q, K, V, 0.37)
        assert np.max(np.abs(a - sdpa(q, K, V, 0.37))) < 1e-12, (L, D)


def pin_bruteforce_small_shapes(O):
    """Many tiny random shapes against the independent numpy evaluation."""
    rng = np.random.default_rng(10)
    for trial in range(60):
        B = int(rng.choice([1, 2, 4, 16]))
        D = int(rng.choice([1, 2, 8]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4]))
        S = int(rng.integers(1, 4))
        lens = rng.integers(0, 41, size=S)
        lens[0] = max(lens[0], 1)
        nbl = [-(-int(L) // B) for L in lens]
        NB = sum(nbl) + int(rng.integers(0, 4))
        mbs = max(max(nbl), 1) + int(rng.integers(0, 2))
        bt = random_tables(rng, lens, B, NB, mbs)
        Lmax = max(int(lens.max()), 1)
        Kl = f32_normal(rng, (S, Hkv, Lmax, D))
        Vl = f32_normal(rng, (S, Hkv, Lmax, D))
        q = f32_normal(rng, (S, Hkv * G, D))
        scale = float(rng.uniform(0.05, 1.5))
        kp, vp = scatter(Kl, Vl, bt, lens, NB, B)
        got = decode_f64(O, q, kp, vp, bt, lens, scale, Hkv, B)
        want = numpy_reference(q, kp, vp, bt, lens, scale, Hkv, B)
        assert np.max(np.abs(got - want)) < 1e-12, trial


# ------------------------------------------------------------------ merge

def _rows(seed, L=45, D=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))


def pin_merge_of_block_partials_equals_one_softmax(O):
    """Split the sequence at every block boundary, fold the partials with
    the merge equation, normalise: equals the one-softmax result."""
    q, K, V = _rows(12)
    B, L, scale = 16, K.shape[0], 0.4
    acc = (-math.inf, 0.0, np.zeros(K.shape[1]))
    for t0 in range(0, L, B):
        acc = O.merge(acc, O.partial(q, K, V, t0, min(t0 + B, L), scale))
    m, l, o = acc
    ref = O.attention(q, K, V, scale)
    assert np.max(np.abs(o / l - ref)) < 1e-12
    full = O.partial(q, K, V, 0, L, scale)
    assert abs(m - full[0]) < 1e-15 and abs(l - full[1]) < 1e-12 * full[1]


def pin_merge_order_does_not_matter(O):
    q, K, V = _rows(13, L=64)
    scale, rng = 0.6, np.random.default_rng(14)
    parts = [O.partial(q, K, V, t0, t0 + 4, scale) for t0 in range(0, 64, 4)]
    ref = O.attention(q, K, V, scale)
    for _ in range(3):
        order = rng.permutation(len(parts))
        acc = (-math.inf, 0.0, np.zeros(K.shape[1]))
        for i in order:
            acc = O.merge(acc, parts[i])
        assert np.max(np.abs(acc[2] / acc[1] - ref)) < 1e-12
    # tree order
    level = parts
    while len(level) > 1:
        level = [O.merge(level[i], level[i + 1]) for i in range(0, len(level), 2)]
    assert np.max(np.abs(level[0][2] / level[0][1] - ref)) < 1e-12


def pin_empty_partial_is_merge_identity(O):
    q, K, V = _rows(15)
    p = O.partial(q, K, V, 3, 20, 0.5)
    e = O.partial(q, K, V, 7, 7, 0.5)
    assert e[0] == -math.inf and e[1] == 0.0 and not np.any(e[2])
    for r in (O.merge(e, p), O.merge(p, e)):
        assert r[0] == p[0] and r[1] == p[1] and np.array_equal(r[2], p[2])
    ee = O.merge(e, e)
    assert ee[0] == -math.inf and ee[1] == 0.0 and not np.any(ee[2])


# ------------------------------------------------ writing the cache
# "PagedAttention: The Cache Was Storing Nothing", §2.2 (the table maps
# logical to physical blocks; only the last block is partly filled) and
# §2.3 (a shared block is copied when a sequence diverges and writes).

def _append_case(seed, B, esize, S=3, H=2, D=16, lens=(9, 16, 3)):
    """Logical rows as raw element bits (uint16 patterns for esize 2,
    float32 values for esize 4) plus tables over a shuffled pool."""
    rng = np.random.default_rng(seed)
    lmax = max(lens)
    if esize == 2:
        rows = rng.integers(1, 65536, size=(2, S, H, lmax, D)).astype(np.float64)
    else:
        rows = rng.standard_normal((2, S, H, lmax, D)).astype(np.float32).astype(np.float64)
    nb = sum(-(-L // B) for L in lens)
    NB = nb + 3
    bt = random_tables(rng, lens, B, NB, max(-(-L // B) for L in lens) + 1)
    return rows[0], rows[1], bt, np.asarray(lens, np.int32), NB


def _storage(x, esize):
    return x.astype(np.uint16) if esize == 2 else x.astype(np.float32)


def _append_all(O, Klog, Vlog, bt, lens, NB, B, esize, fill):
    """Append every token of every sequence, one decode step at a time,
    into pools that start filled with `fill`."""
    S, H, lmax, D = Klog.shape
    Gv = vgroup(B)
    kp = _storage(np.full((NB, H, B, D), fill), esize)
    vp = _storage(np.full((NB, H, B // Gv, D, Gv), fill), esize)
    for t in range(lmax):
        pos = np.where(t < lens, t, -1).astype(np.int32)
        kp, vp = O.append(_storage(Klog[:, :, t, :], esize), _storage(Vlog[:, :, t, :], esize),
                          kp, vp, bt, pos)
    return kp, vp


def pin_append_places_tokens_like_an_independent_scatter(O):
    """Appending tokens 0..L-1 one step at a time builds, bit for bit, the
    pools that numpy fancy indexing builds from the same logical rows
    (16- and 32-bit elements; block sizes 4, 16, 32; every slot no token
    owns keeps its fill)."""
    for B in (4, 16, 32):
        for esize in (2, 4):
            Klog, Vlog, bt, lens, NB = _append_case(11 + B, B, esize)
            fill = 0 if esize == 2 else np.nan
            kp, vp = _append_all(O, Klog, Vlog, bt, lens, NB, B, esize, fill)
            kw, vw = scatter(Klog, Vlog, bt, lens, NB, B, fill=fill)
            assert np.array_equal(kp.view(np.uint8), _storage(kw, esize).view(np.uint8)), (B, esize)
            assert np.array_equal(vp.view(np.uint8), _storage(vw, esize).view(np.uint8)), (B, esize)


def pin_append_then_decode_matches_library_sdpa(O):
    """Tokens appended one by one and then read back by the decode oracle
    give torch's attention on the contiguous logical rows."""
    B = 16
    Klog, Vlog, bt, lens, NB = _append_case(5, B, 4, lens=(40, 17, 1))
    kp, vp = _append_all(O, Klog, Vlog, bt, lens, NB, B, 4, np.nan)
    rng = np.random.default_rng(6)
    S, H, _, D = Klog.shape
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    got = O.paged_decode(q, kp, vp, bt, lens, 0.25, num_kv_heads=H, block_size=B, dtype="f32")
    for b in range(S):
        for h in range(H):
            L = int(lens[b])
            want = sdpa(q[b, h].astype(np.float64), Klog[b, h, :L], Vlog[b, h, :L], 0.25)
            assert np.max(np.abs(got[b, h] - want)) < 1e-12


def pin_append_with_negative_positions_writes_nothing(O):
    Klog, Vlog, bt, lens, NB = _append_case(7, 16, 2)
    rng = np.random.default_rng(8)
    kp = rng.integers(0, 65536, size=(NB, 2, 16, 16)).astype(np.uint16)
    vp = rng.integers(0, 65536, size=(NB, 2, 1, 16, 16)).astype(np.uint16)
    k2, v2 = O.append(_storage(Klog[:, :, 0, :], 2), _storage(Vlog[:, :, 0, :], 2), kp, vp, bt,
                      np.full(3, -1, np.int32))
    assert np.array_equal(k2, kp) and np.array_equal(v2, vp)


def pin_append_out_of_range_is_an_error(O):
    Klog, Vlog, bt, lens, NB = _append_case(9, 16, 4)
    kp = np.zeros((NB, 2, 16, 16), np.float32)
    vp = np.zeros((NB, 2, 1, 16, 16), np.float32)
    for pos in ([bt.shape[1] * 16, -1, -1], [-1, 40, -1]):  # past the table row / unused entry
        try:
            O.append(_storage(Klog[:, :, 0, :], 4), _storage(Vlog[:, :, 0, :], 4), kp, vp, bt,
                     np.asarray(pos, np.int32))
        except ValueError:
            continue
        raise AssertionError(f"append at {pos} should be rejected")


def pin_copy_blocks_matches_numpy_assignment(O):
    """Block dst[i] of both pools becomes block src[i]; every other block
    is untouched (numpy fancy assignment as the reference)."""
    rng = np.random.default_rng(12)
    for (NB, H, B, esize) in ((20, 2, 16, 2), (9, 3, 32, 4), (12, 1, 4, 2)):
        Gv = vgroup(B)
        dt = np.uint16 if esize == 2 else np.uint32
        kp = rng.integers(0, 1 << (8 * esize), size=(NB, H, B, 8), dtype=np.uint64).astype(dt)
        vp = rng.integers(0, 1 << (8 * esize), size=(NB, H, B // Gv, 8, Gv), dtype=np.uint64).astype(dt)
        ids = rng.permutation(NB)
        n = NB // 3
        src, dst = ids[:n].astype(np.int32), ids[n: 2 * n].astype(np.int32)
        k2, v2 = O.copy_blocks(kp, vp, src, dst)
        kw, vw = kp.copy(), vp.copy()
        kw[dst] = kp[src]
        vw[dst] = vp[src]
        assert np.array_equal(k2, kw) and np.array_equal(v2, vw), (NB, H, B, esize)


def pin_copy_on_write_fork_keeps_the_original(O):
    """Two sequences share every block; before the fork appends into the
    shared last block, that block is copied and the fork's table entry
    repointed.  Afterwards each sequence attends to its own new token and
    the original is exactly what it would be without the fork."""
    B, H, D, L = 16, 2, 16, 21
    rng = np.random.default_rng(13)
    Klog = rng.standard_normal((1, H, L + 1, D)).astype(np.float32).astype(np.float64)
    Vlog = rng.standard_normal((1, H, L + 1, D)).astype(np.float32).astype(np.float64)
    NB = 6
    bt = np.asarray([[4, 1, -1]], np.int32)
    kp, vp = scatter(Klog, Vlog, bt, [L], NB, B)
    kp, vp = kp.astype(np.float32), vp.astype(np.float32)
    # fork: sequence 1 shares blocks 4, 1; its last block (1) is copied to 3
    kp, vp = O.copy_blocks(kp, vp, np.asarray([1], np.int32), np.asarray([3], np.int32))
    tables = np.asarray([[4, 1, -1], [4, 3, -1]], np.int32)
    new = rng.standard_normal((2, 2, H, D)).astype(np.float32)  # [k/v][seq][head][dim]
    kp, vp = O.append(new[0], new[1], kp, vp, tables, np.asarray([L, L], np.int32))
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    got = O.paged_decode(q, kp, vp, tables, np.asarray([L + 1, L + 1], np.int32), 0.3,
                         num_kv_heads=H, block_size=B, dtype="f32")
    for b in range(2):
        for h in range(H):
            K = np.concatenate([Klog[0, h, :L], new[0, b, h][None].astype(np.float64)])
            V = np.concatenate([Vlog[0, h, :L], new[1, b, h][None].astype(np.float64)])
            want = sdpa(q[b, h].astype(np.float64), K, V, 0.3)
            assert np.max(np.abs(got[b, h] - want)) < 1e-12


# ------------------------------------------- block-wise eviction scoring
# "PagedEviction: Structured Block-wise KV Cache Pruning ...": token
# importance ||V_t|| / ||K_t|| from the cached rows, block score = mean over
# the block, the lowest block evicted when the last block has just filled.

def _score_case(seed, lens, B, H=3, D=8, cfac=None, grid=None, fill=np.nan):
    """Logical K, V [S][H][Lmax][D] (fp64 values exact in float32), pools
    of the library layout on a shuffled table, `fill` in every other slot."""
    rng = np.random.default_rng(seed)
    S, lmax = len(lens), max(max(lens), 1)
    K = f32_normal(rng, (S, H, lmax, D), grid=grid)
    V = f32_normal(rng, (S, H, lmax, D), grid=grid)
    if cfac is not None:  # V = c_j * K inside block j
        c = np.repeat(np.asarray(cfac, np.float64), B)[:lmax]
        V = K * c[None, None, :, None]
    nb = sum(-(-L // B) for L in lens)
    NB = nb + 5
    bt = random_tables(rng, lens, B, NB, max(-(-L // B) for L in lens) + 2)
    kp, vp = scatter(K, V, bt, lens, NB, B, fill=fill)
    return K, V, bt, np.asarray(lens, np.int32), kp.astype(np.float32), vp.astype(np.float32)


def _numpy_scores(K, V, lens, B, M):
    """Independent evaluation: np.linalg.norm over each token's whole row."""
    S = K.shape[0]
    sc = np.full((S, M), np.nan)
    ev = np.full(S, -1, np.int32)
    for b, L in enumerate(lens):
        full = int(L) // B
        if full:
            kn = np.linalg.norm(K[b, :, : full * B, :].transpose(1, 0, 2).reshape(full * B, -1), axis=1)
            vn = np.linalg.norm(V[b, :, : full * B, :].transpose(1, 0, 2).reshape(full * B, -1), axis=1)
            sc[b, :full] = (vn / kn).reshape(full, B).mean(axis=1)
        if L > 0 and L % B == 0:
            ev[b] = int(np.argmin(sc[b, :full]))
    return sc, ev


def pin_block_scores_match_numpy_norms(O):
    for B in (4, 16, 32):
        lens = [3 * B, 2 * B + 1, 0, 5 * B, B - 1]
        K, V, bt, L, kp, vp = _score_case(40 + B, lens, B)
        got, ev = O.block_scores(kp, vp, bt, L, dtype="f32")
        want, evw = _numpy_scores(K, V, lens, B, bt.shape[1])
        assert np.array_equal(np.isnan(got), np.isnan(want)), B
        ok = ~np.isnan(want)
        assert np.max(np.abs(got[ok] - want[ok]) / want[ok]) < 1e-12, B
        assert np.array_equal(ev, evw), (B, ev, evw)


def pin_block_score_is_the_value_key_ratio_closed_form(O):
    """V = c_j K inside block j: every token's ratio is |c_j|, so the block
    score is |c_j| and the evicted block is the smallest |c_j|."""
    B = 16
    c = [1.5, -0.25, 0.75, 2.0, -1.0]
    K, V, bt, L, kp, vp = _score_case(7, [5 * B], B, cfac=c, grid=6)
    got, ev = O.block_scores(kp, vp, bt, L, dtype="f32")
    assert np.max(np.abs(got[0, :5] - np.abs(c)) / np.abs(c)) < 1e-14
    assert np.all(np.isnan(got[0, 5:]))
    assert ev[0] == 1


def pin_eviction_only_when_the_last_block_just_filled(O):
    B = 16
    lens = [2 * B, 2 * B + 3, 0, 1, B]
    K, V, bt, L, kp, vp = _score_case(8, lens, B, fill=1.0)  # finite slack: a scored partial block shows
    got, ev = O.block_scores(kp, vp, bt, L, dtype="f32")
    assert ev[1] == -1 and ev[2] == -1 and ev[3] == -1
    assert ev[0] in (0, 1) and ev[4] == 0
    assert not np.isnan(got[1, :2]).any() and np.isnan(got[1, 2:]).all()  # partial block unscored
    assert np.isnan(got[2]).all() and np.isnan(got[3]).all()


def pin_equal_block_scores_pick_the_lowest_block(O):
    B = 4
    c = [2.0, 0.5, 1.0, 0.5, 0.5]
    K, V, bt, L, kp, vp = _score_case(9, [5 * B], B, cfac=c, grid=6)
    got, ev = O.block_scores(kp, vp, bt, L, dtype="f32")
    assert ev[0] == 1


def pin_block_scores_do_not_depend_on_physical_placement(O):
    B = 16
    lens = [4 * B, 3 * B + 5]
    K, V, bt, L, kp, vp = _score_case(10, lens, B)
    a, ea = O.block_scores(kp, vp, bt, L, dtype="f32")
    rng = np.random.default_rng(11)
    bt2 = random_tables(rng, lens, B, kp.shape[0], bt.shape[1])
    kp2, vp2 = scatter(K, V, bt2, lens, kp.shape[0], B)
    b, eb = O.block_scores(kp2.astype(np.float32), vp2.astype(np.float32), bt2, L, dtype="f32")
    assert np.array_equal(a, b, equal_nan=True) and np.array_equal(ea, eb)


# ------------------------------------------------------------ paged prefill
# Readings: the n_b query rows of sequence b are its newest tokens (row i at
# position L_b - n_b + i) and each attends tokens 0 .. its position.

def _prefill_case(seed, lens=(9, 16, 5), nq=(9, 4, 1), Hq=4, Hkv=2, D=16, B=4):
    rng = np.random.default_rng(seed)
    S, Lmax = len(lens), max(lens)
    Klog = f32_normal(rng, (S, Hkv, Lmax, D))
    Vlog = f32_normal(rng, (S, Hkv, Lmax, D))
    NB = sum(-(-L // B) for L in lens) + 3
    bt = random_tables(rng, lens, B, NB, -(-Lmax // B) + 1)
    kp, vp = scatter(Klog, Vlog, bt, lens, NB, B, fill=0.0)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = f32_normal(rng, (int(qs[-1]), Hq, D))
    scale = 1.0 / math.sqrt(D)
    return dict(q=q, kp=kp, vp=vp, bt=bt, lens=np.asarray(lens, np.int32), qs=qs,
                Klog=Klog, Vlog=Vlog, Hkv=Hkv, B=B, scale=scale)


def _prefill(O, c):
    return O.paged_prefill(c["q"].astype(np.float32), c["kp"].astype(np.float32),
                           c["vp"].astype(np.float32), c["bt"], c["lens"], c["qs"], c["scale"],
                           num_kv_heads=c["Hkv"], block_size=c["B"], dtype="f32")


def pin_prefill_matches_library_sdpa_with_bottom_right_causal_mask(O):
    c = _prefill_case(11)
    out = _prefill(O, c)
    Hq = c["q"].shape[1]
    G = Hq // c["Hkv"]
    for b, L in enumerate(c["lens"]):
        r0, r1 = int(c["qs"][b]), int(c["qs"][b + 1])
        n = r1 - r0
        pos = L - n + np.arange(n)
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        for h in range(Hq):
            qt = torch.from_numpy(c["q"][r0:r1, h])[None, None]
            K = torch.from_numpy(c["Klog"][b, h // G, :L])[None, None]
            V = torch.from_numpy(c["Vlog"][b, h // G, :L])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=mask,
                                                                   scale=c["scale"])[0, 0].numpy()
            assert np.allclose(out[r0:r1, h], ref, rtol=0, atol=1e-12), (b, h)


def pin_prefill_row_equals_decode_at_its_position(O):
    c = _prefill_case(12, lens=(13, 7, 20), nq=(5, 7, 3))
    out = _prefill(O, c)
    for b, L in enumerate(c["lens"]):
        r0, r1 = int(c["qs"][b]), int(c["qs"][b + 1])
        for i in range(r1 - r0):
            lens = np.zeros_like(c["lens"])
            lens[b] = L - (r1 - r0) + i + 1          # the sequence as it stood at that row
            q = np.zeros((len(c["lens"]),) + c["q"].shape[1:])
            q[b] = c["q"][r0 + i]
            ref = decode_f64(O, q, c["kp"], c["vp"], c["bt"], lens, c["scale"], c["Hkv"], c["B"])
            assert np.allclose(out[r0 + i], ref[b], rtol=0, atol=1e-13), (b, i)


def pin_prefill_first_prompt_row_is_value_row_zero(O):
    c = _prefill_case(13, lens=(6, 11), nq=(6, 11))
    out = _prefill(O, c)
    G = c["q"].shape[1] // c["Hkv"]
    for b in range(2):
        r0 = int(c["qs"][b])
        for h in range(c["q"].shape[1]):
            assert np.array_equal(out[r0, h], c["Vlog"][b, h // G, 0]), (b, h)


def pin_prefill_more_rows_than_tokens_is_an_error(O):
    c = _prefill_case(14, lens=(3, 5), nq=(4, 1))
    try:
        _prefill(O, c)
    except ValueError:
        return
    raise AssertionError("4 query rows over 3 cached tokens were accepted")


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
