"""GPU parity of the cache writes (append one decode token per sequence,
copy-on-write block copy) through the C ABI against the oracle's
byte-level definition.  Pure data movement, so the bar is bit-exact: every
byte of both pools, touched or not, equals the oracle's pools.  The last
test closes the decode loop: append, then decode the grown sequences
against the fp64 oracle on the oracle's appended pools."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_196_amd as pa
import workload
from tests.gpu_util import TOL, device_tensor, max_err

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.load()


def _raw(t: torch.Tensor) -> np.ndarray:
    """Bytes of a device tensor on the host."""
    torch.cuda.synchronize()
    if t.element_size() == 2:
        return t.view(torch.int16).cpu().numpy().view(np.uint8).ravel()
    return t.view(torch.int32).cpu().numpy().view(np.uint8).ravel()


def _grow_tables(w, rng, skip_every=0):
    """Positions for the next decode token of every sequence (slot L_b);
    where L_b starts a new block, an unreferenced block is assigned to the
    table first (the caller's job before an append).  Returns the new
    tables and the positions (-1 for skipped sequences)."""
    bt = w.block_tables.copy()
    used = set(int(x) for x in bt[bt >= 0].ravel())
    free = [i for i in rng.permutation(w.num_blocks) if int(i) not in used]
    pos = w.seq_lens.astype(np.int32).copy()
    B = w.block_size
    for b in range(w.num_seqs):
        if skip_every and b % skip_every == 1:
            pos[b] = -1
            continue
        j = int(pos[b]) // B
        assert j < bt.shape[1], "table row too short for the next token"
        if pos[b] % B == 0:
            bt[b, j] = free.pop()
    return bt, pos


def _new_rows(w, rng):
    shape = (w.num_seqs, w.num_kv_heads, w.head_dim)
    k = workload.round_to(rng.standard_normal(shape, dtype=np.float32), w.dtype).reshape(shape)
    v = workload.round_to(rng.standard_normal(shape, dtype=np.float32), w.dtype).reshape(shape)
    return k, v


def _desc(w, num_seqs=None):
    return pa.PaDesc(w.num_seqs if num_seqs is None else num_seqs, w.num_kv_heads, w.num_kv_heads,
                     w.head_dim, w.block_size, w.num_blocks, w.max_blocks_per_seq,
                     {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16}[w.dtype], pa.PA_F32, 0)


def _append_case(O, w, seed, skip_every=0):
    rng = np.random.default_rng(seed)
    bt, pos = _grow_tables(w, rng, skip_every)
    kn, vn = _new_rows(w, rng)
    # the data-dependent preconditions are checked on the host before launching
    assert pa.pa_validate_append_host(_desc(w), np.ascontiguousarray(bt), pos) == 0
    k = device_tensor(w.k_pool, w.dtype)
    v = device_tensor(w.v_pool, w.dtype)
    pa.append(device_tensor(kn, w.dtype), device_tensor(vn, w.dtype), k, v,
              torch.from_numpy(bt).cuda(), torch.from_numpy(pos).cuda())
    kw, vw = O.append(kn, vn, w.k_pool, w.v_pool, bt, pos)
    assert np.array_equal(_raw(k), kw.view(np.uint8).ravel()), "k_pool differs"
    assert np.array_equal(_raw(v), vw.view(np.uint8).ravel()), "v_pool differs"
    return bt, pos, kw, vw


@pytest.mark.parametrize("dtype,B,H", [("bf16", 16, (8, 2)), ("f16", 32, (8, 8)), ("f32", 16, (1, 1)),
                                       ("bf16", 32, (32, 8))])
def test_append_bit_exact(O, dtype, B, H):
    """Lengths around block boundaries (the next token opens a new block
    where L % B == 0), every other sequence skipped in a second pass."""
    lens = [1, 15, 16, 17, 31, 32, 33, 200, 511, 512]
    w = workload.build(name="append", dtype=dtype, seq_lens=lens, num_q_heads=H[0],
                       num_kv_heads=H[1], head_dim=128, block_size=B, seed=7,
                       max_blocks_per_seq=-(-513 // B) + 1)
    for skip in (0, 2):
        _log(f"[kv_write] append {dtype} B={B} H={H} skip_every={skip}")
        _append_case(O, w, 100 + skip, skip_every=skip)


def test_append_full_size_gqa_batch(O):
    """The benchmark's configuration: the GQA batch-64 workload, one new
    token per sequence; both pools compared byte for byte."""
    w = workload.make(3)
    _log("[kv_write] append full-size gqa-b64")
    _append_case(O, w, 3)


@pytest.mark.parametrize("dtype,B,Hkv,n", [("bf16", 16, 8, 1), ("bf16", 16, 8, 1500), ("f16", 32, 2, 37),
                                           ("f32", 16, 1, 9)])
def test_copy_blocks_bit_exact(O, dtype, B, Hkv, n):
    """Random sources (repeats allowed) into distinct fresh destinations;
    1500 pairs of 32 KiB blocks exceed one pass of the copy grid."""
    lens = list(np.random.default_rng(1).integers(1, 900, size=24))
    w = workload.build(name="copy", dtype=dtype, seq_lens=lens, num_q_heads=Hkv, num_kv_heads=Hkv,
                       head_dim=128, block_size=B, seed=9, num_blocks=2 * n + 2000)
    rng = np.random.default_rng(n)
    ids = rng.permutation(w.num_blocks)
    dst = ids[:n].astype(np.int32)
    src = rng.choice(ids[n:], size=n).astype(np.int32)
    assert pa.pa_validate_copy_host(_desc(w), src, dst, n) == 0
    k = device_tensor(w.k_pool, w.dtype)
    v = device_tensor(w.v_pool, w.dtype)
    _log(f"[kv_write] copy {dtype} B={B} Hkv={Hkv} n={n}")
    pa.copy_blocks(k, v, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    kw, vw = O.copy_blocks(w.k_pool, w.v_pool, src, dst)
    assert np.array_equal(_raw(k), kw.view(np.uint8).ravel()), "k_pool differs"
    assert np.array_equal(_raw(v), vw.view(np.uint8).ravel()), "v_pool differs"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fork_append_decode_loop(O, dtype):
    """One decode step of a forked batch: every sequence gets a twin that
    shares all its blocks; the twin's partly filled last block is copied
    (copy-on-write) before each appends its own next token; then both
    decode.  GPU decode on GPU-written pools vs the fp64 oracle on the
    oracle-written pools."""
    lens = [5, 16, 40, 100, 257]
    S = len(lens)
    Hq, Hkv = (8, 2) if dtype == "bf16" else (2, 2)
    w = workload.build(name="fork", dtype=dtype, seq_lens=lens + lens, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=128, block_size=16, seed=21,
                       tables=None, prefix_group=0, num_blocks=200, max_blocks_per_seq=20)
    bt = w.block_tables.copy()
    bt[S:] = bt[:S]  # twins share every block of their originals
    rng = np.random.default_rng(22)
    used = set(int(x) for x in bt[bt >= 0].ravel())
    free = [int(i) for i in rng.permutation(w.num_blocks) if int(i) not in used]
    src, dst = [], []
    for b in range(S, 2 * S):
        L = lens[b - S]
        if L % 16:  # partly filled shared block: copy before writing into it
            j = L // 16
            src.append(int(bt[b, j]))
            dst.append(free.pop())
            bt[b, j] = dst[-1]
    for b in range(2 * S):
        L = (lens + lens)[b]
        if L % 16 == 0:
            bt[b, L // 16] = free.pop()
    src = np.asarray(src, np.int32)
    dst = np.asarray(dst, np.int32)
    pos = np.asarray(lens + lens, np.int32)
    d = _desc(w)
    assert pa.pa_validate_copy_host(d, src, dst, len(src)) == 0
    assert pa.pa_validate_append_host(d, np.ascontiguousarray(bt), pos) == 0
    kn, vn = _new_rows(w, rng)
    k = device_tensor(w.k_pool, w.dtype)
    v = device_tensor(w.v_pool, w.dtype)
    tb = torch.from_numpy(bt).cuda()
    _log(f"[kv_write] fork/append/decode {dtype}")
    pa.copy_blocks(k, v, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    pa.append(device_tensor(kn, dtype), device_tensor(vn, dtype), k, v, tb, torch.from_numpy(pos).cuda())
    kw, vw = O.copy_blocks(w.k_pool, w.v_pool, src, dst)
    kw, vw = O.append(kn, vn, kw, vw, bt, pos)
    assert np.array_equal(_raw(k), kw.view(np.uint8).ravel())
    assert np.array_equal(_raw(v), vw.view(np.uint8).ravel())
    lens1 = pos + 1
    out = pa.decode(device_tensor(w.q, dtype), k, v, tb, torch.from_numpy(lens1).cuda(), float(w.scale))
    ref = O.paged_decode(w.q, kw, vw, bt, lens1, np.float64(np.float32(w.scale)),
                         num_kv_heads=Hkv, block_size=16, dtype=dtype)
    err = max_err(out, ref)
    _log(f"[kv_write] fork decode {dtype} max_abs_err={err:.3e}")
    assert err <= TOL[dtype]
    # twins differ only by the new token: their outputs must differ
    assert not np.array_equal(ref[:S], ref[S:])


def test_block_manager_drives_fork_append_evict_decode(O):
    """One serving step end to end through the library: the host block
    manager allocates every sequence's blocks and forks each one (its twin
    shares all blocks), prepares the next token's slot (fresh blocks at
    block boundaries, copy-on-write pairs for shared partly filled blocks);
    the GPU copies and appends and decodes; the scan chooses a block to
    evict for every sequence whose last block just filled, the manager
    releases it and the tables are compacted; the GPU decodes again.  Each
    decode is compared with the fp64 oracle on the oracle's own pools."""
    B, Hq, Hkv, NB = 16, 8, 2, 400
    lens0 = [5, 15, 16, 47, 100, 129]
    S = len(lens0)
    bm = pa.BlockManager(NB, B)
    M = 16
    bt = np.full((2 * S, M), -1, np.int32)
    for b, L in enumerate(lens0):
        st, ids = bm.alloc(-(-L // B))
        assert st == 0
        bt[b, : ids.size] = ids
        assert bm.share(ids) == 0
        bt[S + b] = bt[b]
    lens = np.asarray(lens0 + lens0, np.int32)
    w = workload.build(name="bm", dtype="bf16", seq_lens=lens, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=128, block_size=B, seed=31, tables=[list(r[r >= 0]) for r in bt],
                       num_blocks=NB, max_blocks_per_seq=M)
    bt = np.ascontiguousarray(w.block_tables)
    st, pos, src, dst = bm.prepare_append(bt, lens)
    assert st == 0 and list(pos) == list(lens)
    assert len(src) == sum(1 for L in lens0 if L % B)  # one copy per shared, partly filled block
    d = _desc(w)
    assert pa.pa_validate_copy_host(d, src, dst, len(src)) == 0
    assert pa.pa_validate_append_host(d, bt, pos) == 0
    rng = np.random.default_rng(32)
    kn, vn = _new_rows(w, rng)
    k, v = device_tensor(w.k_pool, "bf16"), device_tensor(w.v_pool, "bf16")
    _log("[kv_write] block manager: copy, append, decode")
    pa.copy_blocks(k, v, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    pa.append(device_tensor(kn, "bf16"), device_tensor(vn, "bf16"), k, v, torch.from_numpy(bt).cuda(),
              torch.from_numpy(pos).cuda())
    kw, vw = O.copy_blocks(w.k_pool, w.v_pool, src, dst)
    kw, vw = O.append(kn, vn, kw, vw, bt, pos)
    lens1 = lens + 1
    scale = np.float64(np.float32(w.scale))
    q = device_tensor(w.q, "bf16")
    out = pa.decode(q, k, v, torch.from_numpy(bt).cuda(), torch.from_numpy(lens1).cuda(), float(w.scale))
    ref = O.paged_decode(w.q, kw, vw, bt, lens1, scale, num_kv_heads=Hkv, block_size=B, dtype="bf16")
    assert max_err(out, ref) <= TOL["bf16"]
    # eviction for the sequences whose last block just filled
    sc, ev = pa.block_scores(k, v, torch.from_numpy(bt).cuda(), torch.from_numpy(lens1).cuda())
    ev = ev.cpu().numpy()
    wsc, wev = O.block_scores(kw, vw, bt, lens1, dtype="bf16")
    due = [b for b in range(2 * S) if lens1[b] % B == 0]
    assert due and all(ev[b] >= 0 for b in due) and all(ev[b] == -1 for b in range(2 * S) if b not in due)
    for b in due:
        if ev[b] != wev[b]:  # only a near-tie of the two lowest fp64 scores allows another choice
            w2 = np.sort(wsc[b, : lens1[b] // B])
            assert w2[1] - w2[0] <= 2e-4 * w2[0], (b, ev[b], wev[b])
        j = int(ev[b])
        assert bm.release([bt[b, j]]) == 0
        row = [int(x) for x in bt[b, : lens1[b] // B]]
        del row[j]
        bt[b] = -1
        bt[b, : len(row)] = row
        lens1[b] -= B
    out2 = pa.decode(q, k, v, torch.from_numpy(bt).cuda(), torch.from_numpy(lens1).cuda(), float(w.scale))
    ref2 = O.paged_decode(w.q, kw, vw, bt, lens1, scale, num_kv_heads=Hkv, block_size=B, dtype="bf16")
    err = max_err(out2, ref2)
    _log(f"[kv_write] block manager loop: decode after eviction max_abs_err={err:.3e}")
    assert err <= TOL["bf16"]
    live = set(int(x) for x in bt[bt >= 0].ravel())
    assert bm.num_free() == NB - len(live)
    bm.close()
