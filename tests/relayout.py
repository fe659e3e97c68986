"""Test-side input transforms: read a workload's logical K/V back out of
its paged pools and lay the same values out again differently (another
block size, another physical placement), or shift every key of a (sequence,
KV head) by one vector.  Pure data movement and input rounding; none of the
attention arithmetic."""
from __future__ import annotations

import dataclasses

import numpy as np

import workload


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage of `dtype` -> float32 (exact)."""
    if dtype == "bf16":
        return (np.ascontiguousarray(x).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, np.float32)


def logical_kv(w):
    """Per sequence b: (K, V), each [L_b][Hkv][D] in storage type, token t
    taken from slot t % B of table entry t // B."""
    B = w.block_size
    out = []
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        t = np.arange(L)
        phys = w.block_tables[b, t // B].astype(np.int64)
        s = t % B
        K = w.k_pool[phys, :, s, :]                   # [L][Hkv][D]
        V = w.v_pool[phys, :, s // 16, :, s % 16]     # [L][Hkv][D]
        out.append((K, V))
    return out


def repack(w, block_size: int, seed: int, pool_factor: float = 1.25):
    """The same logical K/V (and q, lengths, scale) in a fresh pool of
    `block_size`-token blocks placed by a seeded random permutation.
    Unattended slots and unreferenced blocks hold NaN."""
    B = block_size
    assert B % 16 == 0
    rng = np.random.default_rng(seed)
    lens = w.seq_lens.astype(np.int64)
    nb = (lens + B - 1) // B
    demand = int(nb.sum())
    NB = max(1, int(np.ceil(pool_factor * demand)))
    ids = rng.permutation(NB)
    mbs = max(1, int(nb.max()) if w.num_seqs else 1)
    bt = np.full((w.num_seqs, mbs), -1, np.int32)
    Hkv, D = w.num_kv_heads, w.head_dim
    nan = workload._nan_value(w.dtype)
    kp = np.full((NB, Hkv, B, D), nan, dtype=w.k_pool.dtype)
    vp = np.full((NB, Hkv, B // 16, D, 16), nan, dtype=w.v_pool.dtype)
    nxt = 0
    for b, (K, V) in enumerate(logical_kv(w)):
        n = int(nb[b])
        bt[b, :n] = ids[nxt: nxt + n]
        nxt += n
        t = np.arange(int(lens[b]))
        phys = bt[b, t // B].astype(np.int64)
        s = t % B
        kp[phys, :, s, :] = K
        vp[phys, :, s // 16, :, s % 16] = V
    return dataclasses.replace(w, block_size=B, num_blocks=NB, max_blocks_per_seq=mbs,
                               block_tables=bt, k_pool=kp, v_pool=vp, shared_prefix_blocks=0)


def shift_keys(w, c: float, head_in_group: int = 0):
    """Every attended key of (b, kvh) plus u = c * q / (scale * |q|^2) for
    q the query of head kvh*G + head_in_group, computed in float32 and
    rounded once to the storage type.  Exact arithmetic would shift that
    head's scores by c and every other head's scores by a constant, which
    leaves attention unchanged; the rounded keys are the new inputs."""
    B, G = w.block_size, w.group
    kp = w.k_pool.copy()
    scale = np.float32(w.scale)
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        phys = w.block_tables[b, t // B].astype(np.int64)
        s = t % B
        for kvh in range(w.num_kv_heads):
            q = to_f32(w.q[b, kvh * G + head_in_group], w.dtype)
            u = np.float32(c) * q / (scale * np.float32(np.dot(q, q)))
            k = to_f32(kp[phys, kvh, s, :], w.dtype) + u[None, :]
            kp[phys, kvh, s, :] = workload.round_to(k, w.dtype).reshape(k.shape)
    return dataclasses.replace(w, k_pool=kp)


def zero_queries(w):
    return dataclasses.replace(w, q=np.zeros_like(w.q))
