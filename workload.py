"""Seeded synthetic decode batches for paged decode attention.

Input generation only: this module draws sequence lengths, block tables
and q/K/V values and lays them out in the library's storage layout.  It
holds none of the attention arithmetic, and both the fp64 oracle and the
gfx950 library consume what it produces.

Storage layouts produced (element = one value of the config dtype):
    q        [S][Hq][D]
    k_pool   [num_blocks][Hkv][B][D]     token-major tile
    v_pool   [num_blocks][Hkv][B/16][D][16]   value rows transposed within
                                              each group of 16 tokens
    tables   int32 [S][max_blocks_per_seq], -1 in unused entries
    seq_lens int32 [S]
fp16 data is numpy float16; bf16 data is the raw bits as uint16; fp32 is
float32.  Values are drawn as float32 N(0,1) and rounded once to the
config dtype (round to nearest even).

Sentinels: every pool slot that no sequence attends (slots of a last block
beyond the longest referencing sequence, and whole unreferenced blocks)
holds NaN, so any read of a slot outside the attended range poisons the
result.

Workloads (the five decode configurations this library is measured on):
    1  toy: 1 sequence of 60 tokens, 1 query head = 1 KV head, D 128, fp32,
       B 16, pool of 16 blocks, block table [7, 1, 12, 4]  ("39 ·
       PagedAttention", §2 worked example)
    2  LLaMA-7B-shaped MHA: batch 8, 32/32 heads, fp16, B 16,
       L ~ U{128..2048}, blocks from a random permutation of a 4096 pool
    3  GQA: batch 64, 32/8 heads, bf16, B 16, L ~ U{512..8192}, shuffled
       pool of ceil(1.25 x demand) blocks
    4  long-context GQA: batch 4, 64/8 heads, bf16, B 32, L = 32768, K of
       KV head h scaled by c_h ~ U(0.5, 2) before rounding
    5  large-batch serving: batch 256, 32/8 heads, bf16, B 16,
       L = clip(round(lognormal(ln 1000, 1)), 16, 16384); groups of 8
       consecutive sequences share their first 32 physical blocks (a
       512-token common prefix); the rest shuffled from ceil(1.25 x demand)
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = ("f32", "f16", "bf16")
ESIZE = {"f32": 4, "f16": 2, "bf16": 2}
_NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    seq_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray  # int32 [S][max_blocks_per_seq]
    q: np.ndarray             # [S][Hq][D]
    k_pool: np.ndarray        # [NB][Hkv][B][D]
    v_pool: np.ndarray        # [NB][Hkv][B/16][D][16]
    scale: np.float32
    seed: int = 0
    shared_prefix_blocks: int = 0  # leading logical blocks shared within prefix groups
    # prefix groups: group i = sequences group_start[i] .. group_start[i+1]-1,
    # whose first group_shared[i] table entries are the same physical blocks
    group_start: np.ndarray = dataclasses.field(default_factory=lambda: np.zeros(1, np.int32))
    group_shared: np.ndarray = dataclasses.field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_groups(self) -> int:
        return int(self.group_shared.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    def blocks_per_seq(self) -> np.ndarray:
        B = self.block_size
        return (self.seq_lens.astype(np.int64) + B - 1) // B


def to_device(x: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    """Upload a storage array of workload dtype `dtype` (bf16 as raw uint16
    bits) as a torch tensor of that type on `dev`."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage of `dtype`, round to nearest even."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]


def _empty_pool(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, np.float32)
    if dtype == "f16":
        return np.full(shape, _NAN_BITS["f16"], np.uint16).view(np.float16)
    return np.full(shape, _NAN_BITS["bf16"], np.uint16)


def _nan_value(dtype: str):
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.uint16(_NAN_BITS["bf16"])


def build(*, name: str, dtype: str, seq_lens, num_q_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, seed: int, num_blocks: int | None = None,
          pool_factor: float = 1.25, max_blocks_per_seq: int | None = None,
          prefix_group: int = 0, prefix_blocks: int = 0, k_head_scale=None,
          tables=None, shuffle: bool = True, chunk_blocks: int = 2048,
          group_sizes=None, group_blocks=None) -> Workload:
    """General seeded builder; every named workload goes through it.

    seq_lens: int lengths (already drawn).  tables: explicit block tables
    (list of lists) instead of drawing them.  prefix_group > 0: consecutive
    groups of that many sequences share their first `prefix_blocks`
    physical blocks.  group_sizes / group_blocks: consecutive groups of the
    given sizes sharing the given numbers of leading blocks (sequences after
    the last group share nothing); a member shorter than its group's shared
    prefix holds only the shared blocks its length needs.  k_head_scale: per-KV-head multipliers applied to K in
    float32 before rounding.  num_blocks: pool size; default
    ceil(pool_factor * demand).
    """
    assert dtype in DTYPES
    rng_len, rng_blk, rng_q, rng_k, rng_v, _ = _streams(seed)
    del rng_len
    lens = np.asarray(seq_lens, np.int64)
    S = lens.shape[0]
    B = block_size
    nb = (lens + B - 1) // B
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(nb.max()) if S else 1)
    bt = np.full((S, max_blocks_per_seq), -1, np.int32)

    if tables is not None:
        for b, row in enumerate(tables):
            bt[b, : len(row)] = row
        assert num_blocks is not None
    else:
        if prefix_group > 0:
            groups = [list(range(s, min(s + prefix_group, S))) for s in range(0, S, prefix_group)]
            gblocks = [prefix_blocks] * len(groups)
        elif group_sizes is not None:
            groups, s0 = [], 0
            for n in group_sizes:
                groups.append(list(range(s0, s0 + n)))
                s0 += n
            assert s0 <= S, "groups exceed the batch"
            gblocks = [int(x) for x in group_blocks]
            assert len(gblocks) == len(groups)
        else:
            groups, gblocks = [], []
        covered = sum(len(g) for g in groups)
        shared_of = np.zeros(S, np.int64)
        for grp, k in zip(groups, gblocks):
            shared_of[grp] = k
        demand = int(sum(gblocks)) + int(np.maximum(nb - shared_of, 0).sum())
        if num_blocks is None:
            num_blocks = max(1, int(math.ceil(pool_factor * demand)))
        assert num_blocks >= demand, "pool smaller than demand"
        ids = rng_blk.permutation(num_blocks) if shuffle else np.arange(num_blocks)
        nxt = 0
        for grp, kg in zip(groups, gblocks):
            pref = ids[nxt: nxt + kg]
            nxt += kg
            for b in grp:
                k = min(kg, int(nb[b]))
                bt[b, :k] = pref[:k]
                rest = int(nb[b]) - k
                bt[b, k: k + rest] = ids[nxt: nxt + rest]
                nxt += rest
        for b in range(covered, S):
            bt[b, : nb[b]] = ids[nxt: nxt + nb[b]]
            nxt += int(nb[b])

    # Longest attended prefix of every physical block (0 = unreferenced).
    valid = np.zeros(num_blocks, np.int64)
    for b in range(S):
        n = int(nb[b])
        if n == 0:
            continue
        row = bt[b, :n].astype(np.int64)
        v = np.full(n, B, np.int64)
        v[-1] = int(lens[b]) - (n - 1) * B
        np.maximum.at(valid, row, v)
    ref = np.nonzero(valid)[0]

    Hkv, D = num_kv_heads, head_dim
    assert B % 16 == 0, "the library's V layout groups tokens by 16"
    NG = B // 16
    k_pool = _empty_pool((num_blocks, Hkv, B, D), dtype)
    v_pool = _empty_pool((num_blocks, Hkv, NG, D, 16), dtype)
    kscale = None if k_head_scale is None else np.asarray(k_head_scale, np.float32).reshape(1, Hkv, 1, 1)
    for c0 in range(0, ref.shape[0], chunk_blocks):
        sel = ref[c0: c0 + chunk_blocks]
        kv = rng_k.standard_normal((sel.shape[0], Hkv, B, D), dtype=np.float32)
        if kscale is not None:
            kv *= kscale
        k_pool[sel] = round_to(kv, dtype).reshape(kv.shape).view(k_pool.dtype)
        vv = rng_v.standard_normal((sel.shape[0], Hkv, NG, D, 16), dtype=np.float32)
        v_pool[sel] = round_to(vv, dtype).reshape(vv.shape).view(v_pool.dtype)
    nanv = _nan_value(dtype)
    for p in np.nonzero((valid > 0) & (valid < B))[0]:
        k_pool[p, :, valid[p]:, :] = nanv
        for slot in range(int(valid[p]), B):
            v_pool[p, :, slot // 16, :, slot % 16] = nanv

    qf = rng_q.standard_normal((S, num_q_heads, D), dtype=np.float32)
    q = round_to(qf, dtype).reshape(qf.shape)
    if tables is None and groups:
        g_start = np.array([g[0] for g in groups] + [groups[-1][-1] + 1], np.int32)
        g_shared = np.array(gblocks, np.int32)
    else:
        g_start, g_shared = np.zeros(1, np.int32), np.zeros(0, np.int32)
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=Hkv,
                    head_dim=D, block_size=B, num_blocks=int(num_blocks),
                    max_blocks_per_seq=int(max_blocks_per_seq),
                    seq_lens=lens.astype(np.int32), block_tables=bt, q=q,
                    k_pool=k_pool, v_pool=v_pool,
                    scale=np.float32(1.0 / math.sqrt(head_dim)), seed=seed,
                    shared_prefix_blocks=int(prefix_blocks) if prefix_group > 1 else 0,
                    group_start=g_start, group_shared=g_shared)


CONFIG_NAMES = {
    1: "toy-60tok-mha1-f32-b16",
    2: "llama7b-mha-b8-h32-f16-b16",
    3: "gqa-b64-h32kv8-bf16-b16",
    4: "longctx-gqa-b4-h64kv8-bf16-b32-L32768",
    5: "serving-b256-h32kv8-bf16-b16-lognormal-prefix512",
}


def make(cfg: int, seed: int | None = None, *, batch: int | None = None,
         max_len: int | None = None) -> Workload:
    """One of the five named workloads.

    seed defaults to the config number.  batch / max_len shrink the batch
    or cap the drawn lengths (same distributions otherwise) for quick tests.
    """
    seed = cfg if seed is None else seed
    rng_len = _streams(seed)[0]
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        return build(name=name, dtype="f32", seq_lens=[60], num_q_heads=1, num_kv_heads=1,
                     head_dim=128, block_size=16, seed=seed, num_blocks=16,
                     max_blocks_per_seq=4, tables=[[7, 1, 12, 4]])
    if cfg == 2:
        S = batch or 8
        lens = rng_len.integers(128, 2048, size=S, endpoint=True)
        if max_len:
            lens = np.minimum(lens, max_len)
        return build(name=name, dtype="f16", seq_lens=lens, num_q_heads=32, num_kv_heads=32,
                     head_dim=128, block_size=16, seed=seed, num_blocks=4096,
                     max_blocks_per_seq=128)
    if cfg == 3:
        S = batch or 64
        lens = rng_len.integers(512, 8192, size=S, endpoint=True)
        if max_len:
            lens = np.minimum(lens, max_len)
        return build(name=name, dtype="bf16", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, block_size=16, seed=seed, max_blocks_per_seq=512)
    if cfg == 4:
        S = batch or 4
        L = max_len or 32768
        kscale = rng_len.uniform(0.5, 2.0, size=8).astype(np.float32)
        nblk = (L + 31) // 32
        return build(name=name, dtype="bf16", seq_lens=[L] * S, num_q_heads=64,
                     num_kv_heads=8, head_dim=128, block_size=32, seed=seed,
                     num_blocks=int(math.ceil(1.25 * S * nblk)), max_blocks_per_seq=nblk,
                     k_head_scale=kscale)
    if cfg == 5:
        S = batch or 256
        lens = np.exp(rng_len.normal(math.log(1000.0), 1.0, size=S))
        lens = np.clip(np.rint(lens), 16, 16384).astype(np.int64)
        if max_len:
            lens = np.minimum(lens, max_len)
        return build(name=name, dtype="bf16", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, block_size=16, seed=seed, max_blocks_per_seq=1024,
                     prefix_group=8, prefix_blocks=32)
    raise ValueError(f"unknown config {cfg}")


def mqa_name(num_q_heads: int, batch: int = 512) -> str:
    return f"mqa-b{batch}-h{num_q_heads}kv1-bf16-b16"


def make_mqa(num_q_heads: int, seed: int | None = None, *, batch: int | None = None,
             max_len: int | None = None) -> Workload:
    """Multi-query decode ("PagedAttention: The Cache Was Storing Nothing",
    §3.1: every query head shares one key head and one value head): the
    GQA decode workload's length distribution (uniform in [512, 8192],
    bf16, block size 16, head_dim 128, shuffled blocks, q/K/V ~ N(0, 1)) on
    one KV head with num_q_heads query heads (32 or 64), and 512 sequences,
    so that the (sequence, KV head) count and the K/V bytes match the GQA
    workload's 64 sequences x 8 KV heads."""
    seed = 30 + num_q_heads if seed is None else seed
    rng_len = _streams(seed)[0]
    S = batch or 512
    lens = rng_len.integers(512, 8192, size=S, endpoint=True)
    if max_len:
        lens = np.minimum(lens, max_len)
    return build(name=mqa_name(num_q_heads, S), dtype="bf16", seq_lens=lens,
                 num_q_heads=num_q_heads, num_kv_heads=1, head_dim=128, block_size=16, seed=seed,
                 max_blocks_per_seq=512)


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, esize: int, layers: int = 1) -> int:
    """K and V bytes one token occupies: 2 x KV heads x head dim x layers x
    element bytes ("PagedAttention: The Cache Was Storing Nothing", §3)."""
    return 2 * num_kv_heads * head_dim * layers * esize


def kv_bytes(w: Workload, unique: bool = False) -> int:
    """K+V bytes the attended tokens occupy: 2 * L * D * esize per
    (sequence, KV head), summed.  unique=True counts each physical
    (block, slot) once, so shared prefix blocks are counted once."""
    per_token = kv_bytes_per_token(w.num_kv_heads, w.head_dim, w.esize)
    if not unique:
        return int(w.seq_lens.astype(np.int64).sum()) * per_token
    B = w.block_size
    valid = np.zeros(w.num_blocks, np.int64)
    nb = w.blocks_per_seq()
    for b in range(w.num_seqs):
        n = int(nb[b])
        if n == 0:
            continue
        v = np.full(n, B, np.int64)
        v[-1] = int(w.seq_lens[b]) - (n - 1) * B
        np.maximum.at(valid, w.block_tables[b, :n].astype(np.int64), v)
    return int(valid.sum()) * per_token


def prefill_queries(w: Workload, q_lens, seed: int):
    """Query rows for a prefill over workload w's cache: sequence b gets
    q_lens[b] rows (its newest q_lens[b] tokens, 0 <= q_lens[b] <=
    seq_lens[b]).  Values N(0, 1), rounded once to w.dtype like the decode
    queries.  Returns (q storage [sum q_lens][Hq][D], q_start int32 [S + 1])."""
    q_lens = np.asarray(q_lens, np.int64)
    assert q_lens.shape == (w.num_seqs,)
    assert np.all(q_lens >= 0) and np.all(q_lens <= w.seq_lens)
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    x = rng.standard_normal((int(q_start[-1]), w.num_q_heads, w.head_dim), dtype=np.float32)
    return round_to(x, w.dtype), q_start


PREFILL_NAME = "prefill GQA 32/8 heads, 8 whole prompts x 2048 tokens, bf16, B=16"


def prefill_workload(seed: int = 6, num_prompts: int = 8, prompt_len: int = 2048,
                     dtype: str = "bf16"):
    """Prompt prefill over the paged cache with the GQA batch's head shapes:
    num_prompts whole prompts of prompt_len tokens, their K/V already in
    shuffled physical blocks, every token a query row.  Returns
    (w, q storage [num_prompts * prompt_len][32][128], q_start)."""
    name = PREFILL_NAME if (num_prompts, prompt_len, dtype) == (8, 2048, "bf16") else \
        f"prefill GQA 32/8 heads, {num_prompts} whole prompts x {prompt_len} tokens, {dtype}, B=16"
    w = build(name=name, dtype=dtype, seq_lens=[prompt_len] * num_prompts,
              num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, seed=seed)
    q, q_start = prefill_queries(w, [prompt_len] * num_prompts, seed)
    return w, q, q_start
