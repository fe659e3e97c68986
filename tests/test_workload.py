"""The seeded input generator (host logic only)."""
import math

import numpy as np
import pytest

import workload


def _finite(x, dtype):
    if dtype == "bf16":
        return (x & 0x7F80) != 0x7F80
    return np.isfinite(x)


def test_deterministic():
    a, b = workload.make(3, 7, batch=3), workload.make(3, 7, batch=3)
    for f in ("seq_lens", "block_tables", "q", "k_pool", "v_pool"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=False) or \
            np.array_equal(getattr(a, f).view(np.uint16), getattr(b, f).view(np.uint16))
    c = workload.make(3, 8, batch=3)
    assert not np.array_equal(a.seq_lens, c.seq_lens)


def test_toy_workload_is_the_pages_example():
    w = workload.make(1)
    assert list(w.seq_lens) == [60] and w.block_tables.tolist() == [[7, 1, 12, 4]]
    assert w.num_blocks == 16 and w.dtype == "f32" and w.scale == np.float32(1 / math.sqrt(128))
    # slots 12..15 of the last block and every other block hold NaN
    assert np.isnan(w.k_pool[4, 0, 12:]).all() and np.isfinite(w.k_pool[4, 0, :12]).all()
    assert np.isnan(w.v_pool[4, 0, 0, :, 12:]).all() and np.isfinite(w.v_pool[4, 0, 0, :, :12]).all()
    for p in set(range(16)) - {7, 1, 12, 4}:
        assert np.isnan(w.k_pool[p]).all() and np.isnan(w.v_pool[p]).all()


@pytest.mark.parametrize("cfg,lo,hi", [(2, 128, 2048), (3, 512, 8192), (5, 16, 16384)])
def test_lengths_in_range(cfg, lo, hi):
    w = workload.make(cfg, 11, batch=48)
    assert w.seq_lens.min() >= lo and w.seq_lens.max() <= hi


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_tables_and_sentinels(cfg):
    w = workload.make(cfg, 12, batch={2: 8, 3: 6, 5: 24}[cfg])
    nb = w.blocks_per_seq()
    B = w.block_size
    for b in range(w.num_seqs):
        row = w.block_tables[b]
        assert (row[: nb[b]] >= 0).all() and (row[: nb[b]] < w.num_blocks).all()
        assert (row[nb[b]:] == -1).all()
        last = int(row[nb[b] - 1])
        valid = int(w.seq_lens[b]) - (int(nb[b]) - 1) * B
        assert _finite(w.k_pool[last, :, :valid], w.dtype).all()
    used = set(int(x) for x in w.block_tables[w.block_tables >= 0])
    for p in range(w.num_blocks):
        if p not in used:
            assert not _finite(w.k_pool[p], w.dtype).any()
            assert not _finite(w.v_pool[p], w.dtype).any()


def test_private_blocks_are_distinct_and_pool_is_125_percent_of_demand():
    w = workload.make(3, 13)
    ids = w.block_tables[w.block_tables >= 0]
    assert len(set(ids.tolist())) == ids.size
    assert w.num_blocks == math.ceil(1.25 * int(w.blocks_per_seq().sum()))


def test_prefix_groups_share_their_first_32_blocks():
    w = workload.make(5, 14, batch=32)
    nb = w.blocks_per_seq()
    for g0 in range(0, 32, 8):
        grp = range(g0, g0 + 8)
        longest = max(grp, key=lambda b: nb[b])
        pref = w.block_tables[longest, : min(32, nb[longest])]
        for b in grp:
            k = min(32, int(nb[b]))
            assert np.array_equal(w.block_tables[b, :k], pref[:k])
    private = [int(x) for b in range(32) for x in w.block_tables[b, 32: nb[b]]]
    assert len(set(private)) == len(private)
    groups = [set(w.block_tables[g0, :32].tolist()) for g0 in range(0, 32, 8)]
    assert all(not (groups[i] & groups[j]) for i in range(4) for j in range(i))


def test_long_context_k_scaled_per_kv_head():
    w = workload.make(4, 15, batch=1, max_len=4096)
    k = workload.torch.from_numpy(w.k_pool.view(np.int16)).view(workload.torch.bfloat16).float().numpy()
    ref = w.block_tables[0, 0]
    stds = [float(np.nanstd(k[w.block_tables[0, :64], h])) for h in range(8)]
    assert all(0.4 < s < 2.2 for s in stds) and max(stds) / min(stds) > 1.2
    assert ref >= 0


def test_unique_bytes_count_shared_blocks_once():
    w = workload.make(5, 16, batch=16)
    assert workload.kv_bytes(w, unique=True) < workload.kv_bytes(w)
    w3 = workload.make(3, 16, batch=4)
    assert workload.kv_bytes(w3, unique=True) == workload.kv_bytes(w3)
    assert workload.kv_bytes(w3) == int(w3.seq_lens.sum()) * 2 * 8 * 128 * 2
