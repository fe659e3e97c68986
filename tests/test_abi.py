"""The C ABI on the CPU: every declared symbol is exported, the host-side
entry points behave as include/pagedattn.h states, and argument errors are
reported before any device work.  No kernel is launched here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import paged_kv_cache_196_amd as pa
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    pa.ensure_built()
    return pa.load()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "pagedattn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[a-z_][\w\s\*]*?\b(pa_\w+|paged_\w+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 10
    assert sorted(pa.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in pa._lib.STATUS.items():
        assert pa.status_str(code).startswith(name)
    assert pa.status_str(12345) == "unknown pa_status"


def test_dtype_sizes():
    assert [pa.pa_dtype_size(d) for d in (pa.PA_F32, pa.PA_F16, pa.PA_BF16, 7)] == [4, 2, 2, 0]


def test_blocks_for_len_gives_the_printed_paged_slots():
    """pa_blocks_for_len against the printed paged-storage example of
    "FlashAttention vs PagedAttention" (section on attention intermediates
    and paged cache storage): requests of 19, 45 and 70 tokens in 16-token
    pages hold 32, 48 and 80 slots, 160 in all, 26 of them empty.  Its MiB
    lines are slot counts times one per-slot size, so they pin the same
    counts as ratios: paged / fixed 20 / 48 MiB = 160 / 384 slots and used /
    paged 16.75 / 20 MiB = 134 / 160 slots."""
    ex = json.load(open(os.path.join(GOLDEN, "sizing_examples.json")))["printed_paged_slots"]
    page = ex["page_tokens"]
    held = [pa.pa_blocks_for_len(n, page) * page for n in ex["request_tokens"]]
    assert held == ex["slots_per_request"]
    in_use = sum(ex["request_tokens"])
    assert sum(held) == ex["slots_held"] and sum(held) - in_use == ex["slots_empty"]
    assert sum(held) * ex["mib_fixed"] == ex["slots_fixed"] * ex["mib_paged"]
    assert in_use * ex["mib_paged"] == sum(held) * ex["mib_used"]
    u = json.load(open(os.path.join(GOLDEN, "sizing_examples.json")))["utilisation_200"]
    n = pa.pa_blocks_for_len(u["length"], u["block_size"])
    assert n == u["blocks"] and n * u["block_size"] == u["slots"]
    assert round(100 * u["length"] / (n * u["block_size"]), 1) == u["utilisation_percent"]
    assert pa.pa_blocks_for_len(0, 16) == 0 and pa.pa_blocks_for_len(-3, 16) == 0
    assert pa.pa_blocks_for_len(16, 16) == 1 and pa.pa_blocks_for_len(17, 16) == 2


def test_kv_bytes_per_token_matches_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "sizing_examples.json")))
    a = fx["llama7b_layer_bytes"]
    per_layer = a["tokens"] * workload.kv_bytes_per_token(a["kv_heads"], a["head_dim"], a["dtype_bytes"])
    assert per_layer == a["exact_bytes"] and round(per_layer / 1e6) == 34 and int(per_layer / 1e6) == a["approx_mb"]
    b = fx["llama3_70b_token_bytes"]
    assert workload.kv_bytes_per_token(b["kv_heads"], b["head_dim"], b["dtype_bytes"], b["layers"]) == b["kib_per_token"] * 1024


def _desc(**kw):
    d = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=64,
             max_blocks_per_seq=8, dtype=pa.PA_BF16, out_dtype=pa.PA_F32, kernel=pa.PA_KERNEL_AUTO)
    d.update(kw)
    return pa.PaDesc(**d)


@pytest.mark.parametrize("field,value,code", [
    ("num_q_heads", 0, 2), ("num_kv_heads", 3, 2), ("num_seqs", -1, 2), ("block_size", 0, 2),
    ("num_blocks", 0, 2), ("max_blocks_per_seq", 0, 2), ("dtype", 5, 3), ("out_dtype", pa.PA_F16, 3),
    ("head_dim", 64, 4), ("block_size", 8, 4), ("block_size", 48, 4), ("kernel", 9, 4),
    ("max_blocks_per_seq", 1 << 26, 4), ("cached_prefix_blocks", -1, 2),
])
def test_descriptor_errors(lib, field, value, code):
    assert pa.pa_check_desc(_desc()) == 0
    assert pa.pa_check_desc(_desc(**{field: value})) == code


def test_batches_beyond_one_launch_are_accepted(lib):
    """A batch of more than 8192 sequences is valid (the decode runs it as
    launches of at most 8192); the int32 flat-unit bound applies to one
    launch's sequences."""
    assert pa.pa_check_desc(_desc(num_seqs=9000)) == 0
    assert pa.pa_check_desc(_desc(num_seqs=1 << 20, max_blocks_per_seq=4096)) == 0
    # 8192 sequences x 32768 blocks x 8 KV heads = 2^31 units in one launch
    assert pa.pa_check_desc(_desc(num_seqs=9000, max_blocks_per_seq=1 << 15)) == 4
    assert pa.pa_check_desc(_desc(num_seqs=8191, max_blocks_per_seq=1 << 15)) == 0


def test_descriptor_fields_match_the_header():
    """The ctypes descriptor mirrors include/pagedattn.h field for field."""
    hdr = open(os.path.join(ROOT, "include", "pagedattn.h")).read()
    body = re.search(r"typedef struct pa_desc \{(.*?)\} pa_desc;", hdr, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [n for n, _ in pa.PaDesc._fields_]
    assert ctypes.sizeof(pa.PaDesc) == 4 * len(fields)


def test_mfma_with_fp32_is_unsupported(lib):
    assert pa.pa_check_desc(_desc(dtype=pa.PA_F32, kernel=pa.PA_KERNEL_MFMA)) == 4
    assert pa.pa_check_desc(_desc(dtype=pa.PA_F32, kernel=pa.PA_KERNEL_VALU)) == 0


def test_every_query_group_is_planned(lib):
    """Any number of query heads per KV head is accepted: a group the
    kernels hold directly (1-16, 32 and 64 heads on the matrix cores; 1, 2,
    4 on the vector ALU for 16-bit types, 1 for fp32) runs as one, a larger or odd
    one as virtual groups of the largest built size dividing it.  The
    workspace is sized by that kernel group, which pins the plan."""
    def ws(G, **kw):
        d = _desc(num_q_heads=2 * G, num_kv_heads=2, **kw)
        assert pa.pa_check_desc(d) == 0, (G, kw)
        return pa.pa_workspace_bytes(d)
    for kernel in (pa.PA_KERNEL_AUTO, pa.PA_KERNEL_MFMA, pa.PA_KERNEL_VALU):
        for G in (1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128):
            ws(G, kernel=kernel)
    per_head = ws(2) - ws(1)                       # one more head per kernel group
    assert per_head > 0 and ws(4) - ws(1) == 3 * per_head
    mf = pa.PA_KERNEL_MFMA
    assert ws(16, kernel=mf) == ws(1) + 15 * per_head
    assert ws(32, kernel=mf) == ws(1) + 31 * per_head and ws(64, kernel=mf) == ws(1) + 63 * per_head
    assert ws(128, kernel=mf) == ws(64, kernel=mf) and ws(96, kernel=mf) == ws(32, kernel=mf)
    assert ws(48, kernel=mf) == ws(16, kernel=mf)
    assert ws(12, kernel=mf) == ws(4, kernel=mf) and ws(24, kernel=mf) == ws(8, kernel=mf)
    assert ws(3, kernel=mf) == ws(5, kernel=mf) == ws(1)
    va = pa.PA_KERNEL_VALU
    assert ws(8, kernel=va) == ws(16, kernel=va) == ws(4, kernel=va) == ws(1) + 3 * per_head
    assert ws(6, kernel=va) == ws(2, kernel=va)
    for G in (2, 4, 8):
        assert ws(G, dtype=pa.PA_F32, kernel=va) == ws(1)


@pytest.mark.parametrize("B", [16, 32])
def test_element_offsets_match_the_workload_arrays(lib, B):
    w = workload.build(name="t", dtype="bf16", seq_lens=[40, 77], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=B, seed=3)
    d = pa.PaDesc(w.num_seqs, 8, 2, 128, B, w.num_blocks, w.max_blocks_per_seq, pa.PA_BF16, pa.PA_F32, 0)
    assert pa.pa_pool_bytes(d) == w.k_pool.nbytes == w.v_pool.nbytes
    rng = np.random.default_rng(0)
    for _ in range(200):
        blk, h, s, dim = (int(rng.integers(w.num_blocks)), int(rng.integers(2)), int(rng.integers(B)),
                          int(rng.integers(128)))
        assert pa.pa_k_elem_offset(d, blk, h, s, dim) == np.ravel_multi_index((blk, h, s, dim), w.k_pool.shape)
        assert pa.pa_v_elem_offset(d, blk, h, s, dim) == np.ravel_multi_index(
            (blk, h, s // 16, dim, s % 16), w.v_pool.shape)
    for bad in ((w.num_blocks, 0, 0, 0), (0, 2, 0, 0), (0, 0, B, 0), (0, 0, 0, 128), (-1, 0, 0, 0)):
        assert pa.pa_k_elem_offset(d, *bad) == -1 and pa.pa_v_elem_offset(d, *bad) == -1


def test_workspace_size_grows_with_group(lib):
    a = pa.pa_workspace_bytes(_desc(num_q_heads=8))
    b = pa.pa_workspace_bytes(_desc(num_q_heads=32))
    assert 0 < a < b
    assert pa.pa_workspace_bytes(_desc(head_dim=64)) == 0


def test_validate_host(lib):
    w = workload.make(5, 3, batch=16)
    d = pa.PaDesc(w.num_seqs, 32, 8, 128, 16, w.num_blocks, w.max_blocks_per_seq, pa.PA_BF16, pa.PA_F32, 0)
    bt = np.ascontiguousarray(w.block_tables)
    lens = np.ascontiguousarray(w.seq_lens)
    assert pa.pa_validate_host(d, bt, lens) == 0
    bad = bt.copy()
    bad[3, 0] = w.num_blocks
    assert pa.pa_validate_host(d, bad, lens) == 8
    bad = bt.copy()
    bad[3, int(w.blocks_per_seq()[3]) - 1] = -1
    assert pa.pa_validate_host(d, bad, lens) == 8
    bad = bt.copy()
    bad[3, int(w.blocks_per_seq()[3])] = 10 ** 6  # beyond n_b: never read, accepted
    assert pa.pa_validate_host(d, bad, lens) == 0
    long = lens.copy()
    long[0] = w.max_blocks_per_seq * 16 + 1
    assert pa.pa_validate_host(d, bt, long) == 8


def test_decode_argument_errors_before_any_launch(lib):
    d = _desc()
    nbytes = pa.pa_workspace_bytes(d)
    P = 1 << 20  # a fake, 16-byte-aligned address; nothing is dereferenced on these paths
    args = [P, P, P, P, P, 0.1, P]
    rc = lib.paged_attn_decode(None, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(d), P, nbytes, None)
    assert rc == 1
    rc = lib.paged_attn_decode(P + 4, *args[1:], pa._lib.ctypes.byref(d), P, nbytes, None)
    assert rc == 6
    rc = lib.paged_attn_decode(*args, pa._lib.ctypes.byref(d), P, nbytes - 1, None)
    assert rc == 5
    rc = lib.paged_attn_decode(*args, pa._lib.ctypes.byref(_desc(head_dim=96)), P, nbytes, None)
    assert rc == 4
    empty = _desc(num_seqs=0)
    assert lib.paged_attn_decode(*args, pa._lib.ctypes.byref(empty), P, nbytes, None) == 0


def test_no_device_is_reported(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _desc()
    P = 1 << 20
    rc = lib.paged_attn_decode(P, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(d), P,
                               pa.pa_workspace_bytes(d), None)
    assert rc == 9
    assert pa.pa_decode_grid(d) == -1


def test_validate_append_host(lib):
    w = workload.make(3, 3, batch=8, max_len=700)
    d = pa.PaDesc(w.num_seqs, 32, 8, 128, 16, w.num_blocks, w.max_blocks_per_seq, pa.PA_BF16, pa.PA_F32, 0)
    bt = np.ascontiguousarray(w.block_tables)
    pos = np.ascontiguousarray(w.seq_lens - 1)  # overwrite each sequence's last token: in its table
    assert pa.pa_validate_append_host(d, bt, pos) == 0
    skip = pos.copy()
    skip[::2] = -1
    assert pa.pa_validate_append_host(d, bt, skip) == 0
    nxt = np.ascontiguousarray(w.seq_lens)  # next slot: fails where it needs a new, unassigned block
    needs_block = (w.seq_lens % 16) == 0
    assert pa.pa_validate_append_host(d, bt, nxt) == (8 if needs_block.any() else 0)
    past = pos.copy()
    past[1] = w.max_blocks_per_seq * 16
    assert pa.pa_validate_append_host(d, bt, past) == 8
    bad = bt.copy()
    bad[2, int(pos[2]) // 16] = w.num_blocks
    assert pa.pa_validate_append_host(d, bad, pos) == 8
    same = bt.copy()
    same[1] = same[0]
    dup = pos.copy()
    dup[1] = dup[0]
    assert pa.pa_validate_append_host(d, same, dup) == 8  # two sequences, one (block, slot)


def test_validate_copy_host(lib):
    d = _desc(num_blocks=10)
    arr = lambda *v: np.asarray(v, np.int32)  # noqa: E731
    assert pa.pa_validate_copy_host(d, arr(1, 2, 3), arr(4, 5, 6), 3) == 0
    assert pa.pa_validate_copy_host(d, arr(1, 1), arr(4, 5), 2) == 0  # one source, two copies
    assert pa.pa_validate_copy_host(d, arr(1, 2), arr(4, 4), 2) == 8  # destination twice
    assert pa.pa_validate_copy_host(d, arr(1, 4), arr(4, 5), 2) == 8  # a destination is a source
    assert pa.pa_validate_copy_host(d, arr(1), arr(10), 1) == 8
    assert pa.pa_validate_copy_host(d, arr(-1), arr(3), 1) == 8
    assert pa.pa_validate_copy_host(d, None, None, 0) == 0
    assert pa.pa_validate_copy_host(d, None, None, 2) == 1
    assert pa.pa_validate_copy_host(d, arr(1), arr(2), -1) == 2


def test_cache_write_argument_errors_before_any_launch(lib):
    d = _desc()
    byref = pa._lib.ctypes.byref
    P = 1 << 20  # fake aligned address; not dereferenced on these paths
    assert lib.paged_kv_append(None, P, P, P, P, P, byref(d), None) == 1
    assert lib.paged_kv_append(P, P, P + 2, P, P, P, byref(d), None) == 6
    assert lib.paged_kv_append(P, P, P, P, P, P, byref(_desc(block_size=8)), None) == 4
    assert lib.paged_kv_append(P, P, P, P, P, P, byref(_desc(num_seqs=0)), None) == 0
    assert lib.paged_kv_copy_blocks(P, P, P, P, -1, byref(d), None) == 2
    assert lib.paged_kv_copy_blocks(P, P, P, P, 0, byref(d), None) == 0
    assert lib.paged_kv_copy_blocks(P, None, P, P, 3, byref(d), None) == 1
    assert lib.paged_kv_copy_blocks(P, P + 8, P, P, 3, byref(d), None) == 6
    assert lib.paged_kv_copy_blocks(P, P, P, P, 3, byref(_desc(dtype=7)), None) == 3
    assert lib.paged_kv_block_scores(P, P, P, P, None, P, byref(d), None) == 1
    assert lib.paged_kv_block_scores(P, P, P, P, P + 2, P, byref(d), None) == 6
    assert lib.paged_kv_block_scores(P + 4, P, P, P, P, P, byref(d), None) == 6
    assert lib.paged_kv_block_scores(P, P, P, P, P, P, byref(_desc(head_dim=64)), None) == 4
    assert lib.paged_kv_block_scores(P, P, P, P, P, P, byref(_desc(num_seqs=0)), None) == 0
    import torch
    if not torch.cuda.is_available():
        assert lib.paged_kv_append(P, P, P, P, P, P, byref(d), None) == 9
        assert lib.paged_kv_copy_blocks(P, P, P, P, 3, byref(d), None) == 9
        assert lib.paged_kv_block_scores(P, P, P, P, P, P, byref(d), None) == 9


def test_binding_refuses_to_run_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(pa._lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pa._lib, "_lib", None)
    with pytest.raises(ImportError):
        pa._lib.load()


def test_validate_prefill_host(lib):
    w = workload.make(3, 3, batch=8, max_len=700)
    d = pa.PaDesc(w.num_seqs, 32, 8, 128, 16, w.num_blocks, w.max_blocks_per_seq, pa.PA_BF16, pa.PA_F32, 0)
    bt = np.ascontiguousarray(w.block_tables)
    lens = np.ascontiguousarray(w.seq_lens)
    n = np.minimum(lens, 37).astype(np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    assert pa.pa_validate_prefill_host(d, bt, lens, qs, int(n.max())) == 0
    assert pa.pa_validate_prefill_host(d, bt, lens, qs, int(n.max()) - 1) == 8  # a chunk beyond max_q_len
    assert pa.pa_validate_prefill_host(d, bt, lens, qs, -1) == 2
    bad = qs.copy()
    bad[0] = 1
    assert pa.pa_validate_prefill_host(d, bt, lens, bad, 10 ** 6) == 8
    bad = qs.copy()
    bad[2] = bad[1] - 1                                                           # negative row count
    assert pa.pa_validate_prefill_host(d, bt, lens, bad, 10 ** 6) == 8
    short = lens.copy()
    short[0] = n[0] - 1                                                           # more rows than tokens
    assert pa.pa_validate_prefill_host(d, bt, short, qs, 10 ** 6) == 8
    bad = bt.copy()
    bad[1, 0] = -5
    assert pa.pa_validate_prefill_host(d, bad, lens, qs, 10 ** 6) == 8


def test_prefill_argument_errors_before_any_launch(lib):
    d = _desc()
    byref = pa._lib.ctypes.byref
    P = 1 << 20  # fake aligned address; not dereferenced on these paths
    args = [P, P, P, P, P, P, 64, 0.1, P]
    assert lib.paged_attn_prefill(None, *args[1:], byref(d), None) == 1
    assert lib.paged_attn_prefill(*args[:5], None, *args[6:], byref(d), None) == 1
    assert lib.paged_attn_prefill(P + 2, *args[1:], byref(d), None) == 6
    assert lib.paged_attn_prefill(*args[:6], -1, *args[7:], byref(d), None) == 2
    assert lib.paged_attn_prefill(*args, byref(_desc(dtype=pa.PA_F32)), None) == 4
    assert lib.paged_attn_prefill(*args, byref(_desc(kernel=pa.PA_KERNEL_VALU)), None) == 4
    assert lib.paged_attn_prefill(*args, byref(_desc(head_dim=64)), None) == 4
    assert lib.paged_attn_prefill(*args, byref(_desc(num_seqs=0)), None) == 0
    assert lib.paged_attn_prefill(*args[:6], 0, *args[7:], byref(d), None) == 0
    import torch
    if not torch.cuda.is_available():
        assert lib.paged_attn_prefill(*args, byref(d), None) == 9


def test_noalloc_argument_errors_before_any_launch(lib):
    """The allocation-free decode checks its arguments like the workspace
    entry point, and without a GPU reports PA_ERR_DEVICE after them."""
    d = _desc()
    P = 1 << 20
    f = lib.paged_attn_decode_noalloc
    assert f(None, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(d), None) == 1
    assert f(P, P, P, None, P, 0.1, P, pa._lib.ctypes.byref(d), None) == 1
    assert f(P + 8, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(d), None) == 6
    assert f(P, P, P, P, P, 0.1, P + 2, pa._lib.ctypes.byref(d), None) == 6
    bad = _desc()
    bad.num_kv_heads = 3
    assert f(P, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(bad), None) == 2
    empty = _desc()
    empty.num_seqs = 0
    assert f(None, None, None, None, None, 0.1, None, pa._lib.ctypes.byref(empty), None) == 0
    import torch
    if not torch.cuda.is_available():
        assert f(P, P, P, P, P, 0.1, P, pa._lib.ctypes.byref(d), None) == 9


def test_shared_prefix_host_checks(lib):
    """pa_validate_shared_host: group bounds and shared counts, and the
    shared table entries equal across members (checked on host copies)."""
    d = _desc(num_seqs=5, max_blocks_per_seq=4, num_blocks=64)
    lens = np.array([40, 64, 10, 0, 33], np.int32)
    bt = np.full((5, 4), -1, np.int32)
    bt[0, :3] = [5, 6, 7]
    bt[1, :4] = [5, 6, 8, 9]
    bt[2, :1] = [5]
    bt[4, :3] = [11, 12, 13]
    ok = pa.pa_validate_shared_host
    gs, gsh = np.array([0, 4, 5], np.int32), np.array([2, 3], np.int32)
    assert ok(d, bt, lens, gs, gsh, 2) == 0
    assert ok(d, bt, lens, None, None, 0) == 0
    assert ok(d, bt, lens, gs, gsh, -1) == 2
    assert ok(d, bt, lens, np.array([0, 4, 6], np.int32), gsh, 2) == 2   # past the batch
    assert ok(d, bt, lens, np.array([0, 4, 3], np.int32), gsh, 2) == 2   # decreasing
    assert ok(d, bt, lens, gs, np.array([2, -1], np.int32), 2) == 2
    assert ok(d, bt, lens, gs, np.array([3, 3], np.int32), 2) == 8       # entry 2 differs
    bt2 = bt.copy()
    bt2[2, 0] = 9                                                         # short member differs
    assert ok(d, bt2, lens, gs, gsh, 2) == 8
    assert pa.pa_shared_workspace_bytes(d) > pa.pa_workspace_bytes(d)
    P = 1 << 20
    f = lib.paged_attn_decode_shared
    nb = pa.pa_shared_workspace_bytes(d)
    assert f(P, P, P, P, P, P, P, -1, 0.1, P, pa._lib.ctypes.byref(d), P, nb, None) == 2
    assert f(P, P, P, P, P, None, P, 1, 0.1, P, pa._lib.ctypes.byref(d), P, nb, None) == 1
    assert f(P, P, P, P, P, P, P, 1, 0.1, P, pa._lib.ctypes.byref(d), P, nb - 1, None) == 5
