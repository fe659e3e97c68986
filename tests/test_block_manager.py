"""The host block manager (pa_bm_*, CPU only).

Part 1 pins the plain model (oracle/block_manager.py) to the pages
("PagedAttention: The Cache Was Storing Nothing", §2.2 and §2.3, and the
sizing example of §2.1): a sequence grown token by token holds exactly
ceil(L / B) blocks (at most one partly filled), any free block will do
(an allocation of n succeeds exactly when n blocks are free), a block is
copied only when a sequence writes into a block another table shares, and
reference counts always equal the table entries pointing at each block.
Planted mistakes in copies of the model must each fail a pin.

Part 2 runs the library and the model side by side on random operation
sequences (allocation, forks, decode steps, eviction, finished sequences)
and requires identical statuses, ids, tables, positions, copy pairs,
reference counts and free counts.  The id policy (never-used blocks in id
order, then released blocks most recent first) is the library's own
convention: the pages fix none."""
import importlib.util
import json
import os

import numpy as np
import pytest

import paged_kv_cache_196_amd as pa
from oracle import block_manager as bmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _grow(m, tables, lens, steps):
    """`steps` decode steps for every sequence; returns the copy pairs."""
    cows = []
    for _ in range(steps):
        st, pos, c = m.prepare_append(tables, lens)
        assert st == bmm.OK
        cows += c
        lens = [L + 1 if L >= 0 else L for L in lens]
    return lens, cows


# ------------------------------------------------------------ model pins

def pin_growth_holds_ceil_blocks(M):
    for B in (1, 4, 16, 32):
        m = M(4096, B)
        tables = [[-1] * 400 for _ in range(5)]
        lens = [0, 0, 0, 0, 0]
        for step in range(1, 400):
            lens, _ = _grow(m, tables, lens, 1)
            held = [sum(1 for x in row if x >= 0) for row in tables]
            assert held == [-(-L // B) for L in lens], (B, step)
            assert all(h * B - L < B for h, L in zip(held, lens))  # at most one partial block


def pin_sizing_example_200_tokens(M):
    fx = json.load(open(os.path.join(ROOT, "tests", "golden", "sizing_examples.json")))["utilisation_200"]
    m = M(64, fx["block_size"])
    tables = [[-1] * 32]
    _grow(m, tables, [0], fx["length"])
    n = sum(1 for x in tables[0] if x >= 0)
    assert n == fx["blocks"] and n * fx["block_size"] == fx["slots"]
    assert round(100 * fx["length"] / fx["slots"], 1) == fx["utilisation_percent"]
    assert m.num_free() == 64 - n


def pin_any_free_block_will_do(M):
    rng = np.random.default_rng(1)
    m = M(50, 16)
    held = []
    for _ in range(400):
        if held and rng.random() < 0.45:
            k = int(rng.integers(1, len(held) + 1))
            idx = rng.choice(len(held), size=k, replace=False)
            out = [held[i] for i in idx]
            assert m.release(out) == bmm.OK
            held = [h for i, h in enumerate(held) if i not in set(idx)]
        n = int(rng.integers(0, 12))
        free_before = m.num_free()
        st, ids = m.alloc(n)
        if n <= free_before:
            assert st == bmm.OK and len(set(ids)) == n and not set(ids) & set(held)
            assert all(0 <= i < 50 for i in ids)
            held += ids
        else:
            assert st == bmm.ERR_NOMEM and m.num_free() == free_before
        assert m.num_free() == 50 - len(held)


def pin_copy_only_when_a_shared_block_is_written(M):
    B = 16
    for L0 in (5, 16, 31, 32, 40):
        m = M(100, B)
        n = -(-L0 // B)
        st, row = m.alloc(n)
        tables = [row + [-1] * 8, None]
        assert m.share(row) == bmm.OK            # the fork shares every block
        tables[1] = list(tables[0])
        st, pos, cows = m.prepare_append(tables, [L0, L0])
        assert pos == [L0, L0]
        if L0 % B == 0:                          # a new block each: nothing shared is written
            assert cows == []
        else:                                    # first writer copies the shared last block;
            assert len(cows) == 1                # the second then owns the original alone
            src, dst = cows[0]
            assert src == row[L0 // B] and tables[0][L0 // B] == dst and tables[1][L0 // B] == src
        for j in range(L0 // B):                 # full blocks stay shared
            assert tables[0][j] == tables[1][j] and m.refcount(tables[0][j]) == 2


def pin_counts_equal_table_references(M):
    rng = np.random.default_rng(2)
    B = 8
    m = M(400, B)
    tables, lens = [], []
    for step in range(300):
        op = rng.random()
        if op < 0.2 or not tables:              # new sequence with a prompt
            L = int(rng.integers(1, 40))
            st, ids = m.alloc(-(-L // B))
            if st != bmm.OK:
                continue
            tables.append(list(ids) + [-1] * 40)
            lens.append(L)
        elif op < 0.3:                          # fork a sequence
            k = int(rng.integers(len(tables)))
            live = [x for x in tables[k] if x >= 0]
            assert m.share(live) == bmm.OK
            tables.append(list(tables[k]))
            lens.append(lens[k])
        elif op < 0.4:                          # a sequence finishes
            k = int(rng.integers(len(tables)))
            assert m.release([x for x in tables[k] if x >= 0]) == bmm.OK
            del tables[k], lens[k]
        else:                                   # one decode step for everyone
            st, pos, cows = m.prepare_append(tables, lens)
            if st == bmm.OK:
                lens = [L + 1 for L in lens]
        refs = {}
        for row in tables:
            for x in row:
                if x >= 0:
                    refs[x] = refs.get(x, 0) + 1
        assert all(m.refcount(x) == c for x, c in refs.items()), step
        assert m.num_free() == 400 - len(refs), step


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__[4:])
def test_model_pin(pin):
    pin(bmm.BlockManagerModel)


MUTANTS = [
    ("copy_unshared_blocks", "if self.refs[old] > 1:", "if self.refs[old] >= 1:"),
    ("no_block_at_boundary", "if L % B == 0:  # the new token opens a block", "if L % B == 1:"),
    ("released_never_reused", "        if self.released:\n", "        if False:\n"),
    ("release_keeps_block", "                del self.refs[block]\n                self.released.append(block)\n",
     "                pass\n"),
    ("share_not_counted", "            self.refs[block] += 1\n", "            pass\n"),
    ("free_count_forgets_released", "return (self.num_blocks - self.next_unused) + len(self.released)",
     "return self.num_blocks - self.next_unused"),
    ("copy_keeps_source_reference", "                    self.release([old])\n", ""),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_in_model_is_caught(tmp_path, name, old, new):
    src = open(bmm.__file__).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"bm_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"bm_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in PINS:
        try:
            pin(mod.BlockManagerModel)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"


# ------------------------------------------------------ library vs model

def _same_state(lib, model, nb):
    assert lib.num_free() == model.num_free()
    assert [lib.refcount(i) for i in range(nb)] == [model.refcount(i) for i in range(nb)]


@pytest.mark.parametrize("seed,B", [(0, 16), (1, 32), (2, 1), (3, 16)])
def test_library_matches_model(seed, B):
    rng = np.random.default_rng(seed)
    NB, M = 300, 48
    lib, model = pa.BlockManager(NB, B), bmm.BlockManagerModel(NB, B)
    tables = np.zeros((0, M), np.int32)
    lens = []
    for step in range(400):
        op = rng.random()
        if op < 0.15 or len(lens) == 0:
            L = int(rng.integers(1, 5 * B))
            n = -(-L // B)
            s1, ids1 = lib.alloc(n)
            s2, ids2 = model.alloc(n)
            assert s1 == s2 and list(ids1) == ids2, step
            if s1 == 0:
                row = np.full((1, M), -1, np.int32)
                row[0, :n] = ids1
                tables = np.concatenate([tables, row])
                lens.append(L)
        elif op < 0.25:
            k = int(rng.integers(len(lens)))
            live = tables[k][tables[k] >= 0]
            assert lib.share(live) == model.share(list(live)) == 0
            tables = np.concatenate([tables, tables[k: k + 1]])
            lens.append(lens[k])
        elif op < 0.33:
            k = int(rng.integers(len(lens)))
            live = tables[k][tables[k] >= 0]
            assert lib.release(live) == model.release(list(live)) == 0
            tables = np.delete(tables, k, axis=0)
            del lens[k]
        elif op < 0.38:  # evict one full block of a sequence (release it, compact the row)
            k = int(rng.integers(len(lens)))
            full = lens[k] // B
            if full >= 2:
                j = int(rng.integers(full))
                blk = int(tables[k][j])
                assert lib.release([blk]) == model.release([blk]) == 0
                row = list(tables[k][tables[k] >= 0])
                del row[j]
                tables[k] = -1
                tables[k][: len(row)] = row
                lens[k] -= B
        else:
            mt = [list(r) for r in tables]
            skip = [L if rng.random() > 0.1 else -1 for L in lens]
            t = np.ascontiguousarray(tables)
            s1, p1, cs, cd = lib.prepare_append(t, skip)
            s2, p2, cows = model.prepare_append(mt, skip)
            assert s1 == s2, step
            assert list(p1) == p2 and list(zip(cs.tolist(), cd.tolist())) == cows, step
            assert t.tolist() == mt, step
            tables = t
            if s1 == 0:
                lens = [L + 1 if s >= 0 else L for L, s in zip(lens, skip)]
            else:  # out of blocks: stop growing
                break
        _same_state(lib, model, NB)
    lib.close()


def test_library_errors():
    lib = pa.BlockManager(8, 16)
    st, ids = lib.alloc(6)
    assert st == 0 and list(ids) == list(range(6))
    assert lib.alloc(3)[0] == 10 and lib.num_free() == 2      # all or nothing
    assert lib.alloc(-1)[0] == 2
    assert lib.release([7]) == 8                               # never allocated
    assert lib.release([2, 2]) == 8 and lib.refcount(2) == 0   # second drop of a free block
    assert lib.share([2]) == 8
    assert lib.share([9]) == 8 and lib.refcount(9) == -1
    t = np.full((1, 2), -1, np.int32)
    assert lib.prepare_append(t, [40])[0] == 8                 # beyond the table row
    t[0, 0] = 5
    assert lib.prepare_append(t, [3])[0] == 0                  # owned: written in place
    st, pos, cs, cd = lib.prepare_append(np.full((1, 4), -1, np.int32), [4])
    assert st == 8                                             # entry is not a live block
    L = pa.load()
    assert L.pa_bm_create(0, 16) is None and L.pa_bm_create(4, 0) is None
    assert L.pa_bm_num_free(None) == -1 and L.pa_bm_refcount(None, 0) == -1
    lib.close()


# ------------------------------------------------------ concurrency

def _canonical(tables):
    """Relabel block ids by order of first appearance (row-major), so that
    two runs that differ only in which physical ids they drew compare equal."""
    names = {}
    return [[names.setdefault(x, len(names)) if x >= 0 else -1 for x in row] for row in tables]


def _drive(m, seed, B, steps=250, width=24):
    """One client's script of operations on its own sequences: new
    sequences, forks (shared rows), finished sequences, decode steps over
    all of its rows.  The script depends on statuses only, never on which
    ids the manager hands out, so run against the library from a thread
    (while other clients work) and against the model alone it must build
    tables of the same sharing structure.  Returns (tables, lens, copies)."""
    rng = np.random.default_rng(seed)
    tables = np.zeros((0, width), np.int32)
    lens, copies = [], 0
    lib = not isinstance(m, bmm.BlockManagerModel)
    for _ in range(steps):
        op = rng.random()
        if op < 0.2 or not lens:
            L = int(rng.integers(1, 4 * B))
            n = -(-L // B)
            st, ids = m.alloc(n)
            assert st == bmm.OK
            row = np.full((1, width), -1, np.int32)
            row[0, :n] = ids
            tables = np.concatenate([tables, row])
            lens.append(L)
        elif op < 0.3:
            k = int(rng.integers(len(lens)))
            assert m.share(list(tables[k][tables[k] >= 0])) == bmm.OK
            tables = np.concatenate([tables, tables[k: k + 1]])
            lens.append(lens[k])
        elif op < 0.4 and len(lens) > 1:
            k = int(rng.integers(len(lens)))
            assert m.release(list(tables[k][tables[k] >= 0])) == bmm.OK
            tables = np.delete(tables, k, axis=0)
            del lens[k]
        else:
            skip = [L if L < width * B - 1 and rng.random() > 0.1 else -1 for L in lens]
            if lib:
                tables = np.ascontiguousarray(tables)
                st, _, cs, _ = m.prepare_append(tables, skip)
                n_cow = len(cs)
            else:
                mt = [list(r) for r in tables]
                st, _, cows = m.prepare_append(mt, skip)
                tables = np.array(mt, np.int32).reshape(-1, width)
                n_cow = len(cows)
            assert st == bmm.OK
            copies += n_cow
            lens = [L + 1 if s >= 0 else L for L, s in zip(lens, skip)]
    return tables, lens, copies


def _run_threads(fn, n):
    import threading
    errors, out = [], [None] * n

    def body(i):
        try:
            out[i] = fn(i)
        except BaseException as e:  # noqa: BLE001 - reported by the main thread
            errors.append(e)

    th = [threading.Thread(target=body, args=(i,)) for i in range(n)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    if errors:
        raise errors[0]
    return out


@pytest.mark.parametrize("B", [16, 1])
def test_concurrent_clients_match_model(B):
    """Eight threads drive one library manager at once (ctypes releases
    the interpreter lock around each call).  Each client's tables must have
    the sharing structure the model builds for the same script alone, no id
    may appear in two clients' tables, and every reference count and the
    free count must equal what the tables hold."""
    T, NB = 8, 12000
    lib = pa.BlockManager(NB, B)
    res = _run_threads(lambda i: _drive(lib, 100 + i, B), T)
    owner = {}
    refs = np.zeros(NB, np.int64)
    for i, (tables, lens, copies) in enumerate(res):
        mt, ml, mc = _drive(bmm.BlockManagerModel(NB, B), 100 + i, B)
        assert _canonical(tables.tolist()) == _canonical(mt.tolist()) and lens == ml and copies == mc, i
        for x in tables[tables >= 0].tolist():
            assert owner.setdefault(x, i) == i, (x, i)   # one client's block only
            refs[x] += 1
    assert [lib.refcount(x) for x in range(NB)] == refs.tolist()
    assert lib.num_free() == NB - len(owner)
    for tables, _, _ in res:
        for row in tables:
            assert lib.release(row[row >= 0]) == 0
    assert lib.num_free() == NB and all(lib.refcount(x) == 0 for x in range(NB))
    lib.close()


def test_concurrent_exhaustion_all_or_nothing():
    """Eight threads contend for a pool far too small for all of them:
    every allocation either hands out all it asked for or fails with
    PA_ERR_NOMEM and nothing, a failed decode step leaves the client's
    table untouched, and after everything is released the pool is whole."""
    T, NB, B, W = 8, 96, 4, 12

    def client(i):
        rng = np.random.default_rng(7 + i)
        rows, lens, fails = [], [], 0
        for _ in range(600):
            op = rng.random()
            if op < 0.35:
                n = int(rng.integers(1, 9))
                st, ids = lib.alloc(n)
                assert st in (0, 10)
                if st == 0:
                    assert len(ids) == n and len(set(ids.tolist())) == n
                    row = np.full(W, -1, np.int32)
                    row[:n] = ids
                    rows.append(row)
                    lens.append(n * B)
                else:
                    assert len(ids) == 0
                    fails += 1
            elif op < 0.6 and rows:
                k = int(rng.integers(len(rows)))
                assert lib.release(rows[k][rows[k] >= 0]) == 0
                del rows[k], lens[k]
            elif rows:
                t = np.ascontiguousarray(np.stack(rows))
                before = t.copy()
                skip = [L if L < W * B else -1 for L in lens]
                st, pos, cs, _ = lib.prepare_append(t, skip)
                assert st in (0, 10) and len(cs) == 0
                if st == 0:
                    rows = list(t)
                    lens = [L + 1 if s >= 0 else L for L, s in zip(lens, skip)]
                else:
                    assert np.array_equal(t, before)
                    fails += 1
        return rows, fails

    lib = pa.BlockManager(NB, B)
    res = _run_threads(client, T)
    held = [x for rows, _ in res for r in rows for x in r[r >= 0].tolist()]
    assert len(held) == len(set(held)) and lib.num_free() == NB - len(held)
    assert sum(f for _, f in res) > 0          # the pool really ran dry
    for rows, _ in res:
        for r in rows:
            assert lib.release(r[r >= 0]) == 0
    assert lib.num_free() == NB
    st, ids = lib.alloc(NB)
    assert st == 0 and sorted(ids.tolist()) == list(range(NB))
    lib.close()


def _sanitizer_build(tmp_path, name, flags):
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / name)
    cmd = [gxx, "-O1", "-g", "-std=c++17", "-pthread", *flags,
           "-I", os.path.join(ROOT, "paged_kv_cache_196_amd", "csrc"),
           os.path.join(ROOT, "tests", "bm_stress.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("name,flags,env", [
    ("tsan", ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"}),
    ("asan", ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"],
     {"ASAN_OPTIONS": "detect_leaks=1"}),
    ("plain", ["-O2"], {}),
])
def test_block_manager_stress_under_sanitizers(tmp_path, name, flags, env):
    """The block manager header compiled on the host alone (no device
    code) into tests/bm_stress.cpp: eight threads of random allocations,
    shares of their own and of other threads' published blocks, and
    releases, singly and in batches, with reference counts and free counts
    checked after every round.  ThreadSanitizer must report no data race,
    AddressSanitizer and UBSan no invalid access, leak or undefined
    behaviour.  The 48-block pool keeps the free list's head under constant
    exchange: a head without its tag (ABA) hands a block out twice or links
    the list into a cycle there, which fails the counts or the time limit."""
    import subprocess
    exe = _sanitizer_build(tmp_path, name, flags)
    runs = [["1024", "8", "4", "20000"], ["48", "8", "4", "20000"]]
    if name == "plain":
        runs.append(["48", "8", "10", "100000"])
    for argv in runs:
        r = subprocess.run([exe, *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 0 and r.stdout.strip() == "ok", (argv, r.stdout + r.stderr)
        assert "WARNING" not in r.stderr and "ERROR" not in r.stderr, r.stderr
