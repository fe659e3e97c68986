"""ctypes marshalling for the C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Every method converts numpy arrays to pointers
and calls the C routine of the same name; the arithmetic is all in
``oracle.c``, which cites the passages it follows.  ``Oracle(path)`` can
load another build of the same source (the test suite compiles mutated
copies to check that its pins catch planted mistakes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

#: element-type codes understood by oracle.c
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp, IEEE semantics kept (no fast-math, no contraction)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _stale() -> bool:
    return (not os.path.exists(LIBRARY)) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (always when force, else only if
    the library is missing or older than the source)."""
    if force or _stale():
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """One loaded build of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_to_f64.argtypes = [_P, _I32, _I64, _P]
        lib.oracle_to_f64.restype = None
        lib.oracle_gather.argtypes = [_P, _P, _P, _I32, _I32, _I64, _I32, _I32, _I32,
                                      _I32, _I32, _I32, _P, _P]
        lib.oracle_gather.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [_P, _P, _P, _I64, _I64, _D, _P, _P]
        lib.oracle_attention.restype = None
        lib.oracle_partial.argtypes = [_P, _P, _P, _I64, _I64, _I64, _D, _P, _P, _P]
        lib.oracle_partial.restype = None
        lib.oracle_merge.argtypes = [_D, _D, _P, _D, _D, _P, _I64, _P, _P, _P]
        lib.oracle_merge.restype = None
        lib.oracle_paged_decode.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _I32, _I32, _D, _P, _I32]
        lib.oracle_paged_decode.restype = ctypes.c_int
        lib.oracle_append.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _I32, _I32]
        lib.oracle_append.restype = ctypes.c_int
        lib.oracle_copy_blocks.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32]
        lib.oracle_copy_blocks.restype = ctypes.c_int
        lib.oracle_block_scores.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                            _I32, _P, _P]
        lib.oracle_block_scores.restype = ctypes.c_int
        lib.oracle_paged_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                             _I32, _I32, _I32, _D, _P, _I32]
        lib.oracle_paged_prefill.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def to_f64(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """Exact widening of raw storage (float32, or 16-bit patterns for f16/bf16)."""
        x = _c(x)
        if dtype != "f32":
            x = x.view(np.uint16)
        out = np.empty(x.shape, np.float64)
        self.lib.oracle_to_f64(_ptr(x), DTYPE_CODES[dtype], x.size, _ptr(out))
        return out

    def attention(self, q, K, V, scale: float) -> np.ndarray:
        """Two-pass softmax attention of one query over contiguous fp64 rows."""
        q = _c(q, np.float64)
        K = _c(K, np.float64)
        V = _c(V, np.float64)
        L, D = K.shape
        out = np.empty(D, np.float64)
        s = np.empty(max(L, 1), np.float64)
        self.lib.oracle_attention(_ptr(q), _ptr(K), _ptr(V), L, D, float(scale), _ptr(out), _ptr(s))
        return out

    def partial(self, q, K, V, t0: int, t1: int, scale: float):
        """(m, l, o) of tokens [t0, t1) of contiguous fp64 rows."""
        q = _c(q, np.float64)
        K = _c(K, np.float64)
        V = _c(V, np.float64)
        D = K.shape[1]
        m = np.zeros(1)
        l = np.zeros(1)
        o = np.empty(D, np.float64)
        self.lib.oracle_partial(_ptr(q), _ptr(K), _ptr(V), t0, t1, D, float(scale),
                                _ptr(m), _ptr(l), _ptr(o))
        return float(m[0]), float(l[0]), o

    def merge(self, p1, p2):
        """Merge two (m, l, o) partials by the page's merge equation."""
        m1, l1, o1 = p1
        m2, l2, o2 = p2
        o1 = _c(o1, np.float64)
        o2 = _c(o2, np.float64)
        D = o1.shape[0]
        m = np.zeros(1)
        l = np.zeros(1)
        o = np.empty(D, np.float64)
        self.lib.oracle_merge(float(m1), float(l1), _ptr(o1), float(m2), float(l2), _ptr(o2),
                              D, _ptr(m), _ptr(l), _ptr(o))
        return float(m[0]), float(l[0]), o

    def gather(self, k_pool, v_pool, block_tables, b: int, g: int, L: int, *,
               num_kv_heads: int, head_dim: int, block_size: int, dtype: str):
        """Contiguous fp64 K[L][D], V[L][D] of (sequence b, KV head g)."""
        k_pool = _c(k_pool)
        v_pool = _c(v_pool)
        bt = _c(block_tables, np.int32)
        K = np.empty((max(L, 1), head_dim), np.float64)
        V = np.empty((max(L, 1), head_dim), np.float64)
        rc = self.lib.oracle_gather(_ptr(k_pool), _ptr(v_pool), _ptr(bt), b, g, L, num_kv_heads,
                                    head_dim, block_size, k_pool.shape[0], bt.shape[1],
                                    DTYPE_CODES[dtype], _ptr(K), _ptr(V))
        if rc != 0:
            raise ValueError("oracle_gather: table entry out of range")
        return K[:L], V[:L]

    def paged_decode(self, q, k_pool, v_pool, block_tables, seq_lens, scale, *,
                     num_kv_heads: int, block_size: int, dtype: str,
                     num_threads: int = 0) -> np.ndarray:
        """fp64 out[S][Hq][D] of paged decode attention.

        q: [S][Hq][D]; k_pool: [NB][Hkv][B][D]; v_pool: [NB][Hkv][B/G][D][G]
        with G = 16 when B is a multiple of 16, else G = B
        (raw storage: float32, or 16-bit patterns for f16/bf16);
        block_tables int32 [S][max_blocks_per_seq]; seq_lens int32 [S];
        scale is used as given (pass the float32 value the GPU receives).
        """
        q = _c(q)
        k_pool = _c(k_pool)
        v_pool = _c(v_pool)
        bt = _c(block_tables, np.int32)
        lens = _c(seq_lens, np.int32)
        S, Hq, D = q.shape
        out = np.zeros((S, Hq, D), np.float64)
        rc = self.lib.oracle_paged_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(bt),
                                          _ptr(lens), S, Hq, num_kv_heads, D, block_size,
                                          k_pool.shape[0], bt.shape[1], DTYPE_CODES[dtype],
                                          float(scale), _ptr(out), int(num_threads))
        if rc != 0:
            raise ValueError(f"oracle_paged_decode failed with code {rc}")
        return out

    def append(self, k_new, v_new, k_pool, v_pool, block_tables, positions, inplace=False):
        """Pools after appending k_new / v_new [S][Hkv][D] at logical slot
        positions[b] of every sequence (skipped where < 0).  Pools as in
        paged_decode (raw storage).  Copies unless inplace (then the given
        C-contiguous pools are written and returned)."""
        kp = k_pool if inplace else np.array(k_pool, copy=True, order="C")
        vp = v_pool if inplace else np.array(v_pool, copy=True, order="C")
        assert kp.flags.c_contiguous and vp.flags.c_contiguous
        kn = _c(k_new)
        vn = _c(v_new)
        bt = _c(block_tables, np.int32)
        pos = _c(positions, np.int32)
        NB, Hkv, B, D = kp.shape
        rc = self.lib.oracle_append(_ptr(kn), _ptr(vn), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(pos),
                                    pos.shape[0], Hkv, D, B, NB, bt.shape[1], kp.itemsize)
        if rc != 0:
            raise ValueError("oracle_append: position or table entry out of range")
        return kp, vp

    def copy_blocks(self, k_pool, v_pool, src, dst, inplace=False):
        """Pools after block dst[i] <- block src[i] in both (copies unless
        inplace)."""
        kp = k_pool if inplace else np.array(k_pool, copy=True, order="C")
        vp = v_pool if inplace else np.array(v_pool, copy=True, order="C")
        assert kp.flags.c_contiguous and vp.flags.c_contiguous
        s = _c(src, np.int32)
        d = _c(dst, np.int32)
        NB, Hkv, B, D = kp.shape
        rc = self.lib.oracle_copy_blocks(_ptr(kp), _ptr(vp), _ptr(s), _ptr(d), s.shape[0], Hkv, D,
                                         B, NB, kp.itemsize)
        if rc != 0:
            raise ValueError("oracle_copy_blocks: block id out of range")
        return kp, vp

    def block_scores(self, k_pool, v_pool, block_tables, seq_lens, *, dtype: str):
        """(scores fp64 [S][max_blocks_per_seq] with NaN past the full
        blocks, evict int32 [S]) of block-wise eviction scoring."""
        kp = _c(k_pool)
        vp = _c(v_pool)
        bt = _c(block_tables, np.int32)
        lens = _c(seq_lens, np.int32)
        NB, Hkv, B, D = kp.shape
        S, M = bt.shape
        scores = np.empty((S, M), np.float64)
        evict = np.empty(S, np.int32)
        if dtype != "f32":
            kp, vp = kp.view(np.uint16), vp.view(np.uint16)
        rc = self.lib.oracle_block_scores(_ptr(kp), _ptr(vp), _ptr(bt), _ptr(lens), S, Hkv, D, B, NB,
                                          M, DTYPE_CODES[dtype], _ptr(scores), _ptr(evict))
        if rc != 0:
            raise ValueError("oracle_block_scores: table entry out of range")
        return scores, evict

    def paged_prefill(self, q, k_pool, v_pool, block_tables, seq_lens, q_start, scale, *,
                      num_kv_heads: int, block_size: int, dtype: str,
                      num_threads: int = 0) -> np.ndarray:
        """fp64 out[total_q][Hq][D] of causal paged prefill.

        q: [total_q][Hq][D]; rows q_start[b] .. q_start[b+1]-1 are the
        newest q_start[b+1]-q_start[b] tokens of sequence b (already in the
        pools), row i of them at position seq_lens[b] - n_b + i, attending
        tokens 0 .. that position.  Pools, tables, dtype and scale as for
        paged_decode.
        """
        q = _c(q)
        k_pool = _c(k_pool)
        v_pool = _c(v_pool)
        bt = _c(block_tables, np.int32)
        lens = _c(seq_lens, np.int32)
        qs = _c(q_start, np.int32)
        T, Hq, D = q.shape
        S = lens.shape[0]
        if qs.shape[0] != S + 1 or qs[-1] != T:
            raise ValueError("q_start must hold num_seqs + 1 offsets ending at the row count")
        out = np.zeros((T, Hq, D), np.float64)
        rc = self.lib.oracle_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(bt), _ptr(lens),
                                           _ptr(qs), S, Hq, num_kv_heads, D, block_size,
                                           k_pool.shape[0], bt.shape[1], DTYPE_CODES[dtype],
                                           float(scale), _ptr(out), int(num_threads))
        if rc != 0:
            raise ValueError(f"oracle_paged_prefill failed with code {rc}")
        return out

    def run_workload(self, w, num_threads: int = 0) -> np.ndarray:
        """paged_decode on a workload.Workload-like object."""
        return self.paged_decode(w.q, w.k_pool, w.v_pool, w.block_tables, w.seq_lens,
                                 np.float64(np.float32(w.scale)), num_kv_heads=w.num_kv_heads,
                                 block_size=w.block_size, dtype=w.dtype, num_threads=num_threads)


_lock = threading.Lock()
_default: Oracle | None = None


def load() -> Oracle:
    """The default build (oracle/liboracle.so), (re)built first if missing or
    older than oracle.c."""
    global _default
    with _lock:
        if _default is None:
            if _stale():
                build(force=True)
            _default = Oracle(LIBRARY)
    return _default
