"""ctypes binding of libpagedattn.so: the C ABI of include/pagedattn.h,
same names, argument marshalling only.  Every step of the computation runs
in the library's gfx950 kernels; there is no fallback."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedattn.so")

PA_OK = 0
STATUS = {
    0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE", 4: "PA_ERR_UNSUPPORTED",
    5: "PA_ERR_WORKSPACE", 6: "PA_ERR_ALIGN", 7: "PA_ERR_LAUNCH", 8: "PA_ERR_TABLE",
    9: "PA_ERR_DEVICE", 10: "PA_ERR_NOMEM", 11: "PA_ERR_SCRATCH",
}
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_KERNEL_AUTO, PA_KERNEL_VALU, PA_KERNEL_MFMA = 0, 1, 2

#: every function include/pagedattn.h declares
EXPORTS = (
    "pa_status_str", "pa_dtype_size", "pa_blocks_for_len", "pa_pool_bytes", "pa_k_elem_offset",
    "pa_v_elem_offset", "pa_workspace_bytes", "pa_validate_host", "pa_check_desc",
    "paged_attn_decode", "pa_decode_grid", "paged_kv_append", "pa_validate_append_host",
    "paged_kv_copy_blocks", "pa_validate_copy_host", "paged_kv_block_scores", "pa_bm_create",
    "pa_bm_destroy", "pa_bm_num_free", "pa_bm_refcount", "pa_bm_alloc", "pa_bm_release",
    "pa_bm_share", "pa_bm_prepare_append", "paged_attn_prefill", "pa_validate_prefill_host",
    "paged_attn_decode_noalloc", "paged_attn_decode_shared", "pa_shared_workspace_bytes",
    "pa_decode_shared_grid", "pa_validate_shared_host",
)


class PaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "dtype", "out_dtype", "kernel", "cached_prefix_blocks")]


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_DP = ctypes.POINTER(PaDesc)


def load() -> ctypes.CDLL:
    """Load the built library; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_196_amd.build`"
                    " (the gfx950 library is required; there is no fallback)")
            lib = ctypes.CDLL(LIB_PATH)
            lib.pa_status_str.argtypes = [ctypes.c_int32]
            lib.pa_status_str.restype = ctypes.c_char_p
            lib.pa_dtype_size.argtypes = [ctypes.c_int32]
            lib.pa_dtype_size.restype = ctypes.c_size_t
            lib.pa_blocks_for_len.argtypes = [ctypes.c_int64, ctypes.c_int32]
            lib.pa_blocks_for_len.restype = ctypes.c_int64
            lib.pa_pool_bytes.argtypes = [_DP]
            lib.pa_pool_bytes.restype = ctypes.c_size_t
            for n in ("pa_k_elem_offset", "pa_v_elem_offset"):
                f = getattr(lib, n)
                f.argtypes = [_DP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                f.restype = ctypes.c_int64
            lib.pa_workspace_bytes.argtypes = [_DP]
            lib.pa_workspace_bytes.restype = ctypes.c_size_t
            lib.pa_validate_host.argtypes = [_DP, _P, _P]
            lib.pa_validate_host.restype = ctypes.c_int32
            lib.pa_check_desc.argtypes = [_DP]
            lib.pa_check_desc.restype = ctypes.c_int32
            lib.paged_attn_decode.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _DP, _P,
                                              ctypes.c_size_t, _P]
            lib.paged_attn_decode.restype = ctypes.c_int32
            lib.paged_attn_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _DP, _P]
            lib.paged_attn_decode_noalloc.restype = ctypes.c_int32
            lib.paged_attn_decode_shared.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                     ctypes.c_float, _P, _DP, _P, ctypes.c_size_t,
                                                     _P]
            lib.paged_attn_decode_shared.restype = ctypes.c_int32
            lib.pa_shared_workspace_bytes.argtypes = [_DP]
            lib.pa_shared_workspace_bytes.restype = ctypes.c_size_t
            lib.pa_decode_shared_grid.argtypes = [_DP, ctypes.c_int32]
            lib.pa_decode_shared_grid.restype = ctypes.c_int32
            lib.pa_validate_shared_host.argtypes = [_DP, _P, _P, _P, _P, ctypes.c_int32]
            lib.pa_validate_shared_host.restype = ctypes.c_int32
            lib.pa_decode_grid.argtypes = [_DP]
            lib.pa_decode_grid.restype = ctypes.c_int32
            lib.paged_kv_append.argtypes = [_P, _P, _P, _P, _P, _P, _DP, _P]
            lib.paged_kv_append.restype = ctypes.c_int32
            lib.pa_validate_append_host.argtypes = [_DP, _P, _P]
            lib.pa_validate_append_host.restype = ctypes.c_int32
            lib.paged_kv_copy_blocks.argtypes = [_P, _P, _P, _P, ctypes.c_int32, _DP, _P]
            lib.paged_kv_copy_blocks.restype = ctypes.c_int32
            lib.pa_validate_copy_host.argtypes = [_DP, _P, _P, ctypes.c_int32]
            lib.pa_validate_copy_host.restype = ctypes.c_int32
            lib.paged_kv_block_scores.argtypes = [_P, _P, _P, _P, _P, _P, _DP, _P]
            lib.paged_kv_block_scores.restype = ctypes.c_int32
            lib.paged_attn_prefill.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                                               _P, _DP, _P]
            lib.paged_attn_prefill.restype = ctypes.c_int32
            lib.pa_validate_prefill_host.argtypes = [_DP, _P, _P, _P, ctypes.c_int32]
            lib.pa_validate_prefill_host.restype = ctypes.c_int32
            lib.pa_bm_create.argtypes = [ctypes.c_int32, ctypes.c_int32]
            lib.pa_bm_create.restype = _P
            lib.pa_bm_destroy.argtypes = [_P]
            lib.pa_bm_destroy.restype = None
            lib.pa_bm_num_free.argtypes = [_P]
            lib.pa_bm_num_free.restype = ctypes.c_int32
            lib.pa_bm_refcount.argtypes = [_P, ctypes.c_int32]
            lib.pa_bm_refcount.restype = ctypes.c_int32
            for n in ("pa_bm_alloc",):
                getattr(lib, n).argtypes = [_P, ctypes.c_int32, _P]
                getattr(lib, n).restype = ctypes.c_int32
            for n in ("pa_bm_release", "pa_bm_share"):
                getattr(lib, n).argtypes = [_P, _P, ctypes.c_int32]
                getattr(lib, n).restype = ctypes.c_int32
            lib.pa_bm_prepare_append.argtypes = [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                                                 _P, _P]
            lib.pa_bm_prepare_append.restype = ctypes.c_int32
            _lib = lib
    return _lib


def status_str(status: int) -> str:
    try:
        return load().pa_status_str(int(status)).decode()
    except ImportError:
        return STATUS.get(int(status), f"status {status}")


def _ptr(x):
    """Device/host address of a torch tensor, or an int / None as given."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(rc: int, where: str) -> int:
    if rc != PA_OK:
        raise PagedAttnError(rc, where)
    return rc


def pa_dtype_size(dtype: int) -> int:
    return int(load().pa_dtype_size(dtype))


def pa_blocks_for_len(length: int, block_size: int) -> int:
    return int(load().pa_blocks_for_len(length, block_size))


def pa_pool_bytes(desc: PaDesc) -> int:
    return int(load().pa_pool_bytes(ctypes.byref(desc)))


def pa_k_elem_offset(desc: PaDesc, block: int, kv_head: int, slot: int, dim: int) -> int:
    return int(load().pa_k_elem_offset(ctypes.byref(desc), block, kv_head, slot, dim))


def pa_v_elem_offset(desc: PaDesc, block: int, kv_head: int, slot: int, dim: int) -> int:
    return int(load().pa_v_elem_offset(ctypes.byref(desc), block, kv_head, slot, dim))


def pa_workspace_bytes(desc: PaDesc) -> int:
    return int(load().pa_workspace_bytes(ctypes.byref(desc)))


def pa_check_desc(desc: PaDesc) -> int:
    return int(load().pa_check_desc(ctypes.byref(desc)))


def pa_validate_host(desc: PaDesc, block_tables_host, seq_lens_host) -> int:
    """block_tables_host / seq_lens_host: contiguous int32 numpy arrays."""
    return int(load().pa_validate_host(ctypes.byref(desc), block_tables_host.ctypes.data,
                                       seq_lens_host.ctypes.data))


def pa_validate_prefill_host(desc: PaDesc, block_tables_host, seq_lens_host, q_start_host,
                             max_q_len: int) -> int:
    """Host copies as contiguous int32 numpy arrays; q_start_host [S + 1]."""
    return int(load().pa_validate_prefill_host(ctypes.byref(desc), block_tables_host.ctypes.data,
                                               seq_lens_host.ctypes.data, q_start_host.ctypes.data,
                                               int(max_q_len)))


def pa_decode_grid(desc: PaDesc) -> int:
    return int(load().pa_decode_grid(ctypes.byref(desc)))


def paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, scale: float, out,
                      desc: PaDesc, workspace, workspace_bytes: int, stream=None) -> int:
    rc = load().paged_attn_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                  _ptr(seq_lens), float(scale), _ptr(out), ctypes.byref(desc),
                                  _ptr(workspace), int(workspace_bytes), _ptr(stream))
    return _check(rc, "paged_attn_decode")


def paged_attn_decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, scale: float, out,
                              desc: PaDesc, stream=None) -> int:
    rc = load().paged_attn_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                          _ptr(seq_lens), float(scale), _ptr(out),
                                          ctypes.byref(desc), _ptr(stream))
    return _check(rc, "paged_attn_decode_noalloc")


def paged_attn_decode_shared(q, k_pool, v_pool, block_tables, seq_lens, group_start, group_shared,
                             num_groups: int, scale: float, out, desc: PaDesc, workspace,
                             workspace_bytes: int, stream=None) -> int:
    rc = load().paged_attn_decode_shared(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                         _ptr(seq_lens), _ptr(group_start), _ptr(group_shared),
                                         int(num_groups), float(scale), _ptr(out),
                                         ctypes.byref(desc), _ptr(workspace),
                                         int(workspace_bytes), _ptr(stream))
    return _check(rc, "paged_attn_decode_shared")


def pa_shared_workspace_bytes(desc: PaDesc) -> int:
    return int(load().pa_shared_workspace_bytes(ctypes.byref(desc)))


def pa_decode_shared_grid(desc: PaDesc, num_groups: int) -> int:
    return int(load().pa_decode_shared_grid(ctypes.byref(desc), int(num_groups)))


def pa_validate_shared_host(desc: PaDesc, block_tables_host, seq_lens_host, group_start_host,
                            group_shared_host, num_groups: int) -> int:
    """Host copies as contiguous int32 numpy arrays (group arrays may be None
    when num_groups is 0)."""
    return int(load().pa_validate_shared_host(
        ctypes.byref(desc), block_tables_host.ctypes.data, seq_lens_host.ctypes.data,
        None if group_start_host is None else group_start_host.ctypes.data,
        None if group_shared_host is None else group_shared_host.ctypes.data, int(num_groups)))


def paged_attn_prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, max_q_len: int,
                       scale: float, out, desc: PaDesc, stream=None) -> int:
    rc = load().paged_attn_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                   _ptr(seq_lens), _ptr(q_start), int(max_q_len), float(scale),
                                   _ptr(out), ctypes.byref(desc), _ptr(stream))
    return _check(rc, "paged_attn_prefill")


def paged_kv_append(k_new, v_new, k_pool, v_pool, block_tables, positions, desc: PaDesc,
                    stream=None) -> int:
    rc = load().paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_tables), _ptr(positions), ctypes.byref(desc),
                                _ptr(stream))
    return _check(rc, "paged_kv_append")


def pa_validate_append_host(desc: PaDesc, block_tables_host, positions_host) -> int:
    """block_tables_host / positions_host: contiguous int32 numpy arrays."""
    return int(load().pa_validate_append_host(ctypes.byref(desc), block_tables_host.ctypes.data,
                                              positions_host.ctypes.data))


def paged_kv_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, num_pairs: int, desc: PaDesc,
                         stream=None) -> int:
    rc = load().paged_kv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(src_blocks),
                                     _ptr(dst_blocks), int(num_pairs), ctypes.byref(desc),
                                     _ptr(stream))
    return _check(rc, "paged_kv_copy_blocks")


def pa_validate_copy_host(desc: PaDesc, src_host, dst_host, num_pairs: int) -> int:
    """src_host / dst_host: contiguous int32 numpy arrays (or None when num_pairs is 0)."""
    return int(load().pa_validate_copy_host(
        ctypes.byref(desc), None if src_host is None else src_host.ctypes.data,
        None if dst_host is None else dst_host.ctypes.data, int(num_pairs)))


def paged_kv_block_scores(k_pool, v_pool, block_tables, seq_lens, block_scores, evict,
                          desc: PaDesc, stream=None) -> int:
    rc = load().paged_kv_block_scores(_ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                      _ptr(seq_lens), _ptr(block_scores), _ptr(evict),
                                      ctypes.byref(desc), _ptr(stream))
    return _check(rc, "paged_kv_block_scores")


class BlockManager:
    """The library's host block manager (pa_bm_*): marshalling only.  Arrays
    are contiguous int32 numpy arrays; methods return the pa_status code."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load()
        self.h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self.h:
            raise ValueError("pa_bm_create failed")
        self.block_size = int(block_size)

    def close(self):
        if self.h:
            self._lib.pa_bm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter teardown
            pass

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self.h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self.h, int(block)))

    def alloc(self, n: int):
        import numpy as np
        ids = np.zeros(max(n, 1), np.int32)
        rc = int(self._lib.pa_bm_alloc(self.h, int(n), ids.ctypes.data))
        return rc, (ids[:n] if rc == PA_OK else ids[:0])

    def release(self, ids) -> int:
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        return int(self._lib.pa_bm_release(self.h, a.ctypes.data if a.size else None, a.size))

    def share(self, ids) -> int:
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        return int(self._lib.pa_bm_share(self.h, a.ctypes.data if a.size else None, a.size))

    def prepare_append(self, block_tables, seq_lens):
        """block_tables: int32 [S][M] numpy array, updated in place.
        Returns (status, positions, cow_src, cow_dst)."""
        import numpy as np
        assert block_tables.dtype == np.int32 and block_tables.flags.c_contiguous
        lens = np.ascontiguousarray(seq_lens, np.int32)
        S, M = block_tables.shape
        pos = np.full(max(S, 1), -1, np.int32)
        src = np.zeros(max(S, 1), np.int32)
        dst = np.zeros(max(S, 1), np.int32)
        n = ctypes.c_int32(0)
        rc = int(self._lib.pa_bm_prepare_append(self.h, block_tables.ctypes.data, M, lens.ctypes.data,
                                                S, pos.ctypes.data, src.ctypes.data, dst.ctypes.data,
                                                ctypes.byref(n)))
        return rc, pos[:S], src[: n.value], dst[: n.value]
