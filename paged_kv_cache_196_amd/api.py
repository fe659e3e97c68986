"""torch conveniences over the C ABI: a descriptor built from tensor
shapes, output / workspace allocation through torch's caching allocator
and the current HIP stream.  Marshalling only; the computation is the
library's."""
from __future__ import annotations

import os

import torch

from . import _lib

_TORCH_DTYPES = {torch.float32: _lib.PA_F32, torch.float16: _lib.PA_F16,
                 torch.bfloat16: _lib.PA_BF16}


def _check_out(out: torch.Tensor, q: torch.Tensor, out_dtype: torch.dtype | None) -> None:
    """A caller's `out` must be what the library writes: q's shape, the
    output type, contiguous, on q's device."""
    want = q.dtype if out_dtype is None else out_dtype
    if out.dtype != want:
        raise TypeError(f"out must be {want} (got {out.dtype})")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)} (got {tuple(out.shape)})")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if out.device != q.device:
        raise ValueError("out must be on q's device")


def ensure_built() -> str:
    """Build libpagedattn.so if it is not there yet; return its path."""
    if not os.path.exists(_lib.LIB_PATH):
        from . import build
        build.build()
    return _lib.LIB_PATH


def pa_dtype_of(t: torch.dtype) -> int:
    try:
        return _TORCH_DTYPES[t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t}") from None


def make_desc(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor, *,
              out_dtype: torch.dtype | None = torch.float32, kernel: int = _lib.PA_KERNEL_AUTO,
              cached_prefix_blocks: int = 0) -> _lib.PaDesc:
    """q [S][Hq][D]; k_pool [NB][Hkv][B][D]; block_tables int32 [S][max_blocks].
    cached_prefix_blocks: leading logical blocks of every sequence that may
    be shared with other sequences (a cache hint; results do not change)."""
    S, Hq, D = q.shape
    NB, Hkv, B, Dk = k_pool.shape
    if Dk != D:
        raise ValueError("q and k_pool head_dim differ")
    dt = pa_dtype_of(q.dtype)
    odt = dt if out_dtype is None else pa_dtype_of(out_dtype)
    return _lib.PaDesc(S, Hq, Hkv, D, B, NB, block_tables.shape[1], dt, odt, kernel,
                       cached_prefix_blocks)


def new_workspace(desc: _lib.PaDesc, device) -> torch.Tensor:
    """A zero-filled workspace for `desc` (the library keeps it zeroed
    between calls, so it can be reused without clearing)."""
    nbytes = _lib.pa_workspace_bytes(desc)
    if nbytes == 0:
        raise _lib.PagedAttnError(_lib.pa_check_desc(desc), "new_workspace")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale: float, *,
           out: torch.Tensor | None = None, out_dtype: torch.dtype | None = torch.float32,
           kernel: int = _lib.PA_KERNEL_AUTO, workspace: torch.Tensor | None = None,
           stream: torch.cuda.Stream | None = None, cached_prefix_blocks: int = 0
           ) -> torch.Tensor:
    """Paged decode attention on device tensors; returns out [S][Hq][D].

    workspace: reuse one from new_workspace() to avoid an allocation per
    call (it must have been zero-filled once; the library keeps it so).
    cached_prefix_blocks: cache hint for a prefix shared across the batch
    (pa_desc.cached_prefix_blocks).

    k_pool [NB][Hkv][B][D] (token-major), v_pool [NB][Hkv][B/16][D][16]
    (transposed within 16-token groups), block_tables / seq_lens int32,
    all on one GPU."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    NB, Hkv, B, D = k_pool.shape
    if B % 16 != 0 or tuple(v_pool.shape) != (NB, Hkv, B // 16, D, 16):
        raise ValueError("v_pool must be [num_blocks][num_kv_heads][block_size/16][head_dim][16]")
    desc = make_desc(q, k_pool, block_tables, out_dtype=out_dtype, kernel=kernel,
                     cached_prefix_blocks=cached_prefix_blocks)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    else:
        _check_out(out, q, out_dtype)
    if workspace is None:
        workspace = new_workspace(desc, q.device)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    _lib.paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out, desc,
                           workspace, workspace.numel() * workspace.element_size(),
                           st.cuda_stream)
    return out


def new_shared_workspace(desc: _lib.PaDesc, device) -> torch.Tensor:
    """A zero-filled workspace for decode_shared (kept zeroed by the library)."""
    nbytes = _lib.pa_shared_workspace_bytes(desc)
    if nbytes == 0:
        raise _lib.PagedAttnError(_lib.pa_check_desc(desc), "new_shared_workspace")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def decode_shared(q, k_pool, v_pool, block_tables, seq_lens, group_start, group_shared,
                  scale: float, *, out: torch.Tensor | None = None,
                  out_dtype: torch.dtype | None = torch.float32, kernel: int = _lib.PA_KERNEL_AUTO,
                  workspace: torch.Tensor | None = None,
                  stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Paged decode attention with prefix groups (paged_attn_decode_shared):
    group i is the sequences group_start[i] .. group_start[i+1]-1, whose
    first group_shared[i] table entries are the same physical blocks; those
    blocks are read once per group.  group_start int32 [num_groups + 1],
    group_shared int32 [num_groups], device tensors.  Other arguments as for
    decode(); the workspace comes from new_shared_workspace()."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("group_start", group_start), ("group_shared", group_shared)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("group_start", group_start), ("group_shared", group_shared)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    ng = group_shared.shape[0]
    if group_start.shape != (ng + 1,):
        raise ValueError("group_start must be [num_groups + 1]")
    NB, Hkv, B, D = k_pool.shape
    if B % 16 != 0 or tuple(v_pool.shape) != (NB, Hkv, B // 16, D, 16):
        raise ValueError("v_pool must be [num_blocks][num_kv_heads][block_size/16][head_dim][16]")
    _check_table(block_tables, q.shape[0])
    desc = make_desc(q, k_pool, block_tables, out_dtype=out_dtype, kernel=kernel)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    else:
        _check_out(out, q, out_dtype)
    if workspace is None:
        workspace = new_shared_workspace(desc, q.device)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    _lib.paged_attn_decode_shared(q, k_pool, v_pool, block_tables, seq_lens, group_start,
                                  group_shared, ng, scale, out, desc, workspace,
                                  workspace.numel() * workspace.element_size(), st.cuda_stream)
    return out


def prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, scale: float, *,
            max_q_len: int | None = None, out: torch.Tensor | None = None,
            out_dtype: torch.dtype | None = torch.float32, kernel: int = _lib.PA_KERNEL_AUTO,
            stream: torch.cuda.Stream | None = None, check_rows: bool = True) -> torch.Tensor:
    """Causal paged prefill on device tensors; returns out [total_q][Hq][D].

    q [total_q][Hq][D]; q_start int32 [S + 1] row offsets: sequence b owns
    rows q_start[b] .. q_start[b+1]-1, its newest tokens (already in the
    pools), row i at position seq_lens[b] - n_b + i attending tokens 0 ..
    that position.  max_q_len: the largest n_b (read from q_start on the
    host when not given).  check_rows (default): read q_start on the host
    (synchronises) and check that it starts at 0, ends at q's row count and
    that max_q_len covers every row range; pass False only with a q_start
    already checked.  Pools and tables as for decode(); fp16 / bf16 only."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_tables", block_tables), ("seq_lens", seq_lens), ("q_start", q_start)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 or q_start.dtype != torch.int32:
        raise TypeError("block_tables, seq_lens and q_start must be int32")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    S = seq_lens.shape[0]
    if q_start.shape != (S + 1,):
        raise ValueError("q_start must be [num_seqs + 1]")
    NB, Hkv, B, D = k_pool.shape
    if B % 16 != 0 or tuple(v_pool.shape) != (NB, Hkv, B // 16, D, 16):
        raise ValueError("v_pool must be [num_blocks][num_kv_heads][block_size/16][head_dim][16]")
    _check_table(block_tables, S)
    T, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q and k_pool head_dim differ")
    if max_q_len is None or check_rows:
        # reads q_start on the host (synchronises): rows must match q, and
        # the launch must cover the longest row range
        qs = q_start.cpu()
        n_b = qs[1:] - qs[:-1]
        if S and (int(qs[0]) != 0 or int(n_b.min()) < 0):
            raise ValueError("q_start must start at 0 and be non-decreasing")
        if int(qs[-1]) != T:
            raise ValueError(f"q_start[-1] = {int(qs[-1])} but q has {T} rows")
        longest = int(n_b.max()) if S else 0
        if max_q_len is None:
            max_q_len = longest
        elif max_q_len < longest:
            raise ValueError(f"max_q_len {max_q_len} is below the longest row range {longest}")
    dt = pa_dtype_of(q.dtype)
    odt = dt if out_dtype is None else pa_dtype_of(out_dtype)
    desc = _lib.PaDesc(S, Hq, Hkv, D, B, NB, block_tables.shape[1], dt, odt, kernel, 0)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    else:
        _check_out(out, q, out_dtype)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    _lib.paged_attn_prefill(q, k_pool, v_pool, block_tables, seq_lens, q_start, max_q_len, scale,
                            out, desc, st.cuda_stream)
    return out


def _check_table(block_tables: torch.Tensor, num_seqs: int) -> None:
    if not block_tables.is_cuda or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous device tensor")
    if block_tables.dtype != torch.int32:
        raise TypeError("block_tables must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")


def _pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor, num_seqs: int,
               max_blocks_per_seq: int) -> _lib.PaDesc:
    """Descriptor for the calls that work on the pools alone (they use the
    pool shape and the table width; the query-head count is set to the
    KV-head count)."""
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if v_pool.dtype != k_pool.dtype:
        raise TypeError("k_pool and v_pool must share a dtype")
    NB, Hkv, B, D = k_pool.shape
    if B % 16 != 0 or tuple(v_pool.shape) != (NB, Hkv, B // 16, D, 16):
        raise ValueError("v_pool must be [num_blocks][num_kv_heads][block_size/16][head_dim][16]")
    dt = pa_dtype_of(k_pool.dtype)
    return _lib.PaDesc(num_seqs, Hkv, Hkv, D, B, NB, max_blocks_per_seq, dt, _lib.PA_F32,
                       _lib.PA_KERNEL_AUTO, 0)


def append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_tables: torch.Tensor, positions: torch.Tensor, *,
           stream: torch.cuda.Stream | None = None) -> None:
    """Write one new token per sequence in place: k_new / v_new
    [S][Hkv][D] go to logical slot positions[b] of sequence b (skipped
    where positions[b] < 0) through its block table."""
    S = positions.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new), ("positions", positions)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if positions.dtype != torch.int32:
        raise TypeError("positions must be int32")
    _check_table(block_tables, S)
    desc = _pool_desc(k_pool, v_pool, S, block_tables.shape[1])
    want = (S, desc.num_kv_heads, desc.head_dim)
    if tuple(k_new.shape) != want or tuple(v_new.shape) != want:
        raise ValueError(f"k_new and v_new must be {list(want)}")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise TypeError("k_new, v_new and the pools must share a dtype")
    st = stream if stream is not None else torch.cuda.current_stream(k_pool.device)
    _lib.paged_kv_append(k_new, v_new, k_pool, v_pool, block_tables, positions, desc,
                         st.cuda_stream)


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, src_blocks: torch.Tensor,
                dst_blocks: torch.Tensor, *, stream: torch.cuda.Stream | None = None) -> None:
    """Copy-on-write step: physical block dst_blocks[i] of both pools
    becomes a copy of src_blocks[i] (int32 device tensors of one length)."""
    n = src_blocks.shape[0]
    if dst_blocks.shape[0] != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    for name, t in (("src_blocks", src_blocks), ("dst_blocks", dst_blocks)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    desc = _pool_desc(k_pool, v_pool, 1, 1)
    st = stream if stream is not None else torch.cuda.current_stream(k_pool.device)
    _lib.paged_kv_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, n, desc, st.cuda_stream)


def block_scores(k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                 seq_lens: torch.Tensor, *, stream: torch.cuda.Stream | None = None):
    """Block-wise eviction scores: (scores float32 [S][max_blocks_per_seq],
    NaN past each sequence's full blocks; evict int32 [S], the block to drop
    for sequences whose last block just filled, else -1)."""
    if not seq_lens.is_cuda or not seq_lens.is_contiguous() or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be a contiguous int32 device tensor")
    S = seq_lens.shape[0]
    _check_table(block_tables, S)
    desc = _pool_desc(k_pool, v_pool, S, block_tables.shape[1])
    scores = torch.empty((S, block_tables.shape[1]), dtype=torch.float32, device=k_pool.device)
    evict = torch.empty(S, dtype=torch.int32, device=k_pool.device)
    st = stream if stream is not None else torch.cuda.current_stream(k_pool.device)
    _lib.paged_kv_block_scores(k_pool, v_pool, block_tables, seq_lens, scores, evict, desc,
                               st.cuda_stream)
    return scores, evict
