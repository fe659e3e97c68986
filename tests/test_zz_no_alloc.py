"""The allocation-free decode entry point (paged_attn_decode_noalloc, static
device scratch) against paged_attn_decode with a caller workspace, both
through the C ABI on the same uploaded inputs: bit-identical outputs (same
kernels, same fold order) and each within the oracle bar.  Two calls in a
row with the second smaller, so the second runs on scratch the first left
behind."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_196_amd as pa
import workload
from tests.gpu_util import TOL, Uploaded, max_err

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.load()


def _run_both(up, kernel, out_dtype=torch.float32):
    w = up.w
    dev = up.q.device
    desc = pa.make_desc(up.q, up.k, up.bt, out_dtype=out_dtype, kernel=kernel)
    st = torch.cuda.current_stream(dev).cuda_stream
    ws = pa.new_workspace(desc, dev)
    with_ws = torch.full(up.q.shape, float("nan"), dtype=out_dtype, device=dev)
    pa.paged_attn_decode(up.q, up.k, up.v, up.bt, up.lens, float(w.scale), with_ws, desc, ws,
                         ws.numel(), st)
    no_alloc = torch.full(up.q.shape, float("nan"), dtype=out_dtype, device=dev)
    pa.paged_attn_decode_noalloc(up.q, up.k, up.v, up.bt, up.lens, float(w.scale), no_alloc, desc,
                                 st)
    torch.cuda.synchronize(dev)
    return with_ws, no_alloc


CASES = [
    # (name, workload kwargs): a larger call, then a smaller one
    ("gqa", dict(cfg=3, seed=111, batch=24, max_len=6000), dict(cfg=3, seed=112, batch=5, max_len=2500)),
    ("serving", dict(cfg=5, seed=113, batch=40), dict(cfg=5, seed=114, batch=9)),
]


@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_no_alloc_matches_workspace_entry(O, name, big, small):
    for label, kw in (("first", big), ("second (smaller)", small)):
        w = workload.make(kw["cfg"], kw["seed"], batch=kw["batch"], max_len=kw.get("max_len"))
        _log(f"[no_alloc] {name} {label}: {w.name} S={w.num_seqs} G={w.group}")
        ref = O.run_workload(w)
        up = Uploaded(w)
        a, b = _run_both(up, pa.PA_KERNEL_AUTO)
        assert torch.equal(a, b), f"{name} {label}: outputs differ"
        err = max_err(b, ref)
        _log(f"[no_alloc] {name} {label}: max_abs_err={err:.3e}")
        assert err <= TOL[w.dtype], (name, label, err)


def test_no_alloc_group16_then_fp32_vector_alu(O):
    """The largest group the matrix cores take (most scratch per slot),
    then an fp32 call on the vector-ALU kernel with a smaller group."""
    rng = np.random.default_rng(7)
    for dtype, G, kern, lens in (("bf16", 16, pa.PA_KERNEL_MFMA, rng.integers(1, 3000, 12)),
                                 ("f32", 2, pa.PA_KERNEL_VALU, rng.integers(1, 900, 5))):
        w = workload.build(name=f"noalloc-{dtype}-g{G}", dtype=dtype, seq_lens=list(lens),
                           num_q_heads=2 * G, num_kv_heads=2, head_dim=128, block_size=16,
                           seed=int(rng.integers(1 << 30)))
        _log(f"[no_alloc] {w.name} S={w.num_seqs}")
        ref = O.run_workload(w)
        a, b = _run_both(Uploaded(w), kern)
        assert torch.equal(a, b), w.name
        assert max_err(b, ref) <= TOL[dtype], w.name


def test_no_alloc_mqa_groups_run_as_virtual_groups(O):
    """MQA groups (64, then 32 query heads on one KV head): the
    column-split kernel's partials would overflow the static scratch, so
    the allocation-free entry runs them as virtual groups of 16 heads.  Its
    output matches the workspace entry's (column-split kernel) to the
    oracle bar, and each is within the bar of the oracle."""
    for Hq, batch, max_len in ((64, 10, 4000), (32, 4, 2000)):
        w = workload.make_mqa(Hq, seed=40 + Hq, batch=batch, max_len=max_len)
        _log(f"[no_alloc] {w.name} S={w.num_seqs}")
        ref = O.run_workload(w)
        a, b = _run_both(Uploaded(w), pa.PA_KERNEL_AUTO)
        assert max_err(a, ref) <= TOL["bf16"] and max_err(b, ref) <= TOL["bf16"], Hq
        assert float((a - b).abs().max()) <= TOL["bf16"], Hq


def test_no_alloc_bf16_output_and_empty_batch():
    w = workload.build(name="noalloc-out16", dtype="bf16", seq_lens=[0, 37, 700, 16], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=32, seed=9)
    a, b = _run_both(Uploaded(w), pa.PA_KERNEL_AUTO, out_dtype=torch.bfloat16)
    assert torch.equal(a, b)
    # a batch of zero sequences launches nothing and succeeds
    up = Uploaded(w)
    desc = pa.make_desc(up.q[:0], up.k, up.bt[:0])
    pa.paged_attn_decode_noalloc(up.q[:0], up.k, up.v, up.bt[:0], up.lens[:0], 1.0,
                                 up.q[:0].float(), desc, None)
