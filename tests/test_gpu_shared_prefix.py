"""GPU parity of the shared-prefix decode (paged_attn_decode_shared, prefix
groups read once per group) through the C ABI: every output against the
fp64 oracle on the same seeded inputs.  The oracle attends each sequence
through its own table row, so sharing blocks changes no result; the bar is
the decode bar, max |out - oracle| <= 2e-3 for fp16 / bf16 inputs with fp32
output (2e-3 + half an ulp of the output type for 16-bit output)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_196_amd as pa
import workload
from tests.gpu_util import TOL, Uploaded, max_err, run_shared

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.load()


def test_serving_workload_full_size(O):
    """Batch 256, groups of 8 sharing 32 blocks (512 tokens), lognormal
    lengths (a quarter of the members end inside the shared prefix): every
    output, fp32 and bf16 output."""
    w = workload.make(5)
    ref = O.run_workload(w)
    up = Uploaded(w)
    _log(f"[shared] {w.name} groups={w.num_groups}")
    err = max_err(run_shared(up), ref)
    _log(f"[shared] full size max_abs_err={err:.3e}")
    assert err <= TOL["bf16"], err
    out16 = run_shared(up, out_dtype=torch.bfloat16).double().cpu().numpy()
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
    assert np.all(np.abs(out16 - ref) <= 2e-3 + half_ulp)


@pytest.mark.parametrize("seed", [101, 102, 103])
def test_serving_workload_reduced(O, seed):
    w = workload.make(5, seed, batch=40)
    ref = O.run_workload(w)
    err = max_err(run_shared(Uploaded(w)), ref)
    _log(f"[shared] reduced seed {seed} max_abs_err={err:.3e}")
    assert err <= TOL["bf16"], (seed, err)


# members shorter than, equal to and longer than the shared prefix, an
# empty member, single-block members
def _edge_batch(rng, B, shared_blocks):
    P = shared_blocks * B
    pool = [1, 2, B - 1, B, B + 1, P - 1, P, P + 1, P + 17, 3 * P + 5, 0]
    return [int(x) for x in rng.choice(pool, size=len(pool), replace=False) if x >= 0]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_shapes(O, dtype, B, G):
    """Groups of 2, 3, 11 and (for G = 1) 40 members (more than one item's
    columns: the group is cut into sub-groups), shared prefixes of 1, 3, 8
    and 5 blocks, member lengths around the prefix end, an empty member and
    ungrouped sequences after the groups."""
    rng = np.random.default_rng(77 + B + 10 * G + (dtype == "f16"))
    sizes, blocks, lens = [2, 3, 11], [1, 3, 8], []
    if G == 1:
        sizes.append(40)
        blocks.append(5)
    for n, k in zip(sizes, blocks):
        e = _edge_batch(rng, B, k)
        lens += [e[i % len(e)] for i in range(n)]
    lens += [1, 333, 70]  # share nothing
    Hkv = 2
    w = workload.build(name=f"groups-{dtype}-B{B}-G{G}", dtype=dtype, seq_lens=lens,
                       num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=128, block_size=B,
                       seed=int(rng.integers(1 << 30)), group_sizes=sizes, group_blocks=blocks)
    ref = O.run_workload(w)
    err = max_err(run_shared(Uploaded(w)), ref)
    _log(f"[shared] {w.name} S={w.num_seqs} max_abs_err={err:.3e}")
    assert err <= TOL[dtype], (dtype, B, G, err)


def test_long_shared_prefix_cut_into_fragments(O):
    """Three groups sharing 700, 400 and 64 blocks with short private tails:
    the items are longer than a workgroup's share of item blocks, so chunk
    boundaries cut them into fragments that meet in the fold."""
    rng = np.random.default_rng(5)
    sizes, blocks = [4, 6, 3], [700, 400, 64]
    lens = []
    for n, k in zip(sizes, blocks):
        lens += [k * 16 + int(x) for x in rng.integers(-900, 300, size=n)]
    w = workload.build(name="long-shared", dtype="bf16", seq_lens=lens, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=16, seed=6, group_sizes=sizes,
                       group_blocks=blocks)
    ref = O.run_workload(w)
    err = max_err(run_shared(Uploaded(w)), ref)
    _log(f"[shared] long shared prefix max_abs_err={err:.3e}")
    assert err <= TOL["bf16"], err


def test_repeatable_and_workspace_reused(O):
    """Three calls on one workspace: the counters the fold uses are left at
    zero, so every call is right and bit-identical (fixed fold order)."""
    w = workload.make(5, 104, batch=64)
    ref = O.run_workload(w)
    up = Uploaded(w)
    ws = pa.new_shared_workspace(pa.make_desc(up.q, up.k, up.bt), up.q.device)
    outs = [run_shared(up, workspace=ws) for _ in range(3)]
    assert max_err(outs[0], ref) <= TOL["bf16"]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    # a different batch on the same workspace
    w2 = workload.make(5, 105, batch=24)
    assert max_err(run_shared(Uploaded(w2), workspace=pa.new_shared_workspace(
        pa.make_desc(Uploaded(w2).q, Uploaded(w2).k, Uploaded(w2).bt), up.q.device)),
        O.run_workload(w2)) <= TOL["bf16"]


def test_descriptors_without_the_shared_kernel_run_the_ordinary_decode(O):
    """Group size 16, fp32 inputs, the vector-ALU kernel and an empty group
    list take the ordinary decode with the same workspace: same results."""
    cases = [("bf16", 16, "auto", [3, 4], [2, 5]), ("f32", 2, "auto", [3, 4], [2, 5]),
             ("bf16", 4, "valu", [3, 4], [2, 5]), ("bf16", 4, "auto", [], [])]
    for dtype, G, kern, sizes, blocks in cases:
        lens = [50, 90, 20, 100, 8, 130, 64, 400]
        w = workload.build(name=f"fallback-{dtype}-{G}-{kern}", dtype=dtype, seq_lens=lens,
                           num_q_heads=2 * G, num_kv_heads=2, head_dim=128, block_size=16,
                           seed=G, group_sizes=sizes or None, group_blocks=blocks or None)
        ref = O.run_workload(w)
        err = max_err(run_shared(Uploaded(w), kernel=kern), ref)
        assert err <= TOL[dtype], (dtype, G, kern, err)
