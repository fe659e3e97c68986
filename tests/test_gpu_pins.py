"""The oracle's pins carried over to the gfx950 library: closed forms that
fix the result without the oracle, and transforms of the inputs that must
leave the result unchanged ("39 · PagedAttention", §2: the paged result is
plain attention over the sequence's own keys and values, however the
blocks are placed and however large the blocks are)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workload
from tests.gpu_util import TOL, Uploaded, kernels_for, max_err
from tests.relayout import logical_kv, repack, shift_keys, to_f32, zero_queries

pytestmark = pytest.mark.gpu

# lengths around block boundaries plus a few long enough to be split over
# several workgroups
LENS = [1, 15, 16, 17, 33, 100, 511, 1000, 2047, 3001, 6000, 8192]


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.load()


def _case(dtype="bf16", G=4, B=16, seed=31, lens=LENS):
    return workload.build(name="pins", dtype=dtype, seq_lens=lens, num_q_heads=2 * G,
                          num_kv_heads=2, head_dim=128, block_size=B, seed=seed)


@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_block_size_16_and_32_agree(O, G):
    """The same logical K/V in 16-token and 32-token blocks (fresh random
    placement): the oracle gives identical fp64 bits, the library stays
    within the bar of it with either block size."""
    w16 = _case(G=G)
    w32 = repack(w16, 32, seed=32)
    ref = O.run_workload(w16)
    assert np.array_equal(O.run_workload(w32), ref)
    a, b = Uploaded(w16), Uploaded(w32)
    for kern in kernels_for("bf16"):
        _log(f"[pins] block size 16 vs 32, G={G} kernel={kern}")
        assert max_err(a.run(kern), ref) <= TOL["bf16"], (kern, 16)
        assert max_err(b.run(kern), ref) <= TOL["bf16"], (kern, 32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_keys_shifted_by_a_common_vector(O, dtype):
    """Adding one vector to every key of a (sequence, KV head) moves each
    head's scores by a constant.  The vector is chosen so the first head
    of each group gains +100 (natural-log units): exp(100) overflows fp32,
    so a kernel that did not subtract the running max would fail.
    Compared with the oracle on the same rounded, shifted keys."""
    w = shift_keys(_case(dtype=dtype, seed=33), 100.0)
    ref = O.run_workload(w)
    up = Uploaded(w)
    for kern in kernels_for(dtype):
        _log(f"[pins] key shift +100, {dtype} kernel={kern}")
        assert max_err(up.run(kern), ref) <= TOL[dtype], kern


def test_zero_query_gives_the_mean_of_exactly_L_values():
    """q = 0: every score is 0, every weight 1/L, so out is the plain mean
    of the sequence's L value rows (computed here from the logical values,
    not by the oracle).  A slack slot of a partial last block taken in, or
    a valid one left out, moves the mean."""
    w = zero_queries(_case(seed=34))
    mean = np.zeros(w.q.shape, np.float64)
    G = w.group
    for b, (K, V) in enumerate(logical_kv(w)):
        v = to_f32(V, w.dtype).astype(np.float64)         # [L][Hkv][D]
        mean[b] = np.repeat(v.mean(axis=0), G, axis=0)    # head h reads KV head h // G
    up = Uploaded(w)
    for kern in kernels_for(w.dtype):
        assert max_err(up.run(kern), mean) <= TOL[w.dtype], kern


@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_single_token_returns_its_value_row_exactly(G):
    """L = 1: the one weight is exactly 1, so out equals the value row
    bit for bit (fp32 output of bf16 values)."""
    w = _case(G=G, seed=35, lens=[1] * 9)
    want = np.zeros(w.q.shape, np.float32)
    for b, (K, V) in enumerate(logical_kv(w)):
        want[b] = np.repeat(to_f32(V[0], w.dtype), G, axis=0)
    up = Uploaded(w)
    for kern in kernels_for(w.dtype):
        got = up.run(kern).cpu().numpy()
        assert np.array_equal(got, want), kern


def test_dominant_score_selects_its_value_row(O):
    """A large scale makes one score dominate: out tends to the value row
    of the arg-max key.  Heads whose two best scores are far apart (every
    other weight below e^-40) must return that row to within 1e-6; every
    head must match the oracle at the same scale."""
    import dataclasses
    w = dataclasses.replace(_case(seed=36, lens=[17, 100, 333, 1000, 4000]), scale=np.float32(40.0))
    G = w.group
    want, clear = np.zeros(w.q.shape), np.zeros(w.q.shape[:2], bool)
    for b, (K, V) in enumerate(logical_kv(w)):
        k = to_f32(K, w.dtype).astype(np.float64)
        v = to_f32(V, w.dtype).astype(np.float64)
        for h in range(w.num_q_heads):
            s = float(w.scale) * (k[:, h // G, :] @ to_f32(w.q[b, h], w.dtype).astype(np.float64))
            top = np.argsort(s)[::-1]
            want[b, h] = v[top[0], h // G]
            clear[b, h] = s[top[0]] - s[top[1]] > 40.0
    assert clear.sum() >= clear.size // 2
    ref = O.run_workload(w)
    up = Uploaded(w)
    for kern in kernels_for(w.dtype):
        got = up.run(kern)
        assert max_err(got, ref) <= TOL[w.dtype], kern
        g = got.double().cpu().numpy()
        assert np.max(np.abs(g - want)[clear]) <= 1e-6, kern
