"""The test-side input transforms, pinned on the CPU with the oracle: a
re-layout must not change what the oracle computes, and the key shift
must shift each head's scores by a constant."""
import numpy as np
import pytest

import oracle
import workload
from tests.relayout import logical_kv, repack, shift_keys, to_f32, zero_queries


@pytest.fixture(scope="module")
def O():
    return oracle.load()


def _small(dtype="bf16", lens=(1, 15, 16, 17, 40, 70), G=2):
    return workload.build(name="t", dtype=dtype, seq_lens=list(lens), num_q_heads=2 * G,
                          num_kv_heads=2, head_dim=128, block_size=16, seed=41)


def test_repack_keeps_the_logical_values_and_the_result(O):
    w = _small()
    w32 = repack(w, 32, seed=1)
    w16 = repack(w32, 16, seed=2)
    for (K, V), (K2, V2) in zip(logical_kv(w), logical_kv(w32)):
        assert np.array_equal(K, K2) and np.array_equal(V, V2)
    ref = O.run_workload(w)
    assert np.array_equal(O.run_workload(w32), ref)
    assert np.array_equal(O.run_workload(w16), ref)
    assert w32.block_size == 32 and not np.array_equal(w16.block_tables, w.block_tables)


def test_logical_kv_reads_the_slots_the_table_names():
    w = workload.make(1)
    K, V = logical_kv(w)[0]
    assert np.array_equal(K[0, 0], w.k_pool[7, 0, 0]) and np.array_equal(K[59, 0], w.k_pool[4, 0, 11])
    assert np.array_equal(V[18, 0], w.v_pool[1, 0, 0, :, 2])
    assert np.isfinite(K).all() and np.isfinite(V).all()


def test_key_shift_moves_each_heads_scores_by_a_constant(O):
    w = _small(dtype="f32")
    ws = shift_keys(w, 100.0)
    G = w.group
    for b, ((K, _), (Ks, _)) in enumerate(zip(logical_kv(w), logical_kv(ws))):
        for h in range(w.num_q_heads):
            q = w.q[b, h].astype(np.float64)
            d = float(w.scale) * (Ks[:, h // G].astype(np.float64) - K[:, h // G]) @ q
            assert np.ptp(d) < 1e-3
            if h % G == 0:
                assert abs(d[0] - 100.0) < 1e-2
    # fp32 keys are rounded once after the shift: the result barely moves
    assert np.max(np.abs(O.run_workload(ws) - O.run_workload(w))) < 1e-4


def test_zero_query_oracle_is_the_mean(O):
    w = zero_queries(_small())
    got = O.run_workload(w)
    for b, (K, V) in enumerate(logical_kv(w)):
        m = to_f32(V, w.dtype).astype(np.float64).mean(axis=0)
        assert np.allclose(got[b], np.repeat(m, w.group, axis=0), rtol=0, atol=1e-12)
