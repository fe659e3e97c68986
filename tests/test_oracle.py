"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import workload
from tests import oracle_pins


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__[4:])
def test_pin(O, pin):
    pin(O)


def test_worked_example_workload_is_finite_and_matches_numpy(O):
    """The toy workload (60 tokens, table 7,1,12,4, NaN in every slot the
    request does not own) through the oracle and the independent numpy
    evaluation."""
    w = workload.make(1)
    got = O.run_workload(w)
    want = oracle_pins.numpy_reference(w.q.astype(np.float64), w.k_pool.astype(np.float64),
                                       w.v_pool.astype(np.float64), w.block_tables, w.seq_lens,
                                       float(w.scale), w.num_kv_heads, w.block_size)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_named_workloads_small_batch_match_numpy(O, cfg):
    """Each named workload at a reduced batch (bf16/f16 storage widened
    exactly) against the independent numpy evaluation."""
    w = workload.make(cfg, batch={2: 1, 3: 1, 4: 1, 5: 9}[cfg], max_len=600)
    got = O.run_workload(w)
    to64 = (lambda x: O.to_f64(x, w.dtype))
    want = oracle_pins.numpy_reference(to64(w.q), to64(w.k_pool), to64(w.v_pool),
                                       w.block_tables, w.seq_lens, float(w.scale),
                                       w.num_kv_heads, w.block_size)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) < 1e-12
