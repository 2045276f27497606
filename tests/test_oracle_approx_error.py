"""The approximation-error measurement (oracle.approx_error) on small cases
(no GPU): with every block kept (alpha = 0) the sparse oracle equals the
dense reference, and with blockwise-constant keys the mean correction makes
it exact at any alpha (the correction then replaces each pruned block by
exactly its own contribution), while the uncorrected output is not."""

import numpy as np

from oracle import OracleProblem
from oracle.approx_error import measure
from synthetic import custom_spec, make_workload


def test_alpha_zero_is_dense():
    prob = OracleProblem.from_workload(make_workload(custom_spec((900,), 4, 1, page_size=64, seed=61)))
    acc = measure(prob, 0, 0, np.arange(7), (0.0,))
    for corr in (True, False):
        mx, _, _, kept, causal = acc[(0.0, corr)]
        assert kept == causal and mx < 1e-12


def test_constant_key_blocks_make_the_correction_exact():
    w = make_workload(custom_spec((1024,), 4, 1, qk_dtype="f32", v_dtype="f32", page_size=128,
                                  paging="identity", seed=62))
    prob = OracleProblem.from_workload(w)
    # every key of a block equal to the block's first key (values untouched)
    k = prob.k_cache.reshape(-1, 1, 128)
    for J in range(8):
        k[J * 128:(J + 1) * 128] = k[J * 128]
    acc = measure(prob, 0, 0, np.arange(8), (0.5,))
    mx_on, _, _, kept, causal = acc[(0.5, True)]
    mx_off = acc[(0.5, False)][0]
    assert kept < causal            # blocks were pruned
    assert mx_on < 1e-12 < mx_off
