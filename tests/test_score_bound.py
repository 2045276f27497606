"""The error bound that the library's selection relies on (no GPU).

The fast block scores use the pooled keys rounded to bf16 with fp32
accumulation; the library stores, per score row, softmax_scale x the largest
query-row norm x the largest |kbar_J - bf16(kbar_J)|_2 + 2^-17 |bf16(kbar_J)|_2
and re-checks in float64 every entry within twice that bound (plus 2e-3) of a
decision.  These tests emulate the fast path on the CPU and check the bound
against the oracle's exact scores, and check that it is reached (so a bound
that dropped a factor would fail)."""

import numpy as np

from gpu_parity_util import score_bound
from oracle import OracleProblem, block_scores, pool_blocks
from oracle.flashprefill import bf16_round
from synthetic import custom_spec, make_workload


def fast_scores(q_rows, kbar, scale):
    """The fast path's arithmetic: kbar rounded to fp32 then bf16, dot
    products of the exact bf16 products accumulated in fp32, the max-
    normalised exp-sum in float64 (the statistics' own rounding is covered
    separately by the selection's 2e-3 allowance)."""
    kb = bf16_round(kbar.astype(np.float32)).astype(np.float32)
    x = (q_rows.astype(np.float32) @ kb.T).astype(np.float64) * scale
    m = x.max(axis=0)
    return m + np.log(np.exp(x - m).sum(axis=0))


def test_fast_scores_within_bound_on_synthetic_rows():
    w = make_workload(custom_spec((1100, 700), 8, 2, page_size=16, seed=11, name="bound"))
    prob = OracleProblem.from_workload(w)
    worst = 0.0
    for s in range(prob.num_seqs):
        for h in range(prob.hkv):
            km, cnt = pool_blocks(prob.keys(s, h), prob.block_size)
            # the library's fp32 pooled keys, laid out [Hkv, N, d]
            k_mean = np.zeros((prob.hkv, int(prob.block_offsets()[-1]), prob.d))
            kb0 = int(prob.block_offsets()[s])
            k_mean[h, kb0:kb0 + len(km)] = km.astype(np.float32)
            for I in prob.query_blocks(s):
                nI = int(cnt[I])
                qg = prob.queries(s, prob.list_heads(h), I * 128 + np.arange(nI)).reshape(-1, prob.d)
                exact = block_scores(qg, km[:I + 1], prob.scale)["L"]
                fast = fast_scores(qg, k_mean[h, kb0:kb0 + I + 1], prob.scale)
                bnd = score_bound(prob, k_mean, h, s, I)
                err = float(np.max(np.abs(fast - exact)))
                assert err <= bnd + 1e-9, (s, h, I, err, bnd)
                worst = max(worst, err / bnd)
    # the realised errors are well inside the bound on random data
    assert worst < 1.0


def test_bound_is_reached_by_an_aligned_query():
    """A single query row along the rounding residual of kbar: its logit moves
    by exactly softmax_scale |q| |kbar - bf16(kbar)| (no fp32 term in play at
    this size), i.e. the Cauchy-Schwarz part of the bound is attained."""
    rng = np.random.default_rng(5)
    d = 128
    scale = 1.0 / np.sqrt(d)
    kbar = rng.normal(size=d).astype(np.float32).astype(np.float64)
    resid = kbar - bf16_round(kbar)
    q = bf16_round(40.0 * resid / np.linalg.norm(resid))  # as consumed (bf16)
    exact = scale * float(q @ kbar)
    fast = scale * float(np.float64(q.astype(np.float32) @ bf16_round(kbar).astype(np.float32)))
    shift = abs(fast - exact)
    cs = scale * np.linalg.norm(q) * np.linalg.norm(resid)
    assert shift <= cs * (1 + 1e-6) + 1e-7
    assert shift >= 0.95 * cs
