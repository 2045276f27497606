"""The error bound that the library's selection relies on (no GPU).

The fast block scores use the exact (float64) pooled keys rounded to bf16
with fp32 accumulation; the library stores, per score row, softmax_scale x
the largest query-row norm x the largest |kbar_J - bf16(kbar_J)|_2 + 2^-15
|bf16(kbar_J)|_2 and re-checks in float64 every entry within twice that
bound (plus the statistics allowance) of a decision.  These tests emulate the fast path on the CPU and check the bound
against the oracle's exact scores, and check that it is reached (so a bound
that dropped a factor would fail)."""

import numpy as np
import pytest

from gpu_parity_util import bf16_round64, score_bound
from oracle import OracleProblem, block_scores, pool_blocks
from synthetic import custom_spec, make_workload


def fast_scores(q_rows, kbar, scale):
    """The fast path's arithmetic: kbar rounded once to bf16, dot products
    of the exact bf16 products accumulated in fp32, the max-normalised
    exp-sum in float64 (the statistics' own rounding is covered separately
    by the selection's allowance)."""
    kb = bf16_round64(kbar).astype(np.float32)
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
            # the float64 pooled keys, laid out [Hkv, N, d]
            k_mean = np.zeros((prob.hkv, int(prob.block_offsets()[-1]), prob.d))
            kb0 = int(prob.block_offsets()[s])
            k_mean[h, kb0:kb0 + len(km)] = km
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
    kbar = rng.normal(size=d)
    resid = kbar - bf16_round64(kbar)
    q = bf16_round64(40.0 * resid / np.linalg.norm(resid))  # as consumed (bf16)
    exact = scale * float(q @ kbar)
    fast = scale * float(np.float64(q.astype(np.float32) @ bf16_round64(kbar).astype(np.float32)))
    shift = abs(fast - exact)
    cs = scale * np.linalg.norm(q) * np.linalg.norm(resid)
    assert shift <= cs * (1 + 1e-6) + 1e-7
    assert shift >= 0.95 * cs


def _stats_fp32(acc, csc, ref=None):
    """The scores kernel's fp32 statistics of one key column, step by step.
    acc [passes, 8 waves, 2 lanes, 32]: fp32 dot products of the column with
    the rows of a query block (a pass covers 512 rows: 8 waves x 2 chunks of
    32 rows; the lane pair l, l^32 of a wave holds 32 rows each); csc is the
    log2-domain logit scale; ref [passes] the column's log2-domain reference
    per pass (None: the column max).  Per wave the lanes' sequential
    exp2-sums against the reference (fma rounded once), added; a wave whose
    sum is below 2^-64 falls back to its own max (per lane the scaled max,
    pair max).  Per pass the waves merged against the largest of their
    references, L = (m + log2 sum) ln 2; passes merged by a log-sum-exp.
    float32 throughout."""
    f = np.float32
    ln2 = f(np.log(2.0))
    L = None

    def wave_sum(pw, r):
        tot = f(0)
        for k in range(2):
            lane = f(0)
            for v in pw[k]:
                lane = f(lane + np.exp2(f(float(v) * float(csc) - float(r))))
            tot = f(tot + lane)
        return tot

    for p, pa in enumerate(acc.astype(np.float32)):
        m_w = np.zeros(pa.shape[0], dtype=f)
        s_w = np.zeros(pa.shape[0], dtype=f)
        for w in range(pa.shape[0]):
            s = None
            if ref is not None:
                m_w[w] = f(ref[p])
                s = wave_sum(pa[w], m_w[w])
            if s is None or not s >= 2.0 ** -64:
                m_w[w] = max(f(float(pa[w, k].max()) * float(csc)) for k in range(2))
                s = wave_sum(pa[w], m_w[w])
            s_w[w] = s
        m = m_w.max()
        ssum = f(0)
        for w in range(pa.shape[0]):
            ssum = f(ssum + f(s_w[w] * np.exp2(f(m_w[w] - m))))
        Lp = f(f(m + np.log2(ssum)) * ln2)
        if L is None:
            L = Lp
        else:
            hi = max(L, Lp)
            L = f(hi + np.log(f(np.exp(f(L - hi)) + np.exp(f(Lp - hi)))))
    return float(L)


@pytest.mark.parametrize("mag", [1.0, 30.0, 1e3, 1e4])
@pytest.mark.parametrize("gap", [None, 0.0, 20.0, 60.0, 75.0])
def test_fp32_statistics_within_the_selection_allowance(mag, gap):
    """The selection allows stat(L) = 1e-3 + 2^-17 |L| for the fp32
    statistics of a score (natural-log units); the emulated fp32 statistics
    stay below 1e-4 + 2^-19 |L| (the figure the interface states) at logit
    magnitudes from 1 to 1e4, i.e. well inside the allowance, whether the sums
    run against the column max (gap None) or against a reference that many
    log2 units above it (75: every wave's sum underflows the 2^-64 floor and
    falls back to its max)."""
    rng = np.random.default_rng(int(mag) + (0 if gap is None else 7 + int(gap)))
    scale = 1.0 / np.sqrt(128)
    csc = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    for _ in range(4):
        # 2 passes x 8 waves x 2 lanes x 32 rows: the 1024 (head, token)
        # rows of a group of 8 heads
        x = rng.normal(size=(2, 8, 2, 32)) * 3.0 + mag
        acc = (x / (scale * 1.4426950408889634)).astype(np.float32)
        exact_x = acc.astype(np.float64) * scale  # natural-log logits of the fp32 dot products
        M = exact_x.max()
        L64 = M + np.log(np.exp(exact_x - M).sum())
        ref = None
        if gap is not None:
            ref = [np.float32(float(pa.max()) * float(csc) + gap) for pa in acc]
        L32 = _stats_fp32(acc, csc, ref)
        err = abs(L32 - L64)
        assert err <= 1e-4 + 2.0 ** -19 * abs(L64), (mag, gap, err)
        assert err <= (1e-3 + 2.0 ** -17 * abs(L64)) / 4