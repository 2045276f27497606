"""The error bound that the library's selection relies on (no GPU).

The fast block scores use the exact (float64) pooled keys times
c = softmax_scale log2(e), rounded to bf16 (s_J), with fp32 accumulation
(log2-domain logits); the library stores, per score row, ln 2 x the largest
query-row norm x the largest |c kbar_J - s_J|_2 + 2^-15 |s_J|_2 and
re-checks in float64 every entry within twice that bound (plus the
statistics allowance) of a decision.  These tests emulate the fast path on
the CPU and check the bound against the oracle's exact scores, and check
that it is reached (so a bound that dropped a factor would fail)."""

import numpy as np
import pytest

from gpu_parity_util import LN2, LOG2E, bf16_round64, score_bound
from oracle import OracleProblem, block_scores, pool_blocks
from synthetic import custom_spec, make_workload


def fast_scores(q_rows, kbar, scale):
    """The fast path's arithmetic: c kbar (c = scale log2(e), in float64)
    rounded once to bf16, dot products of the exact bf16 products
    accumulated in fp32 (log2-domain logits), the max-normalised exp-sum in
    float64, converted to natural log (the statistics' own rounding is
    covered separately by the selection's allowance)."""
    kb = bf16_round64(kbar * (scale * LOG2E)).astype(np.float32)
    x = (q_rows.astype(np.float32) @ kb.T).astype(np.float64) * LN2
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
    """A single query row along the rounding residual of c kbar: its logit
    moves by exactly ln 2 |q| |c kbar - bf16(c kbar)| in natural-log units (no
    fp32 term in play at this size), i.e. the Cauchy-Schwarz part of the
    bound is attained."""
    rng = np.random.default_rng(5)
    d = 128
    scale = 1.0 / np.sqrt(d)
    c = scale * LOG2E
    kbar = rng.normal(size=d)
    resid = c * kbar - bf16_round64(c * kbar)
    q = bf16_round64(40.0 * resid / np.linalg.norm(resid))  # as consumed (bf16)
    exact = scale * float(q @ kbar)
    fast = LN2 * float(np.float64(q.astype(np.float32) @ bf16_round64(c * kbar).astype(np.float32)))
    shift = abs(fast - exact)
    cs = LN2 * np.linalg.norm(q) * np.linalg.norm(resid)
    assert shift <= cs * (1 + 1e-6) + 1e-7
    assert shift >= 0.95 * cs


def _stats_fp32(acc, csc, ref=None, direct=False):
    """The scores kernel's fp32 statistics of one key column, step by step.
    acc [passes, 8 waves, 2 lanes, 32]: fp32 dot products of the column with
    the rows of a query block (a pass covers 512 rows: 8 waves x 2 chunks of
    32 rows; the lane pair l, l^32 of a wave holds 32 rows each); csc the
    factor that makes them log2-domain logits (1 for bf16 queries, the head's
    q_scale for e4m3); ref [passes] the column's log2-domain reference per
    pass (None: the column max); direct: no reference (csc must be 1), the
    lanes sum 2^x of the logits as they are.  Per wave the lanes' sequential
    exp2-sums against the reference (fma rounded once), added; a wave whose
    sum is below 2^-64 falls back to its own max (per lane the scaled max,
    pair max).  Per pass the waves merged against the largest of their
    references, L = (m + log2 sum) ln 2; passes merged by a log-sum-exp.
    float32 throughout."""
    f = np.float32
    ln2 = f(np.log(2.0))
    L = None
    assert not direct or csc == 1

    def wave_sum(pw, r):
        tot = f(0)
        for k in range(2):
            lane = f(0)
            for v in pw[k]:
                arg = v if direct and r == 0 else f(float(v) * float(csc) - float(r))
                lane = f(lane + np.exp2(f(arg)))
            tot = f(tot + lane)
        return tot

    for p, pa in enumerate(acc.astype(np.float32)):
        m_w = np.zeros(pa.shape[0], dtype=f)
        s_w = np.zeros(pa.shape[0], dtype=f)
        for w in range(pa.shape[0]):
            s = None
            if direct:
                m_w[w] = f(0)
                s = wave_sum(pa[w], 0.0)
            elif ref is not None:
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


def _exact_L(acc, csc):
    """float64 log-sum-exp (natural log) of the fp32 dot products' logits."""
    x = acc.astype(np.float64) * float(csc) * np.log(2.0)
    M = x.max()
    return M + np.log(np.exp(x - M).sum())


@pytest.mark.parametrize("csc", [1.0, 0.0371])
@pytest.mark.parametrize("mag", [1.0, 30.0, 1e3, 1e4])
@pytest.mark.parametrize("gap", [None, 0.0, 20.0, 60.0, 75.0])
def test_fp32_statistics_within_the_selection_allowance(mag, gap, csc):
    """The selection allows stat(L) = 1e-3 + 2^-17 |L| for the fp32
    statistics of a score (natural-log units); the emulated fp32 statistics
    stay below 1e-4 + 2^-19 |L| (the figure the interface states) at logit
    magnitudes from 1 to 1e4, i.e. well inside the allowance, whether the sums
    run against the column max (gap None) or against a reference that many
    log2 units above it (75: every wave's sum underflows the 2^-64 floor and
    falls back to its max), with a unit or an e4m3-like per-head factor."""
    rng = np.random.default_rng(int(mag) + (0 if gap is None else 7 + int(gap)) + (csc != 1.0))
    csc = np.float32(csc)
    for _ in range(4):
        # 2 passes x 8 waves x 2 lanes x 32 rows: the 1024 (head, token)
        # rows of a group of 8 heads
        x = rng.normal(size=(2, 8, 2, 32)) * 3.0 + mag  # natural-log logits
        acc = (x / (np.log(2.0) * float(csc))).astype(np.float32)
        L64 = _exact_L(acc, csc)
        ref = None
        if gap is not None:
            ref = [np.float32(float(pa.max()) * float(csc) + gap) for pa in acc]
        L32 = _stats_fp32(acc, csc, ref)
        err = abs(L32 - L64)
        assert err <= 1e-4 + 2.0 ** -19 * abs(L64), (mag, gap, err)
        assert err <= (1e-3 + 2.0 ** -17 * abs(L64)) / 4


@pytest.mark.parametrize("top", [-100.0, -60.0, -20.0, 0.0, 40.0, 112.0])
def test_fp32_direct_statistics_within_the_selection_allowance(top):
    """The reference-free sums (every logit of the pass at most 112 log2
    units, bf16 queries): 2^x summed as is.  Columns whose largest logit is
    `top` log2 units, spread over ~40 units below it: the sums neither
    overflow (top 112: a pass's sum stays below 2^122) nor lose accuracy, and
    columns far below zero (-100: every wave's sum underflows the 2^-64 floor
    and falls back to its max) keep the same accuracy as the other paths."""
    rng = np.random.default_rng(1000 + int(top))
    for _ in range(4):
        x = rng.uniform(-40.0, 0.0, size=(2, 8, 2, 32))
        x += top - x.max()
        acc = x.astype(np.float32)  # log2-domain logits straight from the MFMA
        assert float(acc.max()) <= 112.0
        L64 = _exact_L(acc, 1.0)
        L32 = _stats_fp32(acc, np.float32(1.0), direct=True)
        assert np.isfinite(L32)
        err = abs(L32 - L64)
        assert err <= 1e-4 + 2.0 ** -19 * abs(L64), (top, err)
        assert err <= (1e-3 + 2.0 ** -17 * abs(L64)) / 4


def test_direct_statistics_fallback_is_taken_and_needed():
    """Planted check of the floor: with the fallback switched off, a column
    whose logits all lie between -165 and -145 log2 units loses its sums to
    underflow (terms below 2^-149 vanish, the others keep a few bits: the
    emulation then returns a value far off), so the floor test is what keeps
    such columns exact."""
    rng = np.random.default_rng(77)
    acc = (rng.uniform(-165.0, -145.0, size=(1, 8, 2, 32))).astype(np.float32)
    L64 = _exact_L(acc, 1.0)
    L32 = _stats_fp32(acc, np.float32(1.0), direct=True)
    assert abs(L32 - L64) <= 1e-4 + 2.0 ** -19 * abs(L64)
    f = np.float32
    raw = f(0)
    for v in acc.ravel():
        raw = f(raw + np.exp2(v))
    with np.errstate(divide="ignore"):
        bad = float(f(np.log2(raw)) * f(np.log(2.0)))
    assert not abs(bad - L64) <= 1e-2
