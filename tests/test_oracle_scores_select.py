"""Pins of the oracle's pooling, pooled-score and selection steps against
closed forms, invariants and special cases (no GPU)."""

import math

import numpy as np
import pytest

from oracle import (OracleProblem, block_scores, forced_blocks, pool_blocks,
                    run_pipeline, select_row)
from synthetic import custom_spec, make_workload


# ---------------------------------------------------------------- pooling ---

def test_pool_linear_ramp_closed_form():
    """Rows a + t*b: the mean of block J is a + (first + (n_J-1)/2) * b, also
    for a partial last block."""
    B, d, L = 8, 3, 21
    a = np.array([1.0, -2.0, 0.5])
    b = np.array([0.25, 1.0, -0.125])
    x = a[None] + np.arange(L)[:, None] * b[None]
    means, counts = pool_blocks(x, B)
    assert list(counts) == [8, 8, 5]
    for J in range(3):
        first = J * B
        want = a + (first + (counts[J] - 1) / 2.0) * b
        assert np.allclose(means[J], want, rtol=0, atol=1e-13)


def test_pool_constant_blocks():
    x = np.repeat(np.array([[3.0, -1.0], [0.5, 2.0]]), [4, 3], axis=0)
    means, counts = pool_blocks(x, 4)
    assert np.array_equal(means, [[3.0, -1.0], [0.5, 2.0]])
    assert list(counts) == [4, 3]


def test_paged_gather_independent_of_page_layout():
    """The address rule (page base from the table + in-page offset) must
    give the same token sequence whatever the physical page order."""
    base = dict(seqlens=(300, 129, 1, 640), num_q_heads=4, num_kv_heads=2, seed=7)
    probs = [OracleProblem.from_workload(make_workload(custom_spec(**base, paging=pg, page_size=ps)))
             for pg, ps in [("identity", 128), ("permute", 16), ("roundrobin", 64), ("permute", 256)]]
    for s in range(4):
        for h in range(2):
            k0, v0 = probs[0].keys(s, h), probs[0].values(s, h)
            assert np.isfinite(k0).all() and np.isfinite(v0).all()
            for p in probs[1:]:
                assert np.array_equal(p.keys(s, h), k0)
                assert np.array_equal(p.values(s, h), v0)


# ---------------------------------------------------------- pooled scores ---

def test_scores_two_row_closed_form():
    """rows q1=(1,0), q2=(0,1); pooled keys (a,0), (0,b) with scale 1:
    L_0 = ln(e^a + 1), L_1 = ln(1 + e^b)."""
    a, b = 2.0, -3.0
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    km = np.array([[a, 0.0], [0.0, b]])
    r = block_scores(q, km, 1.0)
    assert np.allclose(r["L"], [math.log(math.exp(a) + 1), math.log(1 + math.exp(b))], atol=1e-14)
    assert np.allclose(r["M"], [a, 0.0])
    assert np.allclose(r["S"], [1 + math.exp(-a), 1 + math.exp(b)], atol=1e-14)
    # re-weighting against the top block: Score_J = sum_r exp(x_rJ - max x)
    assert np.allclose(r["Score"], [1 + math.exp(-a), math.exp(-a) + math.exp(b - a)], atol=1e-14)
    assert np.isclose(r["Shat"][0], 1.0) and np.isclose(
        r["Shat"][1], (1 + math.exp(b)) / (math.exp(a) + 1), atol=1e-14)


def test_scores_identical_rows():
    """R identical query rows: L_J = ln R + scale * q . kbar_J exactly."""
    rng = np.random.default_rng(3)
    R, d, n = 64, 16, 9
    q = np.tile(rng.standard_normal(d), (R, 1))
    km = rng.standard_normal((n, d))
    scale = 0.3
    r = block_scores(q, km, scale)
    assert np.allclose(r["L"], math.log(R) + scale * km @ q[0], atol=1e-12)


def test_scores_large_logits_stay_finite():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((32, 8)) * 400
    km = rng.standard_normal((5, 8)) * 400
    r = block_scores(q, km, 1.0)
    assert np.isfinite(r["L"]).all() and np.isfinite(r["Shat"]).all()
    assert r["Shat"].max() == 1.0 and (r["Shat"] >= 0).all()


# -------------------------------------------------------------- selection ---

def _rows(seed=5, n=40):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(I + 1) * 3 for I in range(n)]


def test_forced_blocks_sinks_and_local():
    f = forced_blocks(10, 256, 512, 128)
    assert list(np.nonzero(f)[0]) == [0, 1, 7, 8, 9, 10]
    # the diagonal block is always forced, even with no local window
    assert list(np.nonzero(forced_blocks(5, 0, 0, 128))[0]) == [5]
    assert list(np.nonzero(forced_blocks(5, 129, 1, 128))[0]) == [0, 1, 5]


def test_alpha_zero_keeps_every_block():
    for I, L in enumerate(_rows()):
        kept, _ = select_row(L, I, 0.0, 256, 512, 128)
        assert list(kept) == list(range(I + 1))


def test_alpha_above_one_keeps_forced_only():
    for I, L in enumerate(_rows()):
        kept, _ = select_row(L, I, 1.5, 256, 512, 128)
        assert list(kept) == list(np.nonzero(forced_blocks(I, 256, 512, 128))[0])


def test_selection_nested_in_alpha_and_contains_argmax():
    alphas = [0.9, 0.2, 0.1, 0.05, 0.025, 0.0125, 1e-6]
    for I, L in enumerate(_rows(6)):
        prev = None
        for a in alphas:
            kept, _ = select_row(L, I, a, 256, 512, 128)
            s = set(kept)
            assert int(np.argmax(L)) in s
            assert len(kept) <= I + 1 and list(kept) == sorted(kept)
            if prev is not None:
                assert prev <= s
            prev = s


def test_selection_invariant_to_row_shift():
    """A positive per-row factor on every score (an additive shift of L)
    leaves the selection unchanged."""
    for I, L in enumerate(_rows(7)):
        k1, _ = select_row(L, I, 0.1, 256, 512, 128)
        k2, _ = select_row(L + 17.25, I, 0.1, 256, 512, 128)
        assert np.array_equal(k1, k2)


def test_threshold_tie_and_band_flags():
    """Scores placed exactly at alpha, and just inside/outside the 1e-5
    relative band around it (I = 20, no forced block among J = 3..12)."""
    alpha = 0.1
    I = 20
    L = np.full(I + 1, -50.0)
    L[3] = 0.0                                   # top block
    L[5] = math.log(alpha)                       # exactly at the threshold -> kept
    L[6] = math.log(alpha * (1 + 0.5e-5))        # in band, above
    L[7] = math.log(alpha * (1 - 0.5e-5))        # in band, below -> dropped
    L[8] = math.log(alpha * (1 + 3e-5))          # outside band, kept
    L[9] = math.log(alpha * (1 - 3e-5))          # outside band, dropped
    kept, band = select_row(L, I, alpha, 0, 128, 128)
    assert 3 in kept and 5 in kept and 6 in kept and 8 in kept
    assert 7 not in kept and 9 not in kept
    assert band[5] and band[6] and band[7]
    assert not band[8] and not band[9] and not band[3]


def test_pipeline_rows_are_nonempty_and_bounded():
    w = make_workload(custom_spec((700, 129), 8, 2, seed=11, page_size=16))
    res = run_pipeline(OracleProblem.from_workload(w), 0.1, attend=False)
    for (h, s, I), r in res.items():
        kept = list(r["kept"])
        assert I in kept and 1 <= len(kept) <= I + 1
        assert all(J in kept for J in range(min(2, I + 1)))
        assert 0.0 < r["Shat"].min() or r["Shat"].min() == 0.0
        assert np.isclose(r["Shat"].max(), 1.0)
