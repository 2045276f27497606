"""Top-k / top-p selection in the oracle ([V1] 二 and 4.4: the prior
methods' selection strategies that the max-based threshold is compared with;
reading R21).  Pins: reductions to the threshold path (all blocks, forced
blocks only, the threshold at the k-th score), nesting, shift invariance and
the defining extremal properties checked element by element."""

import numpy as np
import pytest

from oracle import forced_blocks, rank_order, select_row, select_row_topk, select_row_topp

B = 128


def rows(seed=0, n=12):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        I = int(rng.integers(0, 300))
        L = rng.normal(0, 3, size=I + 1) + rng.normal(0, 0.01)
        yield I, L


@pytest.mark.parametrize("seed", [0, 1])
def test_topk_extremes_reduce_to_threshold_path(seed):
    for I, L in rows(seed):
        allk = select_row_topk(L, I, I + 1, 256, 512, B)
        assert np.array_equal(allk, select_row(L, I, 0.0, 256, 512, B)[0])
        none = select_row_topk(L, I, 0, 256, 512, B)
        assert np.array_equal(none, select_row(L, I, 1.5, 256, 512, B)[0])


def test_topk_is_threshold_at_kth_score():
    """Distinct scores: top-k equals the max-based threshold with alpha set
    to the normalised score of the k-th ranked non-forced block."""
    for I, L in rows(2):
        forced = forced_blocks(I, 256, 512, B)
        ranked = [J for J in rank_order(L, I) if not forced[J]]
        for k in (1, 3, 10):
            if k > len(ranked):
                continue
            alpha = float(np.exp(L[ranked[k - 1]] - L.max()))
            want = select_row(L, I, alpha, 256, 512, B)[0]
            assert np.array_equal(select_row_topk(L, I, k, 256, 512, B), want)


def test_topk_extremal_and_nested():
    for I, L in rows(3):
        forced = forced_blocks(I, 256, 512, B)
        nonforced = int((~forced).sum())
        prev = None
        for k in range(0, min(I + 2, 20)):
            kept = select_row_topk(L, I, k, 256, 512, B)
            ks = set(kept.tolist())
            assert len(kept) == int(forced.sum()) + min(k, nonforced)
            assert set(np.nonzero(forced)[0].tolist()) <= ks
            picked = [J for J in ks if not forced[J]]
            dropped = [J for J in range(I + 1) if not forced[J] and J not in ks]
            for a in picked:       # every picked block outranks every dropped one
                for b in dropped:
                    assert (L[a], -a) > (L[b], -b)
            if prev is not None:
                assert prev <= ks
            prev = ks


def test_topp_minimal_prefix_and_extremes():
    for I, L in rows(4):
        forced = forced_blocks(I, 256, 512, B)
        order = rank_order(L, I)
        w = np.exp(L[order] - L.max())
        tot = w.sum()
        assert np.array_equal(select_row_topp(L, I, 0.0, 256, 512, B),
                              np.nonzero(forced)[0])
        assert np.array_equal(select_row_topp(L, I, 1.0, 256, 512, B), np.arange(I + 1))
        prev = set()
        for p in (0.1, 0.5, 0.9, 0.99):
            ks = set(select_row_topp(L, I, p, 256, 512, B).tolist())
            # the shortest ranked prefix whose mass reaches p (found by a
            # plain scan), plus the forced blocks
            n = next(m for m in range(1, I + 2) if w[:m].sum() >= p * tot)
            assert w[:n - 1].sum() < p * tot
            assert ks == set(order[:n].tolist()) | set(np.nonzero(forced)[0].tolist())
            assert prev <= ks
            prev = ks


def test_ranked_selection_shift_invariant():
    for I, L in rows(5):
        for k in (2, 7):
            assert np.array_equal(select_row_topk(L, I, k, 256, 512, B),
                                  select_row_topk(L + 13.5, I, k, 256, 512, B))
        for p in (0.3, 0.8):
            assert np.array_equal(select_row_topp(L, I, p, 256, 512, B),
                                  select_row_topp(L + 13.5, I, p, 256, 512, B))


def test_ties_go_to_the_lower_block():
    L = np.zeros(20)
    assert list(select_row_topk(L, 19, 3, 0, 128, B)) == [0, 1, 2, 19]
    assert list(select_row_topp(L, 19, 0.1, 0, 128, B)) == [0, 1, 19]
