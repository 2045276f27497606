"""The exact-ranking check used by the GPU ranked-selection parity test
(gpu_parity_util.check_ranked_row), exercised on the CPU: selections made
from scores perturbed within their error bounds pass, and planted mistakes
(a far-apart swap, a top-p prefix that runs past the mass, a dropped forced
block) fail."""
import numpy as np
import pytest

from gpu_parity_util import check_ranked_row
from oracle import forced_blocks, select_row_topk, select_row_topp

I = 60  # 61 causal blocks; sinks 256 and local 512 force blocks 0, 1, 56..60


def _row(seed, spread=3.0):
    rng = np.random.default_rng(seed)
    Lx = rng.normal(size=I + 1) * spread
    err = np.full(I + 1, 0.05)
    Lf = Lx + rng.uniform(-1, 1, size=I + 1) * err
    return Lx, Lf, err


@pytest.mark.parametrize("k", [0, 3, 10, 1000])
def test_topk_from_perturbed_scores_passes(k):
    for seed in range(20):
        Lx, Lf, err = _row(seed, spread=0.05 if seed % 2 else 3.0)  # odd seeds: many near ties
        got = set(select_row_topk(Lf, I, k, 256, 512, 128).tolist())
        n = check_ranked_row("topk", k, I, got, Lf, Lx, err)
        assert n >= 0


@pytest.mark.parametrize("p", [0.0, 0.3, 0.8, 0.99])
def test_topp_from_perturbed_scores_passes(p):
    for seed in range(20):
        Lx, Lf, err = _row(100 + seed, spread=0.05 if seed % 2 else 3.0)
        got = set(select_row_topp(Lf, I, p, 256, 512, 128).tolist())
        check_ranked_row("topp", p, I, got, Lf, Lx, err)


def test_far_apart_swap_fails():
    Lx, Lf, err = _row(7)
    got = set(select_row_topk(Lf, I, 5, 256, 512, 128).tolist())
    forced = forced_blocks(I, 256, 512, 128)
    free = [J for J in np.argsort(Lx) if not forced[J]]
    lowest, kept_best = int(free[0]), max((J for J in got if not forced[J]), key=lambda J: Lx[J])
    assert Lx[kept_best] - Lx[lowest] > 1.0
    bad = (got - {kept_best}) | {lowest}
    with pytest.raises(AssertionError):
        check_ranked_row("topk", 5, I, bad, Lf, Lx, err)


def test_topp_prefix_past_the_mass_fails():
    Lx, Lf, err = _row(11)
    p = 0.5
    got = set(select_row_topp(Lf, I, p, 256, 512, 128).tolist())
    order = [J for J in np.argsort(-Lf, kind="stable")]
    extra = [J for J in order if J not in got][:6]  # six more blocks than the mass needs
    with pytest.raises(AssertionError):
        check_ranked_row("topp", p, I, got | set(extra), Lf, Lx, err)


def test_topp_zero_keeps_forced_only():
    Lx, Lf, err = _row(3)
    forced = set(np.nonzero(forced_blocks(I, 256, 512, 128))[0].tolist())
    assert check_ranked_row("topp", 0.0, I, forced, Lf, Lx, err) == 0
    with pytest.raises(AssertionError):
        check_ranked_row("topp", 0.0, I, forced | {10}, Lf, Lx, err)
