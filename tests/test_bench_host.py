"""Host-side reporting arithmetic of bench.py (pair and block counts from the
CSR lists): per-query-head lists that repeat their group's list count the same
kept and correction pairs as the group lists; the all-blocks CSR counts every
causal pair."""

import numpy as np

import bench
from synthetic import custom_spec


def _group_csr(spec, rng, full=False):
    B = spec.block_size
    rows = []
    for h in range(spec.num_kv_heads):
        for L in spec.seqlens:
            n = -(-L // B)
            for I in range(n):
                if full:
                    rows.append(np.arange(I + 1))
                else:
                    keep = rng.random(I + 1) < 0.4
                    keep[I] = True
                    rows.append(np.nonzero(keep)[0])
    return rows


def _csr(rows):
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    ci = np.concatenate(rows).astype(np.int64)
    return rp, ci


def test_head_lists_repeating_the_group_list_count_the_same_pairs():
    spec = custom_spec((700, 300, 129), 8, 2)
    rows = _group_csr(spec, np.random.default_rng(0))
    nrow = len(rows) // spec.num_kv_heads
    g = spec.group
    head_rows = []
    for hq in range(spec.num_q_heads):
        h = hq // g
        head_rows += rows[h * nrow:(h + 1) * nrow]
    kg, cg = bench.kept_pairs(*_csr(rows), spec)
    kh, ch = bench.kept_pairs(*_csr(head_rows), spec, head_lists=True)
    assert (kg, cg) == (kh, ch)


def test_full_lists_count_every_causal_pair():
    spec = custom_spec((700, 300, 129), 8, 2)
    kp, cp = bench.kept_pairs(*_csr(_group_csr(spec, None, full=True)), spec)
    assert cp == 0
    assert kp == bench.causal_pairs(spec.seqlens) * spec.num_q_heads
    rp, _ = _csr(_group_csr(spec, None, full=True))
    assert rp[-1] == bench.causal_blocks(spec.seqlens, spec.num_kv_heads)


def test_cpu_baseline_times_each_oracle_stage():
    """The oracle leg on a small prompt: every query block of the sample is
    run once through scores, selection and attention, each stage timed, and
    the rate counts the same kept pairs as the oracle's own selection."""
    from oracle import OracleProblem, run_pipeline
    from synthetic import make_workload, spec_for
    w = make_workload(spec_for("toy_2k"))
    r = bench.cpu_baseline(w, 0.1, True, budget_s=60.0)
    st = r["stages_s"]
    assert st["rows"] == 16 and r["kind"] == "oracle" and r["cores"] >= 1
    assert all(st[k] > 0 for k in ("decode_pool_sequence", "score", "select", "attend"))
    # the pairs behind the rate: the oracle pipeline's own lists
    prob = OracleProblem.from_workload(w)
    res = run_pipeline(prob, 0.1, attend=False)
    B, d, g = w.spec.block_size, w.spec.head_dim, w.spec.group
    flops = 0
    for (h, s, I), x in res.items():
        nI = min(B, w.spec.seqlens[s] - I * B)
        flops += 4 * d * g * (int(np.sum(np.asarray(x["kept"]) < I)) * B * nI + nI * (nI + 1) // 2)
    secs = st["score"] + st["select"] + st["attend"]
    assert 0.5 < flops / 1e12 / r["value"] / secs < 1.5


def test_recheck_counts_follow_the_selection_guard():
    """The bench's recount of the float64 re-check work: a row is re-checked
    only when a non-forced entry lies within its guard of the threshold
    (sink and window blocks and entries past the diagonal never count), and
    then its threshold and maximum candidates are evaluated in passes of 8
    keys.  Sinks: J < 2; window: I - J < 4."""
    nq = 20
    seqlens = (128 * nq,)
    L = np.full((1, nq, nq), np.nan, np.float32)  # entries past the diagonal: garbage
    for I in range(nq):
        L[0, I, :I + 1] = -10.0
        L[0, I, 0] = 0.0  # the row maximum, on a sink block
    E = np.full((1, nq), 0.01, np.float32)
    thr = np.log(0.1)
    L[0, 9, 3] = thr + 0.002    # within 2E + stat of the threshold, not forced
    L[0, 8, 7] = thr            # in the window: forced, not a candidate
    L[0, 7, 1:7] = thr - 0.001  # J = 1 (sink) and 4..6 (window) forced; J = 2, 3 candidates
    L[0, 6, 2] = thr + 0.5      # far outside the guard
    L[0, 19, 1:20] = thr        # J = 2..15 candidates (14), the rest forced
    got = bench.recheck_counts(L, E, seqlens, 0.1)
    assert got["rows"] == nq
    assert got["rows_rechecked"] == 3
    # each re-checked row also evaluates its maximum (J = 0)
    assert got["evaluations"] == (1 + 1) + (2 + 1) + (14 + 1)
    assert got["passes"] == 1 + 1 + 2
    # a second list owner with no entry near its threshold adds nothing
    L2 = np.concatenate([L, np.where(np.isnan(L), np.nan, -10.0).astype(np.float32)])
    L2[1, :, 0] = 0.0
    got2 = bench.recheck_counts(L2, np.concatenate([E, E]), seqlens, 0.1)
    assert got2["rows"] == 2 * nq
    assert {k: got2[k] for k in ("rows_rechecked", "evaluations", "passes")} == \
        {k: got[k] for k in ("rows_rechecked", "evaluations", "passes")}
