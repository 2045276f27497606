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
