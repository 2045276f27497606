"""Shared helpers of the GPU parity tests: run the HIP pipeline on a seeded
workload and compare it with the fp64 oracle on the same inputs."""

from __future__ import annotations

import sys
import time

import numpy as np

from oracle import BAND_REL, OracleProblem, pooled_all, run_pipeline

# Output tolerances (max-abs vs the fp64 oracle fed the GPU's own lists).
TOL_OUT = {"bf16": 2e-2, "f32": 2e-2, "e4m3": 6e-2}
# log-sum-exp: the correction pseudo-keys use the pooled keys rounded to
# bf16 (relative error <= 2^-9 per element), which moves each pseudo-key
# logit by at most softmax_scale * sum_i |q_i| |dkbar_i|; on these inputs
# (|q|, |kbar| ~ 17) that is a few 1e-2 in the worst case, and the lse moves
# by at most the largest such shift.
TOL_LSE = 5e-2
# pooled block scores (natural-log units): the fast path rounds
# softmax_scale log2(e) kbar to bf16 and accumulates the exact bf16 products
# in fp32 (log2-domain logits).  Per score row the error is bounded by
# score_bound() below (rounding + accumulation); the fp32 statistics (exp2,
# sums, log) add less than TOL_SCORE_STATS.
TOL_SCORE_STATS = 1e-3
# pooled means: float64 sums of the stored values and one division, on both
# sides (relative to max(1, |mean|))
TOL_POOL = 1e-12
# fp32 accumulation allowance of a 128-term dot product of exact products
ACCUM_REL = 2.0 ** -15
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def bf16_round64(x):
    """float64 -> nearest bfloat16 (ties to even), as float64: the grid
    spacing in the binade of |x| is 2^(e-7); dividing by it is exact and
    numpy's rint rounds half to even.  (Finite values in the bf16 range.)"""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    quantum = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(a / quantum) * quantum
    return np.where(a == 0, v, np.copysign(r, v))


def score_bound(prob, k_mean, h, s, I):
    """Bound on |fast - exact| block score of row (h, s, I), derived from the
    fast path's arithmetic: with c = scale log2(e) and s_J = bf16(c kbar_J),
    the log2-domain logit q_r . s_J is off c q_r . kbar_J by at most
    |q_r| |c kbar_J - s_J| (Cauchy-Schwarz) plus |q_r| ACCUM_REL |s_J| (fp32
    accumulation of 128 exact products); a log-sum-exp over rows moves by at
    most the largest shift, ln 2 of it in natural-log units.  k_mean: float64
    pooled keys (the library's, checked against the oracle's separately, or
    the oracle's own)."""
    B = prob.block_size
    nI = min(B, prob.seqlen(s) - I * B)
    qg = prob.queries(s, prob.list_heads(h), I * B + np.arange(nI)).reshape(-1, prob.d)
    qn = float(np.sqrt((qg * qg).sum(1)).max())
    kb0 = int(prob.block_offsets()[s])
    km = k_mean[prob.list_kv_head(h), kb0:kb0 + I + 1].astype(np.float64) * (prob.scale * LOG2E)
    hi = bf16_round64(km)
    res = np.sqrt(((km - hi) ** 2).sum(1)) + ACCUM_REL * np.sqrt((hi * hi).sum(1))
    return LN2 * qn * float(res.max())


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, alpha, sinks=256, local=512, correction=True, attn_splits=0, head_lists=False,
            softmax_scale=0.0):
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    db = upload(w, "cuda")
    pipe = Pipeline(db, softmax_scale=softmax_scale, attn_splits=attn_splits, head_lists=head_lists)
    pipe.run(alpha, sinks, local, correction)
    torch.cuda.synchronize()
    rp, ci = pipe.csr()
    res = {
        "k_mean": pipe.k_mean.cpu().numpy(),
        "v_mean": pipe.v_mean.cpu().numpy(),
        "scores": pipe.scores.cpu().numpy(),
        "scores_err": pipe.scores_err.cpu().numpy(),
        "row_ptr": rp,
        "col_idx": ci,
        "out": pipe.out.float().cpu().numpy(),
        "lse": pipe.lse.cpu().numpy(),
        "pipe": pipe,
    }
    return res


def compare(w, g, alpha, sinks=256, local=512, correction=True, rows=None,
            check_pool=True, head_lists=False, softmax_scale=0.0):
    """Compare GPU results `g` with the oracle on `rows` ((owner, s, I)
    triples; default all; the owner is the KV head, or the query head with
    head_lists).  softmax_scale: the one the library was given (0: 1/sqrt(d);
    the oracle takes the library's float32 value).  Returns a stats dict;
    raises AssertionError on failure."""
    prob = OracleProblem.from_workload(w)
    prob.head_lists = head_lists
    if softmax_scale > 0:
        prob.softmax_scale = float(np.float32(softmax_scale))
    spec = w.spec
    qoff = prob.query_block_offsets()
    t0 = time.time()
    if check_pool:
        km, vm, _ = pooled_all(prob)
        for name, ref in (("k_mean", km), ("v_mean", vm)):
            err = np.abs(g[name] - ref)
            assert np.all(err <= TOL_POOL * np.maximum(1.0, np.abs(ref))), \
                f"{name}: max err {err.max():.3g}"
    res = run_pipeline(prob, alpha, sinks, local, correction, rows=rows,
                       given_csr=(g["row_ptr"], g["col_idx"]))
    rp, ci = g["row_ptr"], g["col_idx"]
    # every output and lse of the batch must be finite (max() below would
    # silently skip NaN)
    assert np.all(np.isfinite(g["out"])), "non-finite output"
    assert np.all(np.isfinite(g["lse"])), "non-finite lse"
    stats = dict(rows=len(res), band=0, mismatch=0, score_err=0.0, out_err=0.0, lse_err=0.0)
    for (h, s, I), r in res.items():
        heads = prob.list_heads(h)
        row = prob.row_index(h, s, I)
        i0 = prob.ctx(s) // spec.block_size
        # pooled scores (fast path)
        Lg = g["scores"][h, int(qoff[s]) + I - i0, :I + 1].astype(np.float64)
        serr = float(np.max(np.abs(Lg - r["L"])))
        stats["score_err"] = max(stats["score_err"], serr)
        bnd = score_bound(prob, g["k_mean"], h, s, I)
        assert serr <= bnd + TOL_SCORE_STATS, f"row {(h, s, I)}: score err {serr:.3g} > bound {bnd:.3g}"
        # the bound the library reports for the row (used by its selection)
        rep = float(g["scores_err"][h, int(qoff[s]) + I - i0])
        assert bnd * (1 - 1e-5) <= rep <= bnd * 1.01 + 1e-12, (h, s, I, rep, bnd)
        stats["score_bound"] = max(stats.get("score_bound", 0.0), bnd)
        # CSR: exact outside the band
        got = set(int(x) for x in ci[rp[row]:rp[row + 1]])
        want = set(int(x) for x in r["kept"])
        band = set(int(x) for x in np.nonzero(r["band"])[0])
        stats["band"] += len(band)
        diff = (got ^ want) - band
        stats["mismatch"] += len(diff)
        assert list(ci[rp[row]:rp[row + 1]]) == sorted(got), f"row {(h, s, I)} not ascending"
        # outputs
        cu0 = int(w.cu_seqlens[s])
        nI = r["out"].shape[1]
        toks = cu0 + I * spec.block_size - prob.ctx(s) + np.arange(nI)
        og = g["out"][toks][:, heads, :].transpose(1, 0, 2)
        stats["out_err"] = max(stats["out_err"], float(np.max(np.abs(og - r["out"]))))
        lg = g["lse"][heads][:, toks]
        stats["lse_err"] = max(stats["lse_err"], float(np.max(np.abs(lg - r["lse"]))))
    stats["oracle_s"] = time.time() - t0
    log(f"  parity {spec.name}: {stats}")
    assert stats["mismatch"] == 0, stats
    assert stats["out_err"] <= TOL_OUT[spec.qk_dtype], stats
    assert stats["lse_err"] <= TOL_LSE, stats
    return stats


def oracle_scores_all_rows(w, head_lists=False, threads=16):
    """The oracle's block scores L of every (owner, s, I) row of the
    workload (float64), computed once per workload and shared by every
    alpha (the scores do not depend on it).  List owners run in parallel
    threads (numpy releases the GIL in its products and exponentials)."""
    from concurrent.futures import ThreadPoolExecutor
    prob = OracleProblem.from_workload(w)
    prob.head_lists = head_lists
    owners = list(range(prob.list_owners))

    def one(h):
        rows = [(h, s, I) for s in range(prob.num_seqs) for I in prob.query_blocks(s)]
        res = run_pipeline(prob, 1.0, rows=rows, attend=False)
        return {k: r["L"] for k, r in res.items()}

    t0 = time.time()
    out = {}
    with ThreadPoolExecutor(min(threads, len(owners))) as ex:
        for part in ex.map(one, owners):
            out.update(part)
    log(f"  oracle scores of {len(out)} rows in {time.time() - t0:.1f} s")
    return prob, out


def compare_lists_all_rows(prob, scores, rp, ci, alpha, sinks=256, local=512):
    """Every row's GPU list against the oracle's selection from its float64
    scores: identical outside the oracle's 1e-5 band at the threshold.
    Returns (rows, in-band entries, mismatches); raises on a mismatch."""
    from oracle import select_row
    band = mism = 0
    bad = []
    B = prob.block_size
    for (h, s, I), L in scores.items():
        kept, bflag = select_row(L, I, alpha, sinks, local, B)
        row = prob.row_index(h, s, I)
        got = ci[rp[row]:rp[row + 1]]
        if np.any(np.diff(got) <= 0):
            bad.append(("order", h, s, I))
        fl = set(np.nonzero(bflag)[0].tolist())
        band += len(fl)
        d = (set(got.tolist()) ^ set(kept.tolist())) - fl
        if d:
            mism += len(d)
            bad.append((h, s, I, sorted(d)[:4]))
    log(f"  lists alpha={alpha}: {len(scores)} rows, {band} in band, {mism} mismatches")
    assert not bad, bad[:8]
    return len(scores), band, mism


def check_ranked_row(mode, param, I, got, L_fast, L_exact, err, sinks=256, local=512, B=128):
    """One row of a ranked selection (top-k / top-p with parameter param)
    made from the fast scores L_fast, against the exact scores L_exact: a
    decision may differ from the exact selection only between blocks whose
    exact scores are within their error bounds err (array over J <= I) of
    each other, and for top-p the exact mass share of the prefix taken stays
    within the ratio those errors allow.  Returns the number of decisions
    that differ from the exact selection; raises AssertionError otherwise."""
    from oracle import forced_blocks, rank_order, select_row_topk, select_row_topp
    Lx = np.asarray(L_exact, dtype=np.float64)[:I + 1]
    forced = forced_blocks(I, sinks, local, B)
    if mode == "topk":
        ndiff = len(got ^ set(select_row_topk(Lx, I, param, sinks, local, B).tolist()))
    else:
        if param <= 0:
            assert got == set(np.nonzero(forced)[0].tolist()), ("forced only", I)
            return 0
        ndiff = len(got ^ set(select_row_topp(Lx, I, param, sinks, local, B).tolist()))
        # the prefix of the fast ranking ends between the last kept
        # non-forced block and the end of the kept run (forced blocks are kept
        # wherever they rank); some end in that range must meet the top-p
        # condition under the exact scores, up to the slack
        order = rank_order(np.asarray(L_fast, dtype=np.float64)[:I + 1], I)
        m_max = int(np.cumprod([J in got for J in order]).sum()) - 1
        m_min = max([i for i, J in enumerate(order) if J in got and not forced[J]] + [0])
        wx = np.exp(Lx - Lx.max())
        share = np.cumsum(wx[order]) / wx.sum()
        slack = float(np.expm1(2 * float(np.max(err)))) + 1e-4
        ok = [m for m in range(m_min, m_max + 1)
              if share[m] >= param * (1 - slack) and (m == 0 or share[m - 1] < param * (1 + slack))]
        assert ok, ("top-p mass", I, m_min, m_max, share[m_min:m_max + 1])
    # every kept non-forced block ranks no lower than any dropped one, up to
    # the bounds
    ins = [J for J in got if not forced[J]]
    outs = [J for J in range(I + 1) if J not in got]
    if ins and outs:
        lo = min(Lx[J] + err[J] for J in ins)
        hi = max(Lx[J] - err[J] for J in outs)
        assert lo >= hi, ("ranking", I, lo, hi)
    return ndiff


def sample_rows(w, n_per_head, seed=0, head_lists=False):
    """Seeded sample of (owner, s, I) rows, always including each sequence's
    first and last query block."""
    rng = np.random.default_rng(seed)
    prob = OracleProblem.from_workload(w)
    prob.head_lists = head_lists
    rows = []
    for s in range(prob.num_seqs):
        qb = list(prob.query_blocks(s))
        if not qb:
            continue
        for h in range(prob.list_owners):
            pick = set([qb[0], qb[-1]])
            pick |= set(int(x) for x in rng.choice(qb, size=min(len(qb), n_per_head), replace=False))
            rows += [(h, s, I) for I in sorted(pick)]
    return rows
