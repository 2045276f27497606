"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs.  Bars: pooled means within 1e-5 relative; selected block
lists identical outside the 1e-5 relative band at the threshold; outputs
within max-abs 2e-2 (bf16 / fp32 inputs) or 6e-2 (fp8 e4m3 Q/K)."""

import numpy as np
import pytest

from synthetic import chunk_view, custom_spec, make_workload, spec_for

from gpu_parity_util import (TOL_SCORE_STATS, check_ranked_row, compare, compare_lists_all_rows,
                             log, oracle_scores_all_rows, run_gpu, sample_rows, score_bound)

pytestmark = pytest.mark.gpu


SMALL_CASES = [
    # name, spec kwargs, alpha, sinks, local, correction
    ("bf16_ragged_g4_p16", dict(seqlens=(300, 129, 1, 1000), num_q_heads=8, num_kv_heads=2,
                                page_size=16, paging="permute", seed=101), 0.1, 256, 512, True),
    ("bf16_g8_p64", dict(seqlens=(1500, 640), num_q_heads=16, num_kv_heads=2, page_size=64,
                         paging="roundrobin", seed=102), 0.1, 256, 512, True),
    ("bf16_g8_nocorr", dict(seqlens=(1500,), num_q_heads=16, num_kv_heads=2, page_size=64,
                            seed=103), 0.1, 256, 512, False),
    ("bf16_alpha0_dense", dict(seqlens=(700, 257), num_q_heads=4, num_kv_heads=1, page_size=128,
                               seed=104), 0.0, 256, 512, True),
    ("bf16_alpha_gt1_forced_only", dict(seqlens=(1300,), num_q_heads=4, num_kv_heads=1,
                                        page_size=32, seed=105), 1.5, 256, 512, True),
    ("bf16_no_sinks_local128", dict(seqlens=(1200, 333), num_q_heads=8, num_kv_heads=4,
                                    page_size=256, seed=106), 0.05, 0, 128, True),
    ("bf16_g1", dict(seqlens=(900,), num_q_heads=2, num_kv_heads=2, page_size=64, seed=107),
     0.1, 256, 512, True),
    ("bf16_g16", dict(seqlens=(600,), num_q_heads=16, num_kv_heads=1, page_size=64, seed=108),
     0.1, 256, 512, True),
    ("bf16_g3_odd", dict(seqlens=(520,), num_q_heads=6, num_kv_heads=2, page_size=8, seed=109),
     0.1, 128, 256, True),
    ("e4m3_g2_rr", dict(seqlens=(700, 130), num_q_heads=8, num_kv_heads=4, qk_dtype="e4m3",
                        v_dtype="bf16", page_size=64, paging="roundrobin", seed=110),
     0.1, 256, 512, True),
    ("e4m3_g8_p16", dict(seqlens=(1100,), num_q_heads=8, num_kv_heads=1, qk_dtype="e4m3",
                         v_dtype="bf16", page_size=16, seed=111), 0.1, 256, 512, True),
    ("f32_out_f32", dict(seqlens=(640, 100), num_q_heads=4, num_kv_heads=1, qk_dtype="f32",
                         v_dtype="f32", out_dtype="f32", page_size=128, paging="identity",
                         seed=112), 0.1, 256, 512, True),
    ("bf16_out_f32", dict(seqlens=(400,), num_q_heads=4, num_kv_heads=2, out_dtype="f32",
                          page_size=16, seed=113), 0.1, 256, 512, True),
]


@pytest.mark.parametrize("splits", [1, 0], ids=["nosplit", "autosplit"])
@pytest.mark.parametrize("name,kw,alpha,sinks,local,corr", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_full_parity(name, kw, alpha, sinks, local, corr, splits):
    """Small ragged cases, with the attention unsplit and with the automatic
    KV split (these launches have far fewer workgroups than CUs, so every
    row is cut into several parts merged by the combine pass)."""
    log(f"case {name} splits={splits}")
    w = make_workload(custom_spec(name=name, **kw))
    g = run_gpu(w, alpha, sinks, local, corr, attn_splits=splits)
    compare(w, g, alpha, sinks, local, corr)


@pytest.mark.parametrize("qk", ["bf16", "e4m3"])
@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_softmax_scale_parity(scale, qk):
    """A softmax scale other than 1/sqrt(d): the discovery keys (pre-scaled
    by it), the exact re-check and the attention logits all follow it.  At
    0.3 the bf16 discovery's per-row logit bounds run from ~100 to ~190 log2
    units, on both sides of the 112 up to which the sums need no reference
    (both forms of the sums run); at 0.05 they stay below ~32."""
    log(f"case softmax_scale={scale} {qk}")
    kw = dict(seqlens=(1500, 640), num_q_heads=16, num_kv_heads=2, page_size=64,
              paging="roundrobin", seed=130)
    if qk == "e4m3":
        kw.update(qk_dtype="e4m3", v_dtype="bf16")
    w = make_workload(custom_spec(name=f"scale_{qk}_{scale}", **kw))
    g = run_gpu(w, 0.1, softmax_scale=scale)
    stats = compare(w, g, 0.1, softmax_scale=scale)
    log(f"  {stats}")


def test_toy_2k_config_full_parity():
    """2048-token single prompt, fp32 inputs, contiguous KV, g = 4."""
    log("case toy_2k")
    w = make_workload(spec_for("toy_2k"))
    g = run_gpu(w, 0.1)
    compare(w, g, 0.1)


def test_deterministic_rerun():
    w = make_workload(custom_spec((1500, 300), 16, 2, seed=120, page_size=16))
    a = run_gpu(w, 0.1)
    b = run_gpu(w, 0.1)
    for k in ("k_mean", "scores", "row_ptr", "col_idx", "out", "lse"):
        if k == "scores":
            continue  # entries J > I are unspecified
        assert np.array_equal(a[k], b[k]), k


def test_gqa_32k_config_parity():
    """32K prompt, Hq=32 / Hkv=4, paged (64) with a permuted page table:
    pooled means everywhere, every row's list against the oracle's, scores
    and outputs on sampled rows."""
    log("case gqa_32k")
    w = make_workload(spec_for("gqa_32k"))
    g = run_gpu(w, 0.1)
    prob, sc = oracle_scores_all_rows(w)
    compare_lists_all_rows(prob, sc, g["row_ptr"], g["col_idx"], 0.1)
    compare(w, g, 0.1, rows=sample_rows(w, 6), check_pool=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,nrows", [("varlen_4x", 3), ("long_256k", 3)])
def test_full_size_config_parity(name, nrows):
    """Benchmark-size configs at alpha = 0.1 with correction (the bench launch
    configuration): pooled means everywhere; every row's list against the
    oracle's selection from its float64 scores (in-band and mismatch counts
    logged); scores and outputs on a seeded sample of rows per KV head and
    sequence (first and last block of every sequence included)."""
    log(f"case {name}")
    w = make_workload(spec_for(name))
    g = run_gpu(w, 0.1)
    prob, sc = oracle_scores_all_rows(w)
    compare_lists_all_rows(prob, sc, g["row_ptr"], g["col_idx"], 0.1)
    compare(w, g, 0.1, rows=sample_rows(w, nrows), check_pool=True)


@pytest.mark.timeout(1200)
def test_sweep_128k_alpha_correction_grid():
    """The 128K sweep: alpha in {0.2, 0.1, 0.05, 0.025, 0.0125}, each with
    and without mean correction, in the bench launch configuration (one
    discovery, then selection + attention per point).  Per point: every
    row's list against the oracle's (scores computed once), outputs and lse
    on sampled rows against the oracle fed the GPU's lists; pooled means
    everywhere once."""
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    from synthetic import ALPHA_SWEEP
    log("case sweep_128k grid")
    w = make_workload(spec_for("sweep_128k"))
    pipe = Pipeline(upload(w, "cuda"))
    pipe.discover()
    torch.cuda.synchronize()
    prob, sc = oracle_scores_all_rows(w)
    rows = sample_rows(w, 2)
    first = True
    for alpha in ALPHA_SWEEP:
        for corr in (True, False):
            log(f"  point alpha={alpha} correction={corr}")
            pipe.select(alpha)
            pipe.attend(corr)
            torch.cuda.synchronize()
            rp, ci = pipe.csr()
            if corr:  # the lists do not depend on the correction
                compare_lists_all_rows(prob, sc, rp, ci, alpha)
            g = {"k_mean": pipe.k_mean.cpu().numpy(), "v_mean": pipe.v_mean.cpu().numpy(),
                 "scores": pipe.scores.cpu().numpy(), "scores_err": pipe.scores_err.cpu().numpy(),
                 "row_ptr": rp, "col_idx": ci, "out": pipe.out.float().cpu().numpy(),
                 "lse": pipe.lse.cpu().numpy()}
            compare(w, g, alpha, correction=corr, rows=rows, check_pool=first)
            first = False


def test_empty_sequences_in_batch():
    """Zero-length sequences between and around real ones (cu_seqlens with
    repeated offsets): they own no blocks, no lists and no output rows."""
    log("case empty_mix")
    w = make_workload(custom_spec(name="empty_mix", seqlens=(0, 300, 0, 129, 0), num_q_heads=4,
                                  num_kv_heads=2, page_size=16, paging="roundrobin", seed=130))
    g = run_gpu(w, 0.1)
    compare(w, g, 0.1)


def test_max_blocks_per_sequence():
    """One sequence at the 8192-block limit (1,048,576 tokens; Hq=2 / Hkv=1,
    pages of 128, permuted): the per-sequence LDS structures of discovery,
    selection and attention at full size.  Pooled means everywhere; lists,
    scores and outputs on sampled rows; structure of every list."""
    log("case max_blocks_1m")
    w = make_workload(custom_spec(name="max_blocks_1m", seqlens=(8192 * 128,), num_q_heads=2,
                                  num_kv_heads=1, page_size=128, paging="permute", seed=131))
    g = run_gpu(w, 0.1)
    compare(w, g, 0.1, rows=sample_rows(w, 4), check_pool=True)
    rp, ci = g["row_ptr"], g["col_idx"]
    assert rp.shape[0] == 8192 + 1
    for I in range(8192):
        lst = ci[rp[I]:rp[I + 1]]
        assert lst[-1] == I and np.all(np.diff(lst) > 0) and lst[0] >= 0
        assert set(range(min(2, I + 1))) <= set(lst.tolist())
        assert set(range(max(0, I - 3), I + 1)) <= set(lst.tolist())


CHUNK_CASES = [
    # name, spec kwargs, cached prefix per sequence
    ("chunk_bf16_mixed", dict(seqlens=(700, 300, 1000), num_q_heads=8, num_kv_heads=2,
                              page_size=16, paging="permute", seed=140), (256, 0, 896)),
    ("chunk_e4m3_tail", dict(seqlens=(1300, 500), num_q_heads=8, num_kv_heads=1, qk_dtype="e4m3",
                             v_dtype="bf16", page_size=64, paging="roundrobin", seed=141), (1280, 384)),
    ("chunk_prefix_only", dict(seqlens=(640, 257), num_q_heads=4, num_kv_heads=4, page_size=256,
                               seed=142), (640, 128)),
]


@pytest.mark.parametrize("name,kw,ctx", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunked_prefill_parity(name, kw, ctx):
    """Chunked prefill: the query tokens follow a cached prefix of each
    sequence (a sequence may have no query tokens left)."""
    log(f"case {name}")
    w = chunk_view(make_workload(custom_spec(name=name, **kw)), ctx)
    g = run_gpu(w, 0.1)
    compare(w, g, 0.1)


def _chunk_vs_whole(w, ctx, alpha=0.1):
    """GPU rows of the chunk must be bit-identical to the same rows of the
    whole prompt: pooled means, scores, lists, outputs and lse.  The
    attention runs unsplit on both sides (attn_splits = 1: a row's result
    then does not depend on the size of the launch)."""
    from oracle import OracleProblem
    wc = chunk_view(w, ctx)
    gf = run_gpu(w, alpha, attn_splits=1)
    gc = run_gpu(wc, alpha, attn_splits=1)
    pf, pc = OracleProblem.from_workload(w), OracleProblem.from_workload(wc)
    assert np.array_equal(gf["k_mean"], gc["k_mean"]) and np.array_equal(gf["v_mean"], gc["v_mean"])
    G = w.spec.group
    for s in range(pc.num_seqs):
        i0 = ctx[s] // 128
        qf, qc = pf.query_block_offsets(), pc.query_block_offsets()
        for h in range(pc.hkv):
            for I in pc.query_blocks(s):
                a = gf["scores"][h, int(qf[s]) + I, :I + 1]
                b = gc["scores"][h, int(qc[s]) + I - i0, :I + 1]
                assert np.array_equal(a, b), (s, h, I)
                rf, rc = pf.row_index(h, s, I), pc.row_index(h, s, I)
                assert np.array_equal(gf["col_idx"][gf["row_ptr"][rf]:gf["row_ptr"][rf + 1]],
                                      gc["col_idx"][gc["row_ptr"][rc]:gc["row_ptr"][rc + 1]]), (s, h, I)
        tf = np.arange(int(w.cu_seqlens[s]) + ctx[s], int(w.cu_seqlens[s + 1]))
        tc = np.arange(int(wc.cu_seqlens[s]), int(wc.cu_seqlens[s + 1]))
        assert np.array_equal(gf["out"][tf], gc["out"][tc]), s
        assert np.array_equal(gf["lse"][:, tf], gc["lse"][:, tc]), s
    return wc, gc


def test_chunked_prefill_matches_whole_prompt():
    log("case chunk_vs_whole_small")
    w = make_workload(custom_spec(name="chunk_whole", seqlens=(1500, 900, 300), num_q_heads=16,
                                  num_kv_heads=2, page_size=64, paging="permute", seed=143))
    _chunk_vs_whole(w, (1024, 512, 0))


def test_chunked_prefill_128k_last_16k():
    """The last 16K tokens of the 128K prompt as one chunk (the launch
    configuration of the chunked benchmark line): bit-identical to the whole
    prompt's rows; oracle parity on sampled rows of the chunk."""
    log("case chunk_128k_last16k")
    w = make_workload(spec_for("sweep_128k"))
    wc, gc = _chunk_vs_whole(w, (131072 - 16384,))
    compare(wc, gc, 0.1, rows=sample_rows(wc, 4), check_pool=False)


def test_chunked_prefill_varlen_last_8k():
    """The varlen e4m3 batch (16-token pages, round-robin) with the last 8K
    tokens of every sequence as one chunk each (the 8K sequence entirely):
    bit-identical to the whole batch's rows."""
    log("case chunk_varlen_last8k")
    w = make_workload(spec_for("varlen_4x"))
    lens = np.diff(np.asarray(w.cu_seqlens))
    _chunk_vs_whole(w, tuple(int(n) - 8192 for n in lens))


@pytest.mark.parametrize("splits", [2, 3, 8])
def test_forced_kv_split_gqa_32k(splits):
    """32K prompt with every row forced into 2, 3 or 8 parts (parts may be
    empty for short rows): sampled rows against the oracle, and every output
    within rounding of the unsplit result."""
    log(f"case gqa_32k splits={splits}")
    w = make_workload(spec_for("gqa_32k"))
    g1 = run_gpu(w, 0.1, attn_splits=1)
    gs = run_gpu(w, 0.1, attn_splits=splits)
    assert np.array_equal(g1["col_idx"], gs["col_idx"])
    dout = np.abs(g1["out"] - gs["out"])
    dlse = float(np.max(np.abs(g1["lse"] - gs["lse"])))
    log(f"  split vs unsplit: out {float(dout.max()):.3g} lse {dlse:.3g}")
    # each part exponentiates against its own running max, so the bf16
    # probabilities fed to P.V round differently (relative 2^-9 per term);
    # the log-sum-exp, formed in fp32, agrees to rounding
    assert np.all(dout <= 2.0 ** -5 * np.maximum(1.0, np.abs(g1["out"])))
    assert dlse <= 1e-4
    compare(w, gs, 0.1, rows=sample_rows(w, 3), check_pool=False)


def test_small_chunk_auto_split():
    """A 256-token chunk after an 8K prefix (few rows: the automatic split
    cuts each row into 8 parts) against the oracle."""
    log("case chunk_256_after_8k")
    w = chunk_view(make_workload(custom_spec(name="small_chunk", seqlens=(8448,), num_q_heads=8,
                                             num_kv_heads=2, page_size=64, seed=150)), (8192,))
    g = run_gpu(w, 0.1)
    compare(w, g, 0.1)


RANKED = [("topk", 0), ("topk", 3), ("topk", 100000), ("topp", 0.0), ("topp", 0.5), ("topp", 0.95)]


@pytest.mark.parametrize("mode,param", RANKED, ids=[f"{m}_{p}" for m, p in RANKED])
def test_ranked_selection_parity(mode, param):
    """Top-k / top-p selection on the GPU's scores: the lists equal the
    oracle's ranking of the same fp32 scores (top-p: up to the fp32 rounding
    of the running sum at the cut), and attention over them matches the
    oracle."""
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    from oracle import OracleProblem, forced_blocks, rank_order, run_pipeline, select_row_topk
    log(f"case ranked {mode} {param}")
    w = make_workload(custom_spec(name="ranked", seqlens=(1500, 640, 129), num_q_heads=8,
                                  num_kv_heads=2, page_size=16, paging="permute", seed=160))
    pipe = Pipeline(upload(w, "cuda"))
    pipe.discover()
    if mode == "topk":
        pipe.select_topk(param)
    else:
        pipe.select_topp(param)
    pipe.attend()
    torch.cuda.synchronize()
    rp, ci = pipe.csr()
    scores = pipe.scores.cpu().numpy().astype(np.float64)
    out = pipe.out.float().cpu().numpy()
    lse = pipe.lse.cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    prob = OracleProblem.from_workload(w)
    qoff = prob.query_block_offsets()
    for h in range(prob.hkv):
        for s_ in range(prob.num_seqs):
            for I in prob.query_blocks(s_):
                row = prob.row_index(h, s_, I)
                got = set(ci[rp[row]:rp[row + 1]].tolist())
                L = scores[h, int(qoff[s_]) + I, :I + 1]
                forced = set(np.nonzero(forced_blocks(I, 256, 512, 128))[0].tolist())
                if mode == "topk":
                    want = set(select_row_topk(L, I, param, 256, 512, 128).tolist())
                    assert got == want, (h, s_, I)
                else:
                    order = rank_order(L, I)
                    if param <= 0:
                        assert got == forced, (h, s_, I)
                        continue
                    cum = np.cumsum(np.exp(L[order] - L.max()))
                    lo = int(np.searchsorted(cum, param * cum[-1] * (1 - 1e-4)))
                    hi = int(np.searchsorted(cum, param * cum[-1] * (1 + 1e-4)))
                    ok = [set(order[:m + 1].tolist()) | forced for m in range(lo, min(hi, I) + 1)]
                    assert got in ok, (h, s_, I)
    # Against the exact ranking (the oracle's float64 scores): the ranked
    # selections decide on the fp32 fast scores, so a decision may differ from
    # the exact one only between blocks whose exact scores are within the
    # score error bound of each other (a near tie), and for top-p the mass
    # share of the GPU's prefix under the exact scores stays within the ratio
    # those errors allow.
    _, exact = oracle_scores_all_rows(w)
    k_mean = pipe.k_mean.cpu().numpy()
    ndiff = 0
    for (h, s_, I), Lx in exact.items():
        row = prob.row_index(h, s_, I)
        got = set(ci[rp[row]:rp[row + 1]].tolist())
        err = score_bound(prob, k_mean, h, s_, I) + TOL_SCORE_STATS + 2.0 ** -17 * np.abs(Lx)
        ndiff += check_ranked_row(mode, param, I, got, scores[h, int(qoff[s_]) + I, :I + 1], Lx, err)
    log(f"  {mode} {param}: {len(exact)} rows, {ndiff} decisions differ from the exact selection "
        "(all between near ties)")
    res = run_pipeline(prob, 0.1, given_csr=(rp, ci))
    G = w.spec.group
    worst = wl = 0.0
    for (h, s_, I), r in res.items():
        toks = int(w.cu_seqlens[s_]) + I * 128 + np.arange(r["out"].shape[1])
        og = out[toks][:, h * G:(h + 1) * G].transpose(1, 0, 2)
        worst = max(worst, float(np.abs(og - r["out"]).max()))
        wl = max(wl, float(np.abs(lse[h * G:(h + 1) * G][:, toks] - r["lse"]).max()))
    log(f"  out err {worst:.3g} lse err {wl:.3g}")
    assert worst <= 2e-2 and wl <= 5e-2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode,param", [("topk", 8), ("topp", 0.9)], ids=["topk_8", "topp_0.9"])
def test_ranked_selection_32k_vs_exact(mode, param):
    """Ranked selection at 32K (Hq=32 / Hkv=4, paged 64): every row's list
    against the exact (float64) scores, decisions differing from the exact
    selection only between near ties (counted)."""
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    log(f"case ranked_32k {mode} {param}")
    w = make_workload(spec_for("gqa_32k"))
    pipe = Pipeline(upload(w, "cuda"))
    pipe.discover()
    if mode == "topk":
        pipe.select_topk(param)
    else:
        pipe.select_topp(param)
    torch.cuda.synchronize()
    rp, ci = pipe.csr()
    scores = pipe.scores.cpu().numpy()
    k_mean = pipe.k_mean.cpu().numpy()
    prob, exact = oracle_scores_all_rows(w)
    qoff = prob.query_block_offsets()
    ndiff = 0
    for (h, s_, I), Lx in exact.items():
        row = prob.row_index(h, s_, I)
        got = set(ci[rp[row]:rp[row + 1]].tolist())
        err = score_bound(prob, k_mean, h, s_, I) + TOL_SCORE_STATS + 2.0 ** -17 * np.abs(Lx)
        ndiff += check_ranked_row(mode, param, I, got, scores[h, int(qoff[s_]) + I, :I + 1], Lx, err)
    log(f"  {mode} {param}: {len(exact)} rows, {ndiff} decisions differ from the exact selection "
        "(all between near ties)")


HEAD_LIST_CASES = [
    # name, spec kwargs, cached prefix per sequence (None: whole prompts)
    ("heads_bf16_ragged_g4", dict(seqlens=(300, 129, 1, 1000), num_q_heads=8, num_kv_heads=2,
                                  page_size=16, paging="permute", seed=150), None),
    ("heads_e4m3_g8", dict(seqlens=(1100, 260), num_q_heads=8, num_kv_heads=1, qk_dtype="e4m3",
                           v_dtype="bf16", page_size=16, paging="roundrobin", seed=151), None),
    ("heads_bf16_chunk", dict(seqlens=(700, 1000), num_q_heads=8, num_kv_heads=2, page_size=64,
                              seed=152), (256, 896)),
]


@pytest.mark.parametrize("splits", [1, 0], ids=["nosplit", "autosplit"])
@pytest.mark.parametrize("name,kw,ctx", HEAD_LIST_CASES, ids=[c[0] for c in HEAD_LIST_CASES])
def test_per_query_head_lists_parity(name, kw, ctx, splits):
    """One index list per query head (head_lists): scores, lists, outputs
    and lse of every (query head, sequence, query block) row against the
    oracle's per-head reading."""
    log(f"case {name} splits={splits}")
    w = make_workload(custom_spec(name=name, **kw))
    if ctx is not None:
        w = chunk_view(w, ctx)
    g = run_gpu(w, 0.1, attn_splits=splits, head_lists=True)
    assert g["scores"].shape[0] == w.spec.num_q_heads
    compare(w, g, 0.1, head_lists=True)


def test_per_query_head_lists_gqa_32k_sampled():
    """32K prompt, Hq=32 / Hkv=4, per-query-head lists: every one of the
    8192 rows' lists against the oracle's selection from its float64
    per-head scores, scores and outputs on sampled rows."""
    log("case gqa_32k head_lists")
    w = make_workload(spec_for("gqa_32k"))
    g = run_gpu(w, 0.1, head_lists=True)
    prob, sc = oracle_scores_all_rows(w, head_lists=True)
    compare_lists_all_rows(prob, sc, g["row_ptr"], g["col_idx"], 0.1)
    compare(w, g, 0.1, rows=sample_rows(w, 2, head_lists=True), check_pool=False,
            head_lists=True)


def test_per_query_head_lists_group_of_one_is_the_group_path():
    """With one query head per KV head the two list readings are the same
    computation: bit-identical scores, lists, outputs and lse."""
    log("case heads_g1")
    w = make_workload(custom_spec(name="heads_g1", seqlens=(900, 300), num_q_heads=2,
                                  num_kv_heads=2, page_size=32, seed=153))
    a = run_gpu(w, 0.1, attn_splits=1)
    b = run_gpu(w, 0.1, attn_splits=1, head_lists=True)
    for k in ("row_ptr", "col_idx", "out", "lse"):
        assert np.array_equal(a[k], b[k]), k
    # scores: only the causal entries J <= I are written
    qoff = np.concatenate([[0], np.cumsum([-(-n // 128) for n in w.spec.seqlens])])
    for s_ in range(len(w.spec.seqlens)):
        for I in range(int(qoff[s_ + 1] - qoff[s_])):
            r = int(qoff[s_]) + I
            assert np.array_equal(a["scores"][:, r, :I + 1], b["scores"][:, r, :I + 1]), (s_, I)
