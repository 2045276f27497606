"""Benchmark of the block-sparse prefill hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload sweep_128k] [--alpha 0.1]
                    [--no-correction] [--sweep] [--no-cpu-baseline]

One step = fp_discover + fp_select + fp_sparse_attn_paged over the whole
batch (inputs already resident in HBM).  Prints ONE JSON line:
  value    effective TFLOP/s = 4 * d * (kept query-key pairs, summed over
           query heads, causal inside the diagonal block) / step time
  roofline the attention kernel's achieved FLOP/s (kept pairs plus mean-
           correction pairs, 4 d FLOP each) per launch over its average
           launch time, measured with HIP events on the launch stream
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample
           of the same workload, scaled to the same unit.
"""

from __future__ import annotations

import argparse
import json
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "e4m3": 5000.0}  # MI355X dense MFMA TFLOP/s
HBM_PEAK_GBS = 8000.0
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_long_kpool_amd", "csrc", "fp_attn.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_kernel_traffic.json")


def attn_peak(spec, kp, cp, correction):
    """Time-weighted MFMA peak of the attention kernel's contractions: S = QK^T
    runs in the Q/K storage type (e4m3 -> fp8 MFMA, bf16 and fp32 inputs ->
    bf16 MFMA), P.V and every mean-correction product run in bf16."""
    d = spec.head_dim
    qk_peak = PEAK["e4m3"] if spec.qk_dtype == "e4m3" else PEAK["bf16"]
    f_qk, f_pv = 2 * d * kp, 2 * d * kp
    f_corr = 4 * d * cp if correction else 0
    t = f_qk / qk_peak + (f_pv + f_corr) / PEAK["bf16"]
    return (f_qk + f_pv + f_corr) / t


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(workload):
    """HBM traffic of one attention launch from the committed counter record
    (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the copy-kernel
    calibration); None when no record exists for this workload or the kernel
    source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("source_sha256") != source_digest(ATTN_SOURCE):
        return None
    return int(r["hbm_bytes"])


def copy_calibration(mib, reps):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE should read mib MiB per dispatch, WRITE_SIZE too)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}), flush=True)


def causal_pairs(seqlens, B=128, ctx=None):
    """Causal (query, key) pairs per query head (query positions ctx .. L-1)."""
    ctx = ctx or [0] * len(seqlens)
    return int(sum(L * (L + 1) // 2 - c * (c + 1) // 2 for L, c in zip(seqlens, ctx)))


def causal_blocks(seqlens, hkv, B=128, ctx=None):
    """Causal (query block, key block) entries over the query blocks."""
    ctx = ctx or [0] * len(seqlens)
    tot = 0
    for L, c in zip(seqlens, ctx):
        n, i0 = -(-L // B), c // B
        tot += n * (n + 1) // 2 - i0 * (i0 + 1) // 2
    return hkv * tot


def kept_pairs(row_ptr, col_idx, spec, ctx=None, head_lists=False):
    """Kept query-key pairs summed over query heads, and the mean-correction
    (query row, pruned block) pairs, from the CSR lists (host arithmetic on
    the index lists, for reporting only).  ctx: cached prefix per sequence
    (chunked prefill; rows cover the query blocks only).  head_lists: one
    list per query head (rows per query head, each used by one head)."""
    B = spec.block_size
    g = 1 if head_lists else spec.group
    owners = spec.num_q_heads if head_lists else spec.num_kv_heads
    ctx = ctx or [0] * len(spec.seqlens)
    nq = [-(-L // B) - c // B for L, c in zip(spec.seqlens, ctx)]
    qoff = np.concatenate([[0], np.cumsum(nq)])
    nrow = int(qoff[-1])
    kept = 0
    corr = 0
    for h in range(owners):
        for s, L in enumerate(spec.seqlens):
            n, i0 = -(-L // B), ctx[s] // B
            cnt = np.minimum(B, L - np.arange(n) * B)
            for I in range(i0, n):
                r = h * nrow + int(qoff[s]) + I - i0
                J = col_idx[row_ptr[r]:row_ptr[r + 1]]
                nI = int(cnt[I])
                off = J[J < I]
                kept += nI * int(cnt[off].sum()) + nI * (nI + 1) // 2
                corr += nI * (I + 1 - len(J))
    return kept * g, corr * g


def recheck_counts(scores, errb, seqlens, alpha, sinks=256, local=512, B=128, batch=8):
    """The selection's float64 re-check work, recounted on the host from the
    fast scores and their per-row bounds (scores [owners, NQ, n_max], errb
    [owners, NQ]; whole prompts): a row is re-checked when a non-forced entry
    lies within its guard of the threshold, and then every such entry plus
    every candidate for the row maximum is evaluated, in passes of `batch`
    keys over the row's queries.  The guard is the selection's rule
    (2 E + stat(l) + stat(lmax), stat(x) = 1e-3 + 2^-17 |x|, natural log),
    taken here in float64, so an entry right at a guard's edge may count
    differently from the kernel's fp32 test."""
    I = np.concatenate([np.arange(-(-n // B)) for n in seqlens])
    J = np.arange(scores.shape[2])
    valid = J[None, :] <= I[:, None]
    n_sink = -(-sinks // B)
    n_local = max(1, -(-local // B))
    forced = (J[None, :] < n_sink) | (I[:, None] - J[None, :] < n_local)
    rows = evals = passes = 0
    for o in range(scores.shape[0]):
        L = np.where(valid, scores[o].astype(np.float64), -np.inf)
        lmax = L.max(axis=1)
        thr = np.log(alpha) + lmax
        g0 = 2.0 * errb[o].astype(np.float64) + 1e-3 + 2.0 ** -17 * np.abs(lmax)
        with np.errstate(invalid="ignore"):
            g = g0[:, None] + 1e-3 + 2.0 ** -17 * np.abs(np.where(valid, L, 0.0))
            ct = valid & ~forced & (np.abs(L - thr[:, None]) <= g)
            cm = valid & (L >= lmax[:, None] - g)
        need = ct.any(axis=1)
        ev = np.where(need, ct.sum(axis=1) + cm.sum(axis=1), 0)
        rows += int(need.sum())
        evals += int(ev.sum())
        passes += int((-(-ev // batch)).sum())
    return {"rows_rechecked": rows, "rows": int(scores.shape[0] * len(I)),
            "evaluations": evals, "passes": passes}


def gpu_setup(spec, threads=None, ctx=None, attn_splits=0, head_lists=False):
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    from synthetic import chunk_view, make_workload
    t0 = time.time()
    w = make_workload(spec, threads=threads)
    if ctx is not None:
        w = chunk_view(w, ctx)
    t_gen = time.time() - t0
    db = upload(w, "cuda")
    pipe = Pipeline(db, attn_splits=attn_splits, head_lists=head_lists)
    torch.cuda.synchronize()
    return w, pipe, t_gen


def time_steps(pipe, alpha, correction, steps, warmup, sinks=256, local=512, select=None):
    """select: None for the max-based threshold (alpha), else ("topk", k) or
    ("topp", p) for the ranked selections."""
    import torch

    def do_select():
        if select is None:
            pipe.select(alpha, sinks, local)
        elif select[0] == "topk":
            pipe.select_topk(int(select[1]), sinks, local)
        else:
            pipe.select_topp(float(select[1]), sinks, local)
    for _ in range(warmup):
        pipe.discover()
        do_select()
        pipe.attend(correction, True)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        e = ev[k]
        e[0].record(st)
        pipe.discover()
        e[1].record(st)
        do_select()
        e[2].record(st)
        pipe.attend(correction, True)
        e[3].record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    disc = np.mean([e[0].elapsed_time(e[1]) for e in ev])
    sel = np.mean([e[1].elapsed_time(e[2]) for e in ev])
    att = np.mean([e[2].elapsed_time(e[3]) for e in ev])
    tot = np.mean([e[0].elapsed_time(e[3]) for e in ev])
    return dict(wall_ms=wall, step_ms=tot, discover_ms=disc, select_ms=sel, attn_ms=att)


def time_graph(pipe, alpha, correction, steps, warmup, sinks=256, local=512):
    """Whole steps replayed from one HIP graph (captured after an eager step):
    mean replay time (events) and host wall time per step."""
    import torch
    graph = pipe.graph(alpha, sinks, local, correction)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        graph.replay()
    e1.record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return dict(step_ms=e0.elapsed_time(e1) / steps, wall_ms=wall)


def time_dense(pipe, steps, warmup):
    """Dense causal attention steps (every causal block, the aligned dense
    baseline) timed with HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        pipe.attend_dense()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        pipe.attend_dense()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(w, alpha, correction, budget_s=20.0, seed=0):
    """Time the fp64 oracle on a seeded sample of (kv head, query block) rows
    of the same workload, growing the sample until ~budget_s of CPU work.
    The oracle's stage functions run in its own pipeline order (decode + pool
    the sequence once, then per row: scores, selection, attention), each
    timed on its own."""
    from oracle import OracleProblem
    from oracle.flashprefill import attend_block, block_scores, pool_blocks, select_row
    prob = OracleProblem.from_workload(w)
    spec = w.spec
    rng = np.random.default_rng(seed)
    h, s = 0, len(spec.seqlens) - 1
    B = spec.block_size
    n = -(-spec.seqlens[s] // B)
    order = rng.permutation(n)
    # decoding + pooling the sequence's keys/values is done once for all of
    # its rows: timed as its own stage, kept out of the per-row rate
    t0 = time.perf_counter()
    K, V = prob.keys(s, h), prob.values(s, h)
    km, cnt = pool_blocks(K, B)
    vm, _ = pool_blocks(V, B)
    pool_s = time.perf_counter() - t0
    st = {"score": 0.0, "select": 0.0, "attend": 0.0}
    done, flops, secs, cpu = 0, 0.0, 0.0, 0.0
    batch = 4
    while secs < budget_s and done < n:
        r0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        for I in order[done:done + batch]:
            I = int(I)
            nI = int(cnt[I])
            qg = prob.queries(s, prob.list_heads(h), I * B + np.arange(nI))
            ta = time.perf_counter()
            sc = block_scores(qg.reshape(-1, prob.d), km[:I + 1], prob.scale)
            tb = time.perf_counter()
            kept, _ = select_row(sc["L"], I, alpha, 256, 512, B)
            tc = time.perf_counter()
            attend_block(qg, K, V, km, vm, cnt, kept, I, B, prob.scale, correction)
            td = time.perf_counter()
            st["score"] += tb - ta
            st["select"] += tc - tb
            st["attend"] += td - tc
            J = np.asarray(kept)
            full = int(np.sum(J < I)) * B * nI
            flops += 4 * spec.head_dim * spec.group * (full + nI * (nI + 1) // 2)
        dt = time.perf_counter() - t0
        r1 = resource.getrusage(resource.RUSAGE_SELF)
        secs += dt
        cpu += (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
        done += min(batch, n - done)
        batch = min(64, batch * 2)
    return {
        "value": flops / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": max(1, int(round(cpu / secs))),
        "kind": "oracle",
        "sample": f"{done} of {n} query blocks of kv head {h}, sequence {s} "
                  f"(scores, select, attention per row; sequence decode + pooling "
                  f"done once outside the timed region; {secs:.1f} s)",
        "stages_s": {"decode_pool_sequence": round(pool_s, 3), "score": round(st["score"], 3),
                     "select": round(st["select"], 3), "attend": round(st["attend"], 3), "rows": done},
    }


def oracle_scores(w, threads=16):
    """Part of the oracle (cpu_baseline) leg: the fp64 oracle's block scores
    of every (list owner, sequence, query block) row of the workload, list
    owners in parallel threads.  They do not depend on alpha."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import OracleProblem, run_pipeline
    prob = OracleProblem.from_workload(w)

    def owner(h):
        rows = [(h, s, I) for s in range(prob.num_seqs) for I in prob.query_blocks(s)]
        return {k: r["L"] for k, r in run_pipeline(prob, 1.0, rows=rows, attend=False).items()}

    scores = {}
    with ThreadPoolExecutor(min(threads, prob.list_owners)) as ex:
        for part in ex.map(owner, range(prob.list_owners)):
            scores.update(part)
    return prob, scores


def oracle_parity(w, prob, scores, pipe, alpha, correction, rows_per_head=2, seed=0):
    """Part of the oracle (cpu_baseline) leg: the GPU step's results against
    the fp64 oracle on the host.  Index lists: every row against the
    oracle's selection from its float64 scores (entries inside the oracle's
    1e-5 band at the threshold are counted, not compared).  Outputs and lse:
    a seeded sample of rows per list owner (first and last block included)
    against the oracle fed the GPU's own lists.  Returns the fields of the
    measurement line's `parity` object."""
    import torch
    from oracle import run_pipeline, select_row
    t0 = time.time()
    torch.cuda.synchronize()
    rp, ci = pipe.csr()
    out = pipe.out.float().cpu().numpy()
    lse = pipe.lse.cpu().numpy()
    B = prob.block_size
    band = mism = 0
    for (h, s, I), L in scores.items():
        kept, flag = select_row(L, I, alpha, 256, 512, B)
        row = prob.row_index(h, s, I)
        fl = set(np.nonzero(flag)[0].tolist())
        band += len(fl)
        mism += len((set(ci[rp[row]:rp[row + 1]].tolist()) ^ set(kept.tolist())) - fl)
    rng = np.random.default_rng(seed)
    sample = []
    for s in range(prob.num_seqs):
        qb = list(prob.query_blocks(s))
        for h in range(prob.list_owners):
            pick = {qb[0], qb[-1]} | set(int(x) for x in rng.choice(qb, min(len(qb), rows_per_head),
                                                                     replace=False))
            sample += [(h, s, I) for I in sorted(pick)]
    res = run_pipeline(prob, alpha, correction=correction, rows=sample, given_csr=(rp, ci))
    emax = esum = lmax = 0.0
    n = 0
    for (h, s, I), r in res.items():
        heads = prob.list_heads(h)
        toks = int(w.cu_seqlens[s]) + I * B - prob.ctx(s) + np.arange(r["out"].shape[1])
        d = np.abs(out[toks][:, heads, :].transpose(1, 0, 2) - r["out"])
        emax = max(emax, float(d.max()))
        esum += float(d.sum())
        n += d.size
        lmax = max(lmax, float(np.abs(lse[heads][:, toks] - r["lse"]).max()))
    return {
        "rows": len(scores),
        "in_band": int(band),
        "mismatches": int(mism),
        "max_abs_err": round(emax, 6),
        "mean_abs_err": float("%.3g" % (esum / max(1, n))),
        "lse_max_abs_err": round(lmax, 6),
        "sampled_rows": len(res),
        "tolerance": {"bf16": 2e-2, "f32": 2e-2, "e4m3": 6e-2}[w.spec.qk_dtype],
        "oracle": "fp64 CPU oracle: lists of every row; outputs and lse of the sampled rows, "
                  "fed the GPU's lists",
        "seconds": round(time.time() - t0, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sweep_128k")
    ap.add_argument("--alpha", type=float, default=0.1)
    ap.add_argument("--no-correction", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the alpha sweep x correction (written to --sweep-out)")
    ap.add_argument("--sweep-out", default="sweep.jsonl")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select", default="threshold", metavar="MODE",
                    help="block selection: threshold (alpha), topk:K or topp:P (the ranked "
                         "strategies the max-based threshold is compared with)")
    ap.add_argument("--attn-splits", type=int, default=0,
                    help="KV split of the attention: 0 automatic, 1 never, n parts per row")
    ap.add_argument("--chunk-ctx", type=int, default=None, metavar="TOKENS",
                    help="chunked prefill: the first TOKENS tokens of every prompt are already "
                         "cached (a multiple of 128); the step processes the rest")
    ap.add_argument("--head-lists", action="store_true",
                    help="one index list per query head instead of per KV group (ablation)")
    ap.add_argument("--dense", action="store_true",
                    help="also time the dense causal baseline (fp_dense_attn_paged: every causal "
                         "block, same kernel, no lists, no correction) and report the ratio")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--graph", action="store_true",
                    help="also time whole steps replayed from one HIP graph (graph_ms_per_step)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the op would shard by KV head with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synthetic import ALPHA_SWEEP
    from synthetic.workloads import spec_for
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return

    spec = spec_for(args.workload)
    correction = not args.no_correction
    ctx = None if args.chunk_ctx is None else [min(args.chunk_ctx, L) // 128 * 128
                                               for L in spec.seqlens]
    hl = args.head_lists
    w, pipe, t_gen = gpu_setup(spec, ctx=ctx, attn_splits=args.attn_splits, head_lists=hl)
    print(f"# generated {spec.name} in {t_gen:.1f} s", file=sys.stderr, flush=True)
    select = None
    if args.select != "threshold":
        mode, val = args.select.split(":")
        assert mode in ("topk", "topp"), args.select
        select = (mode, float(val))
    t = time_steps(pipe, args.alpha, correction, args.steps, args.warmup, select=select)
    rp, ci = pipe.csr()
    kp, cp = kept_pairs(rp, ci, spec, ctx, hl)
    d = spec.head_dim
    eff = 4 * d * kp / (t["step_ms"] * 1e-3) / 1e12
    attn_flop = 4 * d * (kp + (cp if correction else 0))
    achieved = attn_flop / (t["attn_ms"] * 1e-3) / 1e12
    peak = attn_peak(spec, kp, cp, correction)
    causal = causal_pairs(spec.seqlens, ctx=ctx) * spec.num_q_heads
    nrows = int(rp.shape[0] - 1)
    cblocks = causal_blocks(spec.seqlens, spec.num_q_heads if hl else spec.num_kv_heads, ctx=ctx)
    line = {
        "metric": "sparse prefill attn ms + effective TFLOP/s (% MFMA peak) at 128K, bf16/fp8",
        "value": round(eff, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.qk_dtype,
        "data": "synthetic (seeded centroid/needle/sink generator)",
        "config": {
            "workload": spec.name,
            "seqlens": list(spec.seqlens),
            "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads,
            "head_dim": d,
            "block_size": spec.block_size,
            "qk_dtype": spec.qk_dtype,
            "v_dtype": spec.v_dtype,
            "page_size": spec.page_size,
            "alpha": args.alpha,
            "sink_tokens": 256,
            "local_tokens": 512,
            "mean_correction": correction,
        },
        "stages_ms": {k: round(v, 4) for k, v in t.items()},
        "pct_peak": round(100 * eff / attn_peak(spec, kp, 0, False), 2),
        "discovery_selection_frac": round((t["discover_ms"] + t["select_ms"]) / t["step_ms"], 4),
        "density": {
            "block": round(int(rp[-1]) / cblocks, 5),
            "pair": round(kp / causal, 5),
            "csr_bytes": int(4 * (rp.shape[0] + rp[-1])),
            "rows": nrows,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_kernel",
            "achieved": round(achieved, 3),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            # the same launches counted on kept pairs only (the correction's
            # FLOPs left out), against the peak of the kept pairs' contractions
            "kept_pairs_frac": round(4 * d * kp / (t["attn_ms"] * 1e-3) / 1e12
                                     / attn_peak(spec, kp, 0, False), 4),
            "traffic": traffic_for(spec.name) if args.alpha == 0.1 and correction else None,
            "flop_per_launch": attn_flop,
            "peak_basis": "QK^T at the %s MFMA rate, P.V and correction at bf16"
                          % ("fp8" if spec.qk_dtype == "e4m3" else "bf16"),
        },
        "cpu_baseline": None,
    }
    if select is None and ctx is None and not hl and args.alpha > 0:
        # the selection's float64 re-check work on the timed step's scores
        line["selection"] = recheck_counts(pipe.scores.cpu().numpy(),
                                           pipe.scores_err.cpu().numpy(), spec.seqlens,
                                           args.alpha)
    # the oracle (cpu_baseline) leg: first the correctness of the timed step
    # (before any other configuration overwrites its results), at the end the
    # oracle's own throughput on a bounded sample
    oracle_leg = not args.no_cpu_baseline and ctx is None and select is None and not hl
    oscores = None
    if oracle_leg:
        t_or = time.time()
        oprob, oscores = oracle_scores(w)
        line["parity"] = oracle_parity(w, oprob, oscores, pipe, args.alpha, correction)
        line["parity"]["oracle_scores_s"] = round(time.time() - t_or, 1)
    if args.attn_splits:
        line["config"]["attn_splits"] = args.attn_splits
    if select is not None:
        line["config"]["select"] = args.select
        line["roofline"]["traffic"] = None
    if args.dense:
        causal_all = causal_pairs(spec.seqlens, ctx=ctx) * spec.num_q_heads
        dms = time_dense(pipe, args.dense_steps, 1)
        dflop = 4 * d * causal_all
        dpeak = attn_peak(spec, causal_all, 0, False)
        line["dense"] = {
            "kernel": "attn_kernel (dense instance)",
            "ms": round(dms, 3),
            "achieved": round(dflop / (dms * 1e-3) / 1e12, 3),
            "peak": round(dpeak, 1),
            "unit": "TFLOP/s",
            "frac": round(dflop / (dms * 1e-3) / 1e12 / dpeak, 4),
            "flop_per_launch": dflop,
            "ratio_vs_sparse_step": round(dms / t["step_ms"], 3),
            "ratio_vs_sparse_attn": round(dms / t["attn_ms"], 3),
        }
    if args.graph and select is None:
        tg = time_graph(pipe, args.alpha, correction, args.steps, args.warmup)
        line["graph_ms_per_step"] = round(tg["step_ms"], 4)
        line["graph_wall_ms_per_step"] = round(tg["wall_ms"], 4)
    if hl:
        line["config"]["index_lists"] = "per_query_head"
        line["roofline"]["traffic"] = None
    if ctx is not None:
        line["config"]["chunk"] = {"cached_tokens": ctx, "query_tokens":
                                   [L - c for L, c in zip(spec.seqlens, ctx)]}
        line["roofline"]["traffic"] = None
    if args.sweep:
        os.makedirs(os.path.dirname(args.sweep_out) or ".", exist_ok=True)
        with open(args.sweep_out, "w") as f:
            for a in ALPHA_SWEEP:
                for corr in (True, False):
                    ts = time_steps(pipe, a, corr, max(3, args.steps // 2), 1)
                    r2, c2 = pipe.csr()
                    k2, q2 = kept_pairs(r2, c2, spec, ctx, hl)
                    rec = dict(workload=spec.name, alpha=a, correction=corr,
                               block_density=int(r2[-1]) / cblocks,
                               pair_density=k2 / causal,
                               eff_tflops=4 * d * k2 / (ts["step_ms"] * 1e-3) / 1e12, **ts)
                    if oscores is not None:
                        pf = oracle_parity(w, oprob, oscores, pipe, a, corr)
                        rec.update(in_band=pf["in_band"], mismatches=pf["mismatches"],
                                   max_abs_err=pf["max_abs_err"], mean_abs_err=pf["mean_abs_err"],
                                   lse_max_abs_err=pf["lse_max_abs_err"])
                    f.write(json.dumps(rec) + "\n")
                    print("# sweep " + json.dumps(rec), file=sys.stderr, flush=True)
    if oracle_leg:
        line["cpu_baseline"] = cpu_baseline(w, args.alpha, correction, budget_s=args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
