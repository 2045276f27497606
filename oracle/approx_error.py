"""Approximation error of the method itself, measured with the fp64 oracle.

TEST / MEASUREMENT INFRASTRUCTURE ONLY (like the rest of oracle/): it calls
the oracle and the seeded input generator, nothing of the HIP library.

For a seeded sample of query blocks per KV head of a synthetic workload, it
compares the oracle's block-sparse attention (max-based threshold alpha with
sink / local blocks, with and without the block-mean correction) against
dense causal softmax attention in float64 on the same stored values, for
each alpha of a sweep ("長文本推理越來越長但你的顯卡等不起…FlashPrefill V2",
mean-correction passage: the correction is measured over an alpha sweep from
0.2 down to 0.0125; "FlashPrefill V2 paper reading" 4.1: the correction
replaces each pruned block's exact contribution by its mean term, a second-
order error).  The dense reference is the same oracle step with every causal
block kept and no correction (pinned to torch's dense causal attention by the
oracle tests).

    python -m oracle.approx_error --workload sweep_128k --blocks 64 \\
        --out profiles/oracle_vs_dense_accuracy_sweep_128k_bf16.md
"""

from __future__ import annotations

import argparse
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.flashprefill import OracleProblem, attend_block, block_scores, pool_blocks, select_row  # noqa: E402

ALPHAS = (0.2, 0.1, 0.05, 0.025, 0.0125)


def sample_blocks(prob, s, n, seed):
    """Seeded sample of n query blocks of sequence s (without replacement)."""
    qb = np.asarray(list(prob.query_blocks(s)))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(qb, size=min(n, len(qb)), replace=False))


def measure(prob, s, h, blocks, alphas, sinks=256, local=512):
    """Per (alpha, correction): max-abs and mean-abs error of the sparse
    oracle output against dense attention over the sampled blocks of list
    owner h, and the block density of those rows."""
    B = prob.block_size
    K, V = prob.keys(s, prob.list_kv_head(h)), prob.values(s, prob.list_kv_head(h))
    km, cnt = pool_blocks(K, B)
    vm, _ = pool_blocks(V, B)
    acc = {(a, c): [0.0, 0.0, 0, 0, 0] for a in alphas for c in (True, False)}
    for I in blocks:
        I = int(I)
        nI = int(cnt[I])
        q = prob.queries(s, prob.list_heads(h), I * B + np.arange(nI))
        dense, _ = attend_block(q, K, V, km, vm, cnt, list(range(I + 1)), I, B, prob.scale, False)
        L = block_scores(q.reshape(-1, prob.d), km[:I + 1], prob.scale)["L"]
        for a in alphas:
            kept, _ = select_row(L, I, a, sinks, local, B)
            for corr in (True, False):
                out, _ = attend_block(q, K, V, km, vm, cnt, kept, I, B, prob.scale, corr)
                d = np.abs(out - dense)
                r = acc[(a, corr)]
                r[0] = max(r[0], float(d.max()))
                r[1] += float(d.sum())
                r[2] += d.size
                r[3] += len(kept)
                r[4] += I + 1
    return acc


def main():
    from synthetic import make_workload, spec_for
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="sweep_128k")
    ap.add_argument("--blocks", type=int, default=64, help="query blocks per KV head")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--threads", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    t0 = time.time()
    w = make_workload(spec_for(args.workload))
    prob = OracleProblem.from_workload(w)
    s = prob.num_seqs - 1
    jobs = [(h, sample_blocks(prob, s, args.blocks, args.seed + h)) for h in range(prob.list_owners)]
    with ThreadPoolExecutor(args.threads) as ex:
        parts = list(ex.map(lambda j: measure(prob, s, j[0], j[1], ALPHAS), jobs))
    rows = []
    for a in ALPHAS:
        for corr in (True, False):
            mx = max(p[(a, corr)][0] for p in parts)
            sm = sum(p[(a, corr)][1] for p in parts)
            n = sum(p[(a, corr)][2] for p in parts)
            kept = sum(p[(a, corr)][3] for p in parts)
            causal = sum(p[(a, corr)][4] for p in parts)
            rows.append((a, corr, kept / causal, mx, sm / n))
    secs = time.time() - t0
    spec = w.spec
    lines = [
        f"# Oracle (fp64) block-sparse attention vs dense causal attention: {spec.name}",
        "",
        "Command (from the repository root, CPU only):",
        "",
        "```",
        f"python -m oracle.approx_error --workload {spec.name} --blocks {args.blocks} "
        f"--seed {args.seed} --out <this file>",
        "```",
        "",
        f"Sample: {args.blocks} seeded query blocks per KV head of sequence {s} "
        f"({spec.seqlens[s]} tokens, {spec.num_q_heads} q / {spec.num_kv_heads} kv heads, "
        f"{spec.qk_dtype} Q/K); every (head, token) row of each sampled block.  Both sides in "
        f"float64 on the same stored values; sinks 256, local 512.  {secs:.0f} s on "
        f"{args.threads} threads.",
        "",
        "| alpha | mean correction | block density (sampled rows) | max-abs error vs dense | mean-abs error vs dense |",
        "|---|---|---|---|---|",
    ]
    for a, corr, dens, mx, mean in rows:
        lines.append(f"| {a} | {'on' if corr else 'off'} | {dens:.4f} | {mx:.4g} | {mean:.3g} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
