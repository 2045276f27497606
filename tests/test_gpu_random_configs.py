"""Seeded random small configurations on the GPU, each compared in full with
the oracle: GQA factor, head counts, page size and paging, ragged lengths
(incl. one-token sequences and partial blocks), cached prefixes, dtypes,
output dtype, alpha, sinks / window, correction, per-query-head lists, the
KV split and the softmax scale, drawn together so that their combinations
are exercised.
The draws are fixed by the seed; the printed line names the case."""

import os

import numpy as np
import pytest

from synthetic import chunk_view, custom_spec, make_workload

from gpu_parity_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu

# 200 by default (about 40 s); FP_RANDOM_CASES=N runs seeds 0 .. N-1
N_CASES = int(os.environ.get("FP_RANDOM_CASES", "200"))


def draw(seed):
    rng = np.random.default_rng(9000 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    while hkv * g > 32:
        g //= 2
    nseq = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.choice([1, 5, 127, 128, 129, 300, 640, 777, 1024, 1500], nseq)]
    dt = ["bf16", "e4m3", "f32"][int(rng.integers(0, 3))]
    kw = dict(name=f"rand{seed}", seqlens=tuple(lens), num_q_heads=hkv * g, num_kv_heads=hkv,
              qk_dtype=dt, v_dtype="f32" if dt == "f32" else "bf16",
              out_dtype=str(rng.choice(["bf16", "f32"])),
              page_size=int(rng.choice([16, 32, 64, 128, 256])),
              paging=str(rng.choice(["permute", "roundrobin"])), seed=9100 + seed)
    ctx = None
    if rng.random() < 0.5:
        ctx = [int(rng.integers(0, L // 128 + 1)) * 128 for L in lens]
        if all(c >= L for c, L in zip(ctx, lens)):
            ctx[int(np.argmax(lens))] = 0
    opts = dict(alpha=float(rng.choice([0.05, 0.1, 0.3])),
                sinks=int(rng.choice([0, 128, 256])), local=int(rng.choice([128, 512])),
                correction=bool(rng.random() < 0.75), head_lists=bool(rng.random() < 0.3),
                splits=int(rng.choice([0, 1, 3])))
    # drawn last, so the draws above stay those of the earlier cases; 0 is
    # the default 1/sqrt(d)
    opts["scale"] = float(rng.choice([0.0, 0.0, 0.04, 0.2]))
    return kw, ctx, opts


@pytest.mark.parametrize("seed", range(N_CASES), ids=[f"rand{i}" for i in range(N_CASES)])
def test_random_config_full_parity(seed):
    kw, ctx, o = draw(seed)
    log(f"case rand{seed}: {kw} ctx={ctx} {o}")
    w = make_workload(custom_spec(**kw))
    if ctx is not None:
        w = chunk_view(w, ctx)
    g = run_gpu(w, o["alpha"], o["sinks"], o["local"], o["correction"], attn_splits=o["splits"],
                head_lists=o["head_lists"], softmax_scale=o["scale"])
    compare(w, g, o["alpha"], o["sinks"], o["local"], o["correction"], head_lists=o["head_lists"],
            softmax_scale=o["scale"])
