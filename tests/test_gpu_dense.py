"""The dense causal baseline (fp_dense_attn_paged): every causal block of
each row on the same kernel, no index lists, no correction.  Against the
fp64 oracle at alpha = 0 without correction (pinned to textbook dense causal
attention by the oracle tests), and bit-identical to the sparse kernel fed
every causal block."""

import numpy as np
import pytest

from synthetic import chunk_view, custom_spec, make_workload, spec_for

from gpu_parity_util import TOL_LSE, TOL_OUT, log, sample_rows

pytestmark = pytest.mark.gpu

CASES = [
    ("dense_bf16_ragged_g4", dict(seqlens=(300, 129, 1, 1000), num_q_heads=8, num_kv_heads=2,
                                  page_size=16, paging="permute", seed=181), None, False),
    ("dense_e4m3_g8_rr", dict(seqlens=(1100, 260), num_q_heads=8, num_kv_heads=1,
                              qk_dtype="e4m3", v_dtype="bf16", page_size=64,
                              paging="roundrobin", seed=182), None, False),
    ("dense_f32_out_f32", dict(seqlens=(640, 100), num_q_heads=4, num_kv_heads=1, qk_dtype="f32",
                               v_dtype="f32", out_dtype="f32", page_size=128, paging="identity",
                               seed=183), None, False),
    ("dense_chunk_prefix", dict(seqlens=(700, 1000), num_q_heads=8, num_kv_heads=2, page_size=64,
                                seed=184), (256, 896), False),
    ("dense_head_lists_ignored", dict(seqlens=(900, 300), num_q_heads=8, num_kv_heads=2,
                                      page_size=32, seed=185), None, True),
]


def _dense_gpu(w, head_lists=False, attn_splits=0):
    import torch
    from block_sparse_long_kpool_amd import Pipeline, upload
    pipe = Pipeline(upload(w, "cuda"), attn_splits=attn_splits, head_lists=head_lists)
    pipe.attend_dense()
    torch.cuda.synchronize()
    return pipe, pipe.out.float().cpu().numpy(), pipe.lse.cpu().numpy()


def _oracle_compare(w, out, lse, rows=None):
    from oracle import OracleProblem, run_pipeline
    prob = OracleProblem.from_workload(w)
    res = run_pipeline(prob, 0.0, correction=False, rows=rows)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    eo = el = 0.0
    for (h, s, I), r in res.items():
        heads = prob.group_heads(h)
        toks = int(w.cu_seqlens[s]) + I * 128 - prob.ctx(s) + np.arange(r["out"].shape[1])
        eo = max(eo, float(np.abs(out[toks][:, heads, :].transpose(1, 0, 2) - r["out"]).max()))
        el = max(el, float(np.abs(lse[heads][:, toks] - r["lse"]).max()))
    log(f"  dense {w.spec.name}: out err {eo:.3g} lse err {el:.3g} over {len(res)} rows")
    assert eo <= TOL_OUT[w.spec.qk_dtype] and el <= TOL_LSE
    return eo, el


@pytest.mark.parametrize("splits", [1, 0], ids=["nosplit", "autosplit"])
@pytest.mark.parametrize("name,kw,ctx,hl", CASES, ids=[c[0] for c in CASES])
def test_dense_matches_oracle(name, kw, ctx, hl, splits):
    log(f"case {name} splits={splits}")
    w = make_workload(custom_spec(name=name, **kw))
    if ctx is not None:
        w = chunk_view(w, ctx)
    _, out, lse = _dense_gpu(w, head_lists=hl, attn_splits=splits)
    _oracle_compare(w, out, lse)


def test_dense_equals_sparse_with_every_block():
    """alpha = 0 keeps every causal block, so the sparse kernel without
    correction walks the same tiles in the same order: bit-identical out
    and lse."""
    import torch
    log("case dense_vs_sparse_alpha0")
    w = make_workload(custom_spec(name="dense_vs_sparse", seqlens=(1500, 640, 129), num_q_heads=16,
                                  num_kv_heads=2, page_size=16, paging="permute", seed=186))
    pipe, out_d, lse_d = _dense_gpu(w)
    pipe.run(0.0, correction=False)
    torch.cuda.synchronize()
    assert np.array_equal(out_d, pipe.out.float().cpu().numpy())
    assert np.array_equal(lse_d, pipe.lse.cpu().numpy())


def test_dense_gqa_32k_sampled():
    log("case dense gqa_32k")
    w = make_workload(spec_for("gqa_32k"))
    _, out, lse = _dense_gpu(w)
    _oracle_compare(w, out, lse, rows=sample_rows(w, 3))
