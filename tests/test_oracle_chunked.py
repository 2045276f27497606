"""Chunked prefill in the oracle ([V2a] chunked-prefill passage, reading
R20): a chunk whose first ctx tokens are cached must reproduce, row by row,
exactly what the whole-prompt oracle computes for the same query blocks
(same pooled keys, same rows, same arithmetic), and its CSR must be the
whole prompt's CSR restricted to those rows."""

import numpy as np
import pytest

from oracle import OracleProblem, csr_from_results, run_pipeline
from synthetic import chunk_view, custom_spec, make_workload

CASES = [
    # seqlens, ctx per sequence, Hq, Hkv, qk dtype, page size
    ((700, 300, 1000), (256, 0, 896), 8, 2, "bf16", 16),
    ((1300,), (1280,), 4, 1, "e4m3", 64),     # one partial block left
    ((640, 257), (640, 128), 4, 4, "bf16", 32),  # first sequence fully cached
]


@pytest.mark.parametrize("seqlens,ctx,hq,hkv,qk,page", CASES)
def test_chunk_equals_whole_prompt_rows(seqlens, ctx, hq, hkv, qk, page):
    spec = custom_spec(seqlens, hq, hkv, qk_dtype=qk, v_dtype="bf16", page_size=page,
                       seed=300 + len(seqlens), name="chunk_case")
    w = make_workload(spec)
    wc = chunk_view(w, ctx)
    full = OracleProblem.from_workload(w)
    part = OracleProblem.from_workload(wc)
    assert part.qlen(0) == seqlens[0] - ctx[0]
    assert [part.seqlen(s) for s in range(part.num_seqs)] == list(seqlens)
    rf = run_pipeline(full, 0.1)
    rc = run_pipeline(part, 0.1)
    want = {k: v for k, v in rf.items() if k[2] >= ctx[k[1]] // 128}
    assert sorted(rc) == sorted(want)
    for key, r in rc.items():
        f = want[key]
        assert np.array_equal(r["kept"], f["kept"]), key
        assert np.array_equal(r["L"], f["L"]), key
        assert np.array_equal(r["out"], f["out"]), key
        assert np.array_equal(r["lse"], f["lse"]), key
    # library-order CSR of the chunk = whole-prompt CSR rows of the chunk
    rp_c, ci_c = csr_from_results(part, rc)
    rp_f, ci_f = csr_from_results(full, rf)
    for (h, s, I) in rc:
        a = ci_c[rp_c[part.row_index(h, s, I)]:rp_c[part.row_index(h, s, I) + 1]]
        b = ci_f[rp_f[full.row_index(h, s, I)]:rp_f[full.row_index(h, s, I) + 1]]
        assert np.array_equal(a, b)


def test_chunk_view_keeps_storage():
    w = make_workload(custom_spec((384, 200), 4, 2, seed=310, page_size=16))
    wc = chunk_view(w, (128, 0))
    assert wc.k_cache is w.k_cache and wc.v_cache is w.v_cache
    assert list(wc.cu_seqlens) == [0, 256, 456]
    assert np.array_equal(wc.q[:256], w.q[128:384])
    assert np.array_equal(wc.q[256:], w.q[384:])
    with pytest.raises(ValueError):
        chunk_view(w, (100, 0))
