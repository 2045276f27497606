"""fp_select_noalloc (fp_select with the library's static device scratch
instead of a caller workspace) against fp_select through the C ABI: two
calls in a row on one stream, the second on a smaller batch, each list
bit-identical to fp_select's on the same scores."""

import numpy as np
import pytest

from synthetic import custom_spec, make_workload

from gpu_parity_util import log

pytestmark = pytest.mark.gpu


def _lists_both_ways(w, alpha):
    import torch
    from block_sparse_long_kpool_amd import Pipeline, fp_select_noalloc, upload
    pipe = Pipeline(upload(w, "cuda"))
    pipe.discover()
    pipe.select(alpha)
    rp_ref = pipe.row_ptr.clone()
    ci_ref = pipe.col_idx.clone()
    # poison the outputs, then the allocation-free call into the same buffers
    pipe.row_ptr.fill_(-7)
    pipe.col_idx.fill_(-7)
    fp_select_noalloc(pipe.problem, pipe.db.q, pipe.k_mean, pipe.scores, alpha, 256, 512,
                      pipe.row_ptr, pipe.col_idx)
    torch.cuda.synchronize()
    rp = pipe.row_ptr.cpu().numpy()
    n = int(rp[-1])
    assert np.array_equal(rp, rp_ref.cpu().numpy())
    assert np.array_equal(pipe.col_idx[:n].cpu().numpy(), ci_ref[:n].cpu().numpy())
    return n


def test_noalloc_select_equals_select_twice_smaller_second():
    big = make_workload(custom_spec(name="noalloc_big", seqlens=(5000, 1300, 700), num_q_heads=16,
                                    num_kv_heads=2, page_size=16, paging="permute", seed=171))
    small = make_workload(custom_spec(name="noalloc_small", seqlens=(900, 129), num_q_heads=8,
                                      num_kv_heads=1, qk_dtype="e4m3", v_dtype="bf16",
                                      page_size=64, paging="roundrobin", seed=172))
    n1 = _lists_both_ways(big, 0.05)
    n2 = _lists_both_ways(small, 0.1)
    log(f"  noalloc lists: {n1} then {n2} entries, identical to fp_select")
    assert n2 < n1
