"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function declared in include/flashprefill.h, answers size queries and
rejects invalid descriptors with the documented status codes before any
device work."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashprefill.h")


@pytest.fixture(scope="module")
def bind():
    import block_sparse_long_kpool_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libflashprefill.so is not built (run __graft_entry__.build())")
    m.load_library()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("fp_discover", "fp_select", "fp_sparse_attn_paged", "fp_dense_attn_paged"):
        assert n in names


def test_library_exports_every_declared_symbol(bind):
    lib = ctypes.CDLL(bind.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(bind.EXPORTED) == declared_functions()


def _problem(bind, seqlens=(300, 129, 1), hq=8, hkv=2, page=16, qk="bf16", v="bf16",
             out="bf16", **kw):
    import torch
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    ctx = kw.get("ctx_lens") or [0] * len(seqlens)
    maxp = max(1, -(-max(a + max(b, 0) for a, b in zip(seqlens, ctx)) // page))
    table = torch.zeros((len(seqlens), maxp), dtype=torch.int32)
    return bind.Problem(cu.tolist(), hq, hkv, table, page, 1000, qk, v, out,
                        cu_seqlens_dev=torch.from_numpy(cu), **kw)


def test_size_queries(bind):
    p = _problem(bind, seqlens=(300, 129, 1, 1000))
    n = [3, 2, 1, 8]
    assert p.num_blocks == sum(n)
    assert p.max_blocks == 8
    assert p.num_rows == 2 * sum(n)
    assert p.scores_elems == 2 * sum(n) * (8 + 1)  # scores + one bound per row
    assert p.csr_capacity == 2 * sum(x * (x + 1) // 2 for x in n)
    for which in (bind.FP_WS_DISCOVER, bind.FP_WS_SELECT, bind.FP_WS_ATTN, bind.FP_WS_DENSE):
        assert p.workspace_bytes(which) > 0
        assert p.workspace_bytes(which) % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(hq=6, hkv=4), -1),                 # Hq not a multiple of Hkv
    (dict(page=48), -2),                     # page size neither divides nor is a multiple of 128
    (dict(qk="e4m3", v="bf16"), -1),         # e4m3 without scales
    (dict(qk="bf16", v="f32"), -2),          # unsupported dtype combination
    (dict(hq=34, hkv=2), -2),                # group of 17 heads
])
def test_invalid_descriptors_are_rejected(bind, kw, status):
    p = _problem(bind, **kw)
    with pytest.raises(bind.FpError) as e:
        _ = p.num_blocks
    lib = bind.load_library()
    # the calls themselves return the same status without touching the device
    st = lib.fp_discover(p.ref, 1, 1, 1, 1, 1, 1, 256, 1 << 20, None)
    assert st == status, lib.fp_last_error()
    assert lib.fp_last_error()


def test_null_pointers_and_small_workspace_are_rejected(bind):
    p = _problem(bind)
    lib = bind.load_library()
    assert lib.fp_discover(p.ref, None, 1, 1, 1, 1, 1, 256, 1 << 30, None) == bind.FpError(-1, "").status
    need = p.workspace_bytes(bind.FP_WS_DISCOVER)
    assert lib.fp_discover(p.ref, 1, 1, 1, 1, 1, 1, 256, need - 1, None) == -3
    assert lib.fp_select(p.ref, 1, 1, 1, 0.1, 256, 512, 1, 1, p.csr_capacity - 1, 256,
                         1 << 30, None) == -4
    assert lib.fp_select(p.ref, 1, 1, 1, float("nan"), 256, 512, 1, 1, p.csr_capacity, 256,
                         1 << 30, None) == -1
    assert lib.fp_sparse_attn_paged(p.ref, 1, 1, 1, 1, 1, None, None, 1, 1, None, 256,
                                    1 << 30, None) == -1
    assert lib.fp_status_string(-3) == b"workspace too small"


def test_size_queries_chunked_prefill(bind):
    """Cached prefixes (chunked prefill): key blocks cover prefix + chunk,
    rows cover the chunk's query blocks only."""
    ctx = [256, 0, 512, 128]
    p = _problem(bind, seqlens=(300, 129, 0, 1000), ctx_lens=ctx)
    nk = [5, 2, 4, 9]          # ceil((ctx + q) / 128)
    i0 = [2, 0, 4, 1]          # first query block
    nq = [a - b for a, b in zip(nk, i0)]
    assert p.num_blocks == sum(nk)
    assert p.num_query_blocks == sum(nq)
    assert p.max_blocks == 9
    assert p.num_rows == 2 * sum(nq)
    assert p.scores_elems == 2 * sum(nq) * (9 + 1)
    assert p.csr_capacity == 2 * sum(a * (a + 1) // 2 - b * (b + 1) // 2 for a, b in zip(nk, i0))


@pytest.mark.parametrize("ctx", [[100, 0, 0], [-128, 0, 0]])
def test_invalid_prefix_lengths_are_rejected(bind, ctx):
    p = _problem(bind, ctx_lens=ctx)
    with pytest.raises(bind.FpError):
        _ = p.num_blocks
    lib = bind.load_library()
    assert lib.fp_discover(p.ref, 1, 1, 1, 1, 1, 1, 256, 1 << 20, None) == -1


def test_attn_split_workspace_and_validation(bind):
    """Small launches split the attention automatically; the partial outputs
    live in the attention workspace.  attn_splits = 1 never splits."""
    p0 = _problem(bind, seqlens=(300, 129))                  # automatic
    p1 = _problem(bind, seqlens=(300, 129), attn_splits=1)   # never
    p4 = _problem(bind, seqlens=(300, 129), attn_splits=4)
    w0, w1, w4 = (p.workspace_bytes(bind.FP_WS_ATTN) for p in (p0, p1, p4))
    T, hq = 429, 8
    assert w4 - w1 >= 4 * T * hq * 129 * 4   # 4 parts x (128 outputs + lse) per (token, head)
    assert w0 > w1
    with pytest.raises(bind.FpError):
        _ = _problem(bind, attn_splits=-1).num_blocks


def test_size_queries_per_query_head_lists(bind):
    """head_lists = 1: one index list per query head, so the score and CSR
    rows (and the CSR capacity) scale with Hq instead of Hkv; pooled rows and
    workspaces for pooling stay per KV head."""
    n = [3, 2, 1, 8]
    base = _problem(bind, seqlens=(300, 129, 1, 1000))
    per = _problem(bind, seqlens=(300, 129, 1, 1000), head_lists=True)
    assert per.list_owners == 8 and base.list_owners == 2
    assert per.num_blocks == base.num_blocks == sum(n)
    assert per.num_rows == 8 * sum(n)
    assert per.scores_elems == 8 * sum(n) * (8 + 1)
    assert per.csr_capacity == 4 * base.csr_capacity
    assert per.workspace_bytes(bind.FP_WS_SELECT) > base.workspace_bytes(bind.FP_WS_SELECT)
    bad = _problem(bind)
    bad.c.head_lists = 2
    with pytest.raises(bind.FpError, match="head_lists"):
        bad.num_rows


def test_csr_beyond_int32_offsets_is_rejected(bind):
    """row_ptr / col_idx offsets are int32: a batch whose every-causal-block
    capacity exceeds INT32_MAX is refused by the size queries and by every
    call before any launch (two 1M-token prompts with one list per query
    head: 2 x 32 x 8192 x 8193 / 2 entries).  Just below the limit it is
    accepted."""
    big = _problem(bind, seqlens=(8192 * 128, 8192 * 128), hq=32, hkv=4, page=128,
                   head_lists=True)
    with pytest.raises(bind.FpError, match="int32"):
        _ = big.csr_capacity
    lib = bind.load_library()
    assert lib.fp_discover(big.ref, 1, 1, 1, 1, 1, 1, 256, 1 << 30, None) == -2
    assert lib.fp_select(big.ref, 1, 1, 1, 0.1, 256, 512, 1, 1, 1 << 40, 256, 1 << 30, None) == -2
    assert lib.fp_sparse_attn_paged(big.ref, 1, 1, 1, 1, 1, 1, 1, 1, 1, None, 256,
                                    1 << 30, None) == -2
    ok = _problem(bind, seqlens=(8192 * 128, 8192 * 128), hq=32, hkv=4, page=128)
    assert ok.csr_capacity == 2 * 4 * 8192 * 8193 // 2 < 2 ** 31 - 1


def test_noalloc_select_rejects_batches_beyond_its_scratch(bind):
    """fp_select_noalloc refuses, before touching the device, a batch whose
    select workspace exceeds its static 8 MiB scratch (1M tokens with one
    list per query head: 262144 rows x 1 KiB of bitmask)."""
    p = _problem(bind, seqlens=(8192 * 128,), hq=32, hkv=4, page=128, head_lists=True)
    assert p.workspace_bytes(bind.FP_WS_SELECT) > 8 << 20
    lib = bind.load_library()
    st = lib.fp_select_noalloc(p.ref, 1, 1, 1, 0.1, 256, 512, 1, 1, p.csr_capacity, None)
    assert st == -3
    assert b"static scratch" in lib.fp_last_error()
    small = _problem(bind)
    assert small.workspace_bytes(bind.FP_WS_SELECT) <= 8 << 20
    # argument errors are reported before the device is touched as well
    assert lib.fp_select_noalloc(small.ref, None, 1, 1, 0.1, 256, 512, 1, 1,
                                 small.csr_capacity, None) == -1


def test_dense_call_validation(bind):
    """fp_dense_attn_paged: NULL tensors and a short workspace are refused
    before any launch; its workspace does not depend on head_lists (the
    dense kernel always packs the query heads of a KV head)."""
    p = _problem(bind)
    lib = bind.load_library()
    need = p.workspace_bytes(bind.FP_WS_DENSE)
    assert lib.fp_dense_attn_paged(p.ref, None, 1, 1, 1, None, 256, need, None) == -1
    assert lib.fp_dense_attn_paged(p.ref, 1, 1, 1, 1, None, 256, need - 1, None) == -3
    ph = _problem(bind, head_lists=True)
    assert ph.workspace_bytes(bind.FP_WS_DENSE) == need
