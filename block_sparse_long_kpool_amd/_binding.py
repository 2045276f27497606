"""ctypes binding of libflashprefill.so (argument marshalling only).

Every step of the path runs in the HIP library; this module turns torch
tensors into device pointers, fills the C descriptor, and raises on a
non-zero status.  torch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libflashprefill.so")

FP_F32, FP_BF16, FP_E4M3 = 0, 1, 2
FP_WS_DISCOVER, FP_WS_SELECT, FP_WS_ATTN, FP_WS_DENSE = 0, 1, 2, 3
DTYPE_CODES = {"f32": FP_F32, "bf16": FP_BF16, "e4m3": FP_E4M3}

EXPORTED = (
    "fp_num_blocks", "fp_num_query_blocks", "fp_max_blocks", "fp_num_rows", "fp_scores_elems",
    "fp_csr_capacity",
    "fp_workspace_bytes", "fp_status_string", "fp_last_error",
    "fp_discover", "fp_select", "fp_select_noalloc", "fp_select_topk", "fp_select_topp",
    "fp_sparse_attn_paged", "fp_dense_attn_paged",
)


class FpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class FpProblemC(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("page_table_dev", ctypes.c_void_p),
        ("qk_dtype", ctypes.c_int32),
        ("v_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("q_scale_dev", ctypes.c_void_p),
        ("k_scale_dev", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("ctx_lens_host", ctypes.POINTER(ctypes.c_int32)),
        ("ctx_lens_dev", ctypes.c_void_p),
        ("attn_splits", ctypes.c_int32),
        ("head_lists", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once.  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m block_sparse_long_kpool_amd.build` "
            "(hipcc, gfx950).  There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(FpProblemC)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "fp_num_blocks": (i64, [P]),
        "fp_num_query_blocks": (i64, [P]),
        "fp_max_blocks": (i32, [P]),
        "fp_num_rows": (i64, [P]),
        "fp_scores_elems": (i64, [P]),
        "fp_csr_capacity": (i64, [P]),
        "fp_workspace_bytes": (sz, [P, i32]),
        "fp_status_string": (ctypes.c_char_p, [i32]),
        "fp_last_error": (ctypes.c_char_p, []),
        "fp_discover": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fp_select": (ctypes.c_int, [P, vp, vp, vp, f32, i32, i32, vp, vp, i64, vp, sz, vp]),
        "fp_select_noalloc": (ctypes.c_int, [P, vp, vp, vp, f32, i32, i32, vp, vp, i64, vp]),
        "fp_select_topk": (ctypes.c_int, [P, vp, i32, i32, i32, vp, vp, i64, vp, sz, vp]),
        "fp_select_topp": (ctypes.c_int, [P, vp, f32, i32, i32, vp, vp, i64, vp, sz, vp]),
        "fp_sparse_attn_paged": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]),
        "fp_dense_attn_paged": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise FpError(status, lib.fp_last_error().decode() or lib.fp_status_string(status).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _ptr_f64(t) -> Optional[int]:
    """Pointer of a float64 tensor (the pooled means are float64 in the ABI)."""
    if t is None:
        return None
    import torch
    if isinstance(t, torch.Tensor) and t.dtype != torch.float64:
        raise TypeError(f"pooled means must be float64 tensors, got {t.dtype}")
    return _ptr(t)


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Problem:
    """Shape/layout descriptor of one prefill batch (owns the host copy of
    cu_seqlens and keeps the device tensors it points to alive)."""

    def __init__(self, cu_seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                 page_table, page_size: int, num_pages: int, qk_dtype: str, v_dtype: str,
                 out_dtype: str, cu_seqlens_dev=None, q_scale=None, k_scale=None,
                 softmax_scale: float = 0.0, device=None, ctx_lens: Optional[Sequence[int]] = None,
                 attn_splits: int = 0, head_lists: bool = False):
        import torch
        self.device = device or page_table.device
        cu = [int(x) for x in cu_seqlens]
        self.cu_host = (ctypes.c_int32 * len(cu))(*cu)
        self.cu_dev = cu_seqlens_dev if cu_seqlens_dev is not None else \
            torch.tensor(cu, dtype=torch.int32, device=self.device)
        # cached prefix per sequence (chunked prefill); None = whole prompts
        self.ctx_host = None
        self.ctx_dev = None
        if ctx_lens is not None:
            ctx = [int(x) for x in ctx_lens]
            self.ctx_host = (ctypes.c_int32 * len(ctx))(*ctx)
            self.ctx_dev = torch.tensor(ctx, dtype=torch.int32, device=self.device)
        self.page_table = page_table
        self.q_scale = q_scale
        self.k_scale = k_scale
        self.qk_dtype, self.v_dtype, self.out_dtype = qk_dtype, v_dtype, out_dtype
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        # index-list owners: KV heads, or query heads with head_lists
        self.head_lists = bool(head_lists)
        self.list_owners = num_q_heads if head_lists else num_kv_heads
        self.total_tokens = cu[-1]
        c = FpProblemC()
        c.num_seqs = len(cu) - 1
        c.cu_seqlens_host = self.cu_host
        c.cu_seqlens_dev = _ptr(self.cu_dev)
        c.num_q_heads = num_q_heads
        c.num_kv_heads = num_kv_heads
        c.head_dim = 128
        c.block_size = 128
        c.page_size = page_size
        c.max_pages_per_seq = int(page_table.shape[1])
        c.num_pages = num_pages
        c.page_table_dev = _ptr(page_table)
        c.qk_dtype = DTYPE_CODES[qk_dtype]
        c.v_dtype = DTYPE_CODES[v_dtype]
        c.out_dtype = DTYPE_CODES[out_dtype]
        c.q_scale_dev = _ptr(q_scale)
        c.k_scale_dev = _ptr(k_scale)
        c.softmax_scale = softmax_scale
        if self.ctx_host is not None:
            c.ctx_lens_host = self.ctx_host
            c.ctx_lens_dev = _ptr(self.ctx_dev)
        c.attn_splits = attn_splits
        c.head_lists = 1 if head_lists else 0
        self.c = c
        self.lib = load_library()

    @property
    def ref(self):
        return ctypes.byref(self.c)

    def _q(self, fn):
        v = int(fn(self.ref))
        if v < 0:
            raise FpError(-1, self.lib.fp_last_error().decode())
        return v

    @property
    def num_blocks(self) -> int:
        return self._q(self.lib.fp_num_blocks)

    @property
    def num_query_blocks(self) -> int:
        return self._q(self.lib.fp_num_query_blocks)

    @property
    def max_blocks(self) -> int:
        return self._q(self.lib.fp_max_blocks)

    @property
    def num_rows(self) -> int:
        return self._q(self.lib.fp_num_rows)

    @property
    def scores_elems(self) -> int:
        return self._q(self.lib.fp_scores_elems)

    @property
    def csr_capacity(self) -> int:
        return self._q(self.lib.fp_csr_capacity)

    def workspace_bytes(self, which: int) -> int:
        return int(self.lib.fp_workspace_bytes(self.ref, which))


def fp_discover(p: Problem, q, k_cache, v_cache, k_mean, v_mean, block_scores, ws,
                stream=None) -> None:
    _check(p.lib.fp_discover(p.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr_f64(k_mean),
                             _ptr_f64(v_mean), _ptr(block_scores), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)))


def fp_select(p: Problem, q, k_mean, block_scores, alpha: float, sink_tokens: int,
              local_tokens: int, row_ptr, col_idx, ws, stream=None) -> None:
    _check(p.lib.fp_select(p.ref, _ptr(q), _ptr_f64(k_mean), _ptr(block_scores), float(alpha),
                           int(sink_tokens), int(local_tokens), _ptr(row_ptr), _ptr(col_idx),
                           col_idx.numel(), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)))


def fp_select_noalloc(p: Problem, q, k_mean, block_scores, alpha: float, sink_tokens: int,
                      local_tokens: int, row_ptr, col_idx, stream=None):
    """fp_select with the library's static scratch instead of a workspace."""
    _check(p.lib.fp_select_noalloc(p.ref, _ptr(q), _ptr_f64(k_mean), _ptr(block_scores),
                                   float(alpha), int(sink_tokens), int(local_tokens),
                                   _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                   _stream(stream)))


def fp_select_topk(p: Problem, block_scores, top_k: int, sink_tokens: int, local_tokens: int,
                   row_ptr, col_idx, ws, stream=None) -> None:
    _check(p.lib.fp_select_topk(p.ref, _ptr(block_scores), int(top_k), int(sink_tokens),
                                int(local_tokens), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def fp_select_topp(p: Problem, block_scores, top_p: float, sink_tokens: int, local_tokens: int,
                   row_ptr, col_idx, ws, stream=None) -> None:
    _check(p.lib.fp_select_topp(p.ref, _ptr(block_scores), float(top_p), int(sink_tokens),
                                int(local_tokens), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def fp_sparse_attn_paged(p: Problem, q, k_cache, v_cache, row_ptr, col_idx, k_mean, v_mean,
                         mean_correction: bool, out, lse, ws, stream=None) -> None:
    _check(p.lib.fp_sparse_attn_paged(
        p.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(row_ptr), _ptr(col_idx),
        _ptr_f64(k_mean), _ptr_f64(v_mean), 1 if mean_correction else 0, _ptr(out), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def fp_dense_attn_paged(p: Problem, q, k_cache, v_cache, out, lse, ws, stream=None) -> None:
    _check(p.lib.fp_dense_attn_paged(p.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                     _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))
