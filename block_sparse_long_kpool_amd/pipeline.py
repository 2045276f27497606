"""Buffer-owning wrapper of the three library calls.

`Pipeline` allocates (with torch, on the device) every buffer the three calls
need for one batch shape, then runs discover -> select -> attention on the
current stream.  `upload` copies host arrays of a batch (numpy, storage
formats) to device tensors.  No arithmetic of the method happens here.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

from ._binding import (FP_WS_ATTN, FP_WS_DENSE, FP_WS_DISCOVER, FP_WS_SELECT, Problem,
                       fp_dense_attn_paged, fp_discover, fp_select, fp_select_topk,
                       fp_select_topp, fp_sparse_attn_paged)


@dataclass
class DeviceBatch:
    q: object
    k_cache: object
    v_cache: object
    page_table: object
    cu_seqlens: object
    q_scale: Optional[object]
    k_scale: Optional[object]
    cu_host: list
    qk_dtype: str
    v_dtype: str
    out_dtype: str
    num_q_heads: int
    num_kv_heads: int
    page_size: int
    ctx_lens: Optional[list] = None  # cached prefix per sequence (chunked prefill)


def upload(batch, device="cuda", out_dtype: Optional[str] = None) -> DeviceBatch:
    """Copy a host batch (attributes q, k_cache, v_cache, page_table,
    cu_seqlens, q_scale, k_scale and spec.{qk_dtype, v_dtype, out_dtype})
    to device tensors, keeping the storage bits unchanged."""
    import numpy as np
    import torch

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    spec = batch.spec
    return DeviceBatch(
        q=dev(batch.q), k_cache=dev(batch.k_cache), v_cache=dev(batch.v_cache),
        page_table=dev(batch.page_table.astype(np.int32)),
        cu_seqlens=dev(batch.cu_seqlens.astype(np.int32)),
        q_scale=dev(batch.q_scale), k_scale=dev(batch.k_scale),
        cu_host=[int(x) for x in batch.cu_seqlens], qk_dtype=spec.qk_dtype,
        v_dtype=spec.v_dtype, out_dtype=out_dtype or spec.out_dtype,
        num_q_heads=int(batch.q.shape[1]), num_kv_heads=int(batch.k_cache.shape[2]),
        page_size=int(batch.k_cache.shape[1]),
        ctx_lens=None if getattr(batch, "ctx_lens", None) is None
        else [int(x) for x in batch.ctx_lens])


class Pipeline:
    """All device buffers of one batch shape, and the three calls in order."""

    def __init__(self, db: DeviceBatch, softmax_scale: float = 0.0, attn_splits: int = 0,
                 head_lists: bool = False):
        import torch
        self.db = db
        dev = db.q.device
        self.problem = Problem(db.cu_host, db.num_q_heads, db.num_kv_heads, db.page_table,
                               db.page_size, int(db.k_cache.shape[0]), db.qk_dtype, db.v_dtype,
                               db.out_dtype, cu_seqlens_dev=db.cu_seqlens, q_scale=db.q_scale,
                               k_scale=db.k_scale, softmax_scale=softmax_scale,
                               ctx_lens=db.ctx_lens, attn_splits=attn_splits,
                               head_lists=head_lists)
        p = self.problem
        N, NQ = p.num_blocks, p.num_query_blocks
        hkv, T, hq = db.num_kv_heads, p.total_tokens, db.num_q_heads
        f32 = torch.float32
        # pooled means, float64 (exact block means up to float64 rounding)
        self.k_mean = torch.empty((hkv, N, 128), dtype=torch.float64, device=dev)
        self.v_mean = torch.empty((hkv, N, 128), dtype=torch.float64, device=dev)
        # score rows per index-list owner (KV head, or query head with head_lists),
        # then one error bound per score row (scores_err)
        nsc = p.list_owners * NQ * p.max_blocks
        self.scores_buf = torch.empty(p.scores_elems, dtype=f32, device=dev)
        self.scores = self.scores_buf[:nsc].view(p.list_owners, NQ, p.max_blocks)
        self.scores_err = self.scores_buf[nsc:].view(p.list_owners, NQ)
        self.row_ptr = torch.empty(p.num_rows + 1, dtype=torch.int32, device=dev)
        self.col_idx = torch.empty(p.csr_capacity, dtype=torch.int32, device=dev)
        odt = torch.float32 if db.out_dtype == "f32" else torch.bfloat16
        self.out = torch.empty((T, hq, 128), dtype=odt, device=dev)
        self.lse = torch.empty((hq, T), dtype=f32, device=dev)
        self.ws = {k: torch.empty(max(256, p.workspace_bytes(k)), dtype=torch.uint8, device=dev)
                   for k in (FP_WS_DISCOVER, FP_WS_SELECT, FP_WS_ATTN)}
        self._dense_ws = None

    def discover(self, stream=None):
        d = self.db
        fp_discover(self.problem, d.q, d.k_cache, d.v_cache, self.k_mean, self.v_mean,
                    self.scores, self.ws[FP_WS_DISCOVER], stream)

    def select(self, alpha: float, sink_tokens: int = 256, local_tokens: int = 512, stream=None):
        fp_select(self.problem, self.db.q, self.k_mean, self.scores, alpha, sink_tokens,
                  local_tokens, self.row_ptr, self.col_idx, self.ws[FP_WS_SELECT], stream)

    def select_topk(self, top_k: int, sink_tokens: int = 256, local_tokens: int = 512, stream=None):
        fp_select_topk(self.problem, self.scores, top_k, sink_tokens, local_tokens, self.row_ptr,
                       self.col_idx, self.ws[FP_WS_SELECT], stream)

    def select_topp(self, top_p: float, sink_tokens: int = 256, local_tokens: int = 512, stream=None):
        fp_select_topp(self.problem, self.scores, top_p, sink_tokens, local_tokens, self.row_ptr,
                       self.col_idx, self.ws[FP_WS_SELECT], stream)

    def attend(self, correction: bool = True, with_lse: bool = True, stream=None):
        d = self.db
        fp_sparse_attn_paged(self.problem, d.q, d.k_cache, d.v_cache, self.row_ptr,
                             self.col_idx, self.k_mean, self.v_mean, correction, self.out,
                             self.lse if with_lse else None, self.ws[FP_WS_ATTN], stream)

    def attend_dense(self, with_lse: bool = True, stream=None):
        """Dense causal attention over every causal block (the aligned dense
        baseline), into the same out / lse buffers."""
        import torch
        if self._dense_ws is None:
            n = max(256, self.problem.workspace_bytes(FP_WS_DENSE))
            self._dense_ws = torch.empty(n, dtype=torch.uint8, device=self.db.q.device)
        d = self.db
        fp_dense_attn_paged(self.problem, d.q, d.k_cache, d.v_cache, self.out,
                            self.lse if with_lse else None, self._dense_ws, stream)

    def run(self, alpha: float, sink_tokens: int = 256, local_tokens: int = 512,
            correction: bool = True, stream=None):
        self.discover(stream)
        self.select(alpha, sink_tokens, local_tokens, stream)
        self.attend(correction, True, stream)
        return self.out

    def graph(self, alpha: float, sink_tokens: int = 256, local_tokens: int = 512,
              correction: bool = True):
        """Capture one whole step (discover, select, attention) into a HIP graph
        on this pipeline's buffers and return it (a torch.cuda.CUDAGraph).  A
        replay recomputes everything from the current contents of the input
        tensors, so new inputs of the same shape are copied into them in place.
        One eager step runs first: kernel attributes are set on a kernel's
        first launch, which must not happen inside the capture.  The library
        records no memset or allocation, only kernel launches."""
        import torch
        self.run(alpha, sink_tokens, local_tokens, correction)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(alpha, sink_tokens, local_tokens, correction)
        return g

    def csr(self):
        """(row_ptr, col_idx) on the host as numpy int64 arrays."""
        rp = self.row_ptr.cpu().numpy().astype("int64")
        return rp, self.col_idx[: int(rp[-1])].cpu().numpy().astype("int64")
