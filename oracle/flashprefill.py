"""Plain fp64 CPU oracle of FlashPrefill block-sparse causal prefill attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py`, never by the product path.  It shares no
code, header, table or helper with the HIP library; the only common module is
the seeded input generator (`synthetic`), which holds none of the method's
arithmetic.

Sources (the pages that describe the method), cited below by tag + section:
  [V1] "「微信、中科院」FlashPrefill：长上下文加速 28 倍" (mhpn.cn summary of
       FlashPrefill V1): 3.1 instantaneous pattern discovery (key mean
       pooling, query-block max-normalised exp sums, global re-weighting),
       3.2 max-based dynamic threshold with sink/local safety net,
       3.3 index compaction.
  [V2] "FlashPrefill V2 paper reading" (inkeast.github.io MessageDaily,
       2026-08-22): section 四 (two-stage flow, B=128, alpha=0.1, 256 sinks,
       512 local), 4.1 (block-mean correction sums), 4.3 (paged KV).
  [V2a] "長文本推理越來越長但你的顯卡等不起…FlashPrefill V2" (animattoys.com):
       mean-correction section, CSR / paged-KV section (address rule),
       chunked-prefill (分塊預填充) passage (selection redone per chunk).

Every step is computed in float64 on the exact values the GPU consumes:
bf16 bit patterns and e4m3 codes are decoded exactly (e4m3 code x fp32 scale
formed in fp64); fp32 inputs are rounded to bf16 first (the library ingests
fp32 by rounding to bf16, nearest-even).

Readings taken where the pages leave a step open:
  R1 pooling statistic is the mean ([V1] 3.1 key pooling; [V2] 4.1 uses the
     block key mean); n_J = number of tokens actually in block J.
  R2 discovery score: rows(I) = every (query head of the KV group, token of
     block I); x_rJ = scale * q_r . kbar_J; per (I, J) the max over rows
     M_IJ normalises the exp sum S_IJ = sum_r exp(x_rJ - M_IJ); re-weighting
     against the top block of row I gives Score_IJ = S_IJ exp(M_IJ - M_I),
     M_I = max_J M_IJ, and the normalised score Shat_IJ = Score_IJ / max_J
     Score_IJ.  Equivalently L_IJ = M_IJ + ln S_IJ and Shat = exp(L - max L).
  R3 discovery logits use the attention scale 1/sqrt(d).
  R4 scores are aggregated per KV group (one index list per KV head and
     query block).
  R5 the diagonal block enters discovery with its full key mean (no intra
     block causal mask).
  R6 the max runs over every causal J <= I (sinks, local and diagonal too).
  R7 keep when Shat_IJ >= alpha (ties kept).
  R8 sink blocks: J < ceil(sink_tokens / B) of each sequence.
  R9 local window: I - J < ceil(local_tokens / B); the diagonal block is kept
     in every case (a query always sees its own block).
  R10 partial last block: n_J is its true token count, ln n_J enters the
     correction, only existing query rows are scored.
  R11 correction pseudo-key: logit scale * q . kbar_J + ln n_J, value vbar_J,
     for every pruned J <= I; pruned blocks lie strictly before the diagonal,
     so every one of their tokens is causally visible.
  R12 index lists hold block indices inside the sequence, ascending.
  R19 an entry whose Shat lies within 1e-5 * alpha of alpha is "in band":
     both decisions are correct there; such entries are flagged.
  R21 top-k / top-p selection ([V1] 二: the prior methods sort (top-k) or
     accumulate probability mass (top-p); 4.4 ablates them against the
     max-based threshold): ranked by L_IJ (equivalently Score_IJ), ties toward
     the lower J; top-k adds the k best non-forced blocks to the forced ones;
     top-p adds the fewest best causal blocks whose share of sum_J e^{L_IJ}
     reaches p.  Both keep the same sink / local safety net.
  R22 per-query-head lists (the alternative to R4 that the index-memory
     figure of [V2a]'s CSR / paged-KV section suggests: its CSR size at 128K
     fits one list per query head, while PackGQA implies one per KV group):
     rows(I) are the tokens of block I for that query head alone; the head's
     keys, values and pooled blocks are those of its KV head hq // g; each
     head attends over its own list and corrects with its own pruned blocks.
     Library rows are then (query head, sequence, query block).
  R20 chunked prefill ([V2a] chunked-prefill passage): a chunk's queries are
     positions ctx .. ctx + qlen - 1 of a sequence whose first ctx tokens
     (a multiple of B) are already cached.  Pooling covers every cached key
     block; only the chunk's query blocks are scored, selected and attended,
     each exactly as the same block of the whole prompt would be (sinks,
     window and causality in positions counted from the sequence start).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

BAND_REL = 1e-5


# ---------------------------------------------------------------------------
# exact decoding of the storage formats
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bf16 is the top half of an IEEE
    binary32, so widening by 16 zero bits is exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64.  Layout s.eeee.mmm, exponent bias 7,
    E=0 encodes subnormals m/8 * 2^-6, the all-ones pattern (0x7F/0xFF) is NaN,
    there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float64.

    Works on the value, not the bits: the bf16 grid spacing in the binade of
    |x| is 2^(e-7); the quotient is rounded with numpy's half-to-even rint.
    """
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    quantum = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(a / quantum) * quantum
    return np.where(a == 0, v, np.copysign(r, v))


def decode_storage(arr: np.ndarray, dtype_name: str,
                   scale: Optional[np.ndarray] = None,
                   head_axis: int = -2) -> np.ndarray:
    """Values the GPU consumes for one stored tensor, in float64."""
    if dtype_name == "bf16":
        return decode_bf16(arr)
    if dtype_name == "f32":
        return bf16_round(arr)
    if dtype_name == "e4m3":
        vals = decode_e4m3(arr)
        shape = [1] * vals.ndim
        shape[head_axis] = -1
        return vals * np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(shape)
    raise ValueError(dtype_name)


# ---------------------------------------------------------------------------
# problem view: paged K/V and packed varlen Q
# ---------------------------------------------------------------------------

@dataclass
class OracleProblem:
    """Storage-format inputs of one prefill batch (same arrays the GPU reads)."""
    q: np.ndarray            # [T, Hq, d]
    k_cache: np.ndarray      # [num_pages, page_size, Hkv, d]
    v_cache: np.ndarray      # [num_pages, page_size, Hkv, d]
    page_table: np.ndarray   # [num_seqs, max_pages]
    cu_seqlens: np.ndarray   # [num_seqs + 1]
    qk_dtype: str
    v_dtype: str
    block_size: int = 128
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    softmax_scale: Optional[float] = None
    # Chunked prefill ([V2a] chunked-prefill passage): ctx_lens[s] tokens of
    # sequence s are already in the KV cache; the queries of this call are the
    # positions ctx .. ctx + qlen - 1 and only their blocks are scored,
    # selected and attended (reading R20: ctx is a multiple of B, so every
    # query block is a whole block of the sequence).  None: whole prompts.
    ctx_lens: Optional[np.ndarray] = None
    # Reading R22: one index list per query head instead of per KV group.
    head_lists: bool = False

    @classmethod
    def from_workload(cls, w) -> "OracleProblem":
        return cls(q=w.q, k_cache=w.k_cache, v_cache=w.v_cache,
                   page_table=w.page_table, cu_seqlens=w.cu_seqlens,
                   qk_dtype=w.spec.qk_dtype, v_dtype=w.spec.v_dtype,
                   block_size=w.spec.block_size, q_scale=w.q_scale,
                   k_scale=w.k_scale, ctx_lens=getattr(w, "ctx_lens", None))

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def hq(self) -> int:
        return self.q.shape[1]

    @property
    def hkv(self) -> int:
        return self.k_cache.shape[2]

    @property
    def d(self) -> int:
        return self.q.shape[2]

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.d)

    def ctx(self, s: int) -> int:
        return 0 if self.ctx_lens is None else int(self.ctx_lens[s])

    def qlen(self, s: int) -> int:
        return int(self.cu_seqlens[s + 1] - self.cu_seqlens[s])

    def seqlen(self, s: int) -> int:
        """Tokens in the KV cache of sequence s (cached prefix + queries)."""
        return self.ctx(s) + self.qlen(s)

    def nblocks(self, s: int) -> int:
        return -(-self.seqlen(s) // self.block_size)

    def query_blocks(self, s: int) -> range:
        return range(self.ctx(s) // self.block_size, self.nblocks(s))

    def block_offsets(self) -> np.ndarray:
        """Pooled-row offsets (key blocks) per sequence."""
        n = [self.nblocks(s) for s in range(self.num_seqs)]
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int64)

    def query_block_offsets(self) -> np.ndarray:
        """Score / CSR row offsets (query blocks) per sequence."""
        n = [len(self.query_blocks(s)) for s in range(self.num_seqs)]
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int64)

    def row_index(self, h: int, s: int, I: int) -> int:
        """Library row of (list owner, sequence, query block); the owner is the
        KV head, or the query head under reading R22."""
        qoff = self.query_block_offsets()
        return h * int(qoff[-1]) + int(qoff[s]) + I - self.ctx(s) // self.block_size

    def _paged_rows(self, cache: np.ndarray, s: int, h: int, pos: np.ndarray) -> np.ndarray:
        # [V2a] paged-KV section / [V2] 4.3: a token's address is the base of
        # its page (looked up in the page table) plus its offset in the page.
        P = cache.shape[1]
        pages = self.page_table[s, pos // P]
        return cache[pages, pos % P, h, :]

    def keys(self, s: int, h: int, pos: Optional[np.ndarray] = None) -> np.ndarray:
        if pos is None:
            pos = np.arange(self.seqlen(s))
        raw = self._paged_rows(self.k_cache, s, h, pos)
        if self.qk_dtype == "e4m3":
            return decode_e4m3(raw) * float(np.float32(self.k_scale[h]))
        return decode_storage(raw, self.qk_dtype)

    def values(self, s: int, h: int, pos: Optional[np.ndarray] = None) -> np.ndarray:
        if pos is None:
            pos = np.arange(self.seqlen(s))
        return decode_storage(self._paged_rows(self.v_cache, s, h, pos), self.v_dtype)

    def queries(self, s: int, heads: Sequence[int], pos: np.ndarray) -> np.ndarray:
        """float64 [len(heads), len(pos), d]; pos: positions in the sequence
        (cached prefix included), all >= ctx(s)."""
        t = int(self.cu_seqlens[s]) + pos - self.ctx(s)
        raw = self.q[t][:, list(heads), :]
        if self.qk_dtype == "e4m3":
            vals = decode_e4m3(raw) * np.asarray(self.q_scale, np.float32)[list(heads)] \
                .astype(np.float64)[None, :, None]
        else:
            vals = decode_storage(raw, self.qk_dtype)
        return vals.transpose(1, 0, 2)

    def group_heads(self, h: int) -> List[int]:
        g = self.group
        return list(range(h * g, (h + 1) * g))

    # List owners: KV heads (R4), or query heads under reading R22.
    @property
    def list_owners(self) -> int:
        return self.hq if self.head_lists else self.hkv

    def list_kv_head(self, o: int) -> int:
        """KV head whose keys, values and pooled blocks list owner o uses."""
        return o // self.group if self.head_lists else o

    def list_heads(self, o: int) -> List[int]:
        """Query heads whose rows list owner o scores and attends."""
        return [o] if self.head_lists else self.group_heads(o)


# ---------------------------------------------------------------------------
# step 1: block pooling            [V1] 3.1 key pooling; [V2] 4.1 kbar, vbar
# ---------------------------------------------------------------------------

def pool_blocks(x: np.ndarray, block_size: int):
    """Per-block mean of the rows of x ([L, d]); returns (means [n, d],
    counts [n]).  The last block may be partial (R10)."""
    L = x.shape[0]
    n = -(-L // block_size)
    means = np.empty((n, x.shape[1]), dtype=np.float64)
    counts = np.empty(n, dtype=np.int64)
    for J in range(n):
        rows = x[J * block_size:min(L, (J + 1) * block_size)]
        counts[J] = rows.shape[0]
        means[J] = rows.sum(axis=0) / rows.shape[0]
    return means, counts


# ---------------------------------------------------------------------------
# step 2: pooled block scores      [V1] 3.1 query pooling + global re-weighting
# ---------------------------------------------------------------------------

def block_scores(q_rows: np.ndarray, k_means: np.ndarray, scale: float) -> Dict[str, np.ndarray]:
    """Scores of one query block I against the pooled keys J = 0..I.

    q_rows: [R, d] every (head, token) row of the KV group in block I (R4).
    k_means: [I+1, d].
    Returns per J: tile max M, max-normalised exp sum S, re-weighted Score,
    normalised Shat (in (0, 1]) and the log form L = M + ln S (R2).
    """
    x = scale * (q_rows @ k_means.T)                 # [R, I+1] pooled-key logits
    M = x.max(axis=0)                                # max over the query block's rows
    S = np.exp(x - M[None, :]).sum(axis=0)           # max-normalised exp sum
    M_row = M.max()                                  # top block of the row
    Score = S * np.exp(M - M_row)                    # global re-weighting
    Shat = Score / Score.max()
    return {"M": M, "S": S, "Score": Score, "Shat": Shat, "L": M + np.log(S)}


# ---------------------------------------------------------------------------
# step 3: threshold + forced blocks + compaction   [V1] 3.2, 3.3; [V2] 四
# ---------------------------------------------------------------------------

def forced_blocks(I: int, sink_tokens: int, local_tokens: int, block_size: int) -> np.ndarray:
    J = np.arange(I + 1)
    n_sink = -(-sink_tokens // block_size)
    n_local = max(1, -(-local_tokens // block_size))
    return (J < n_sink) | (I - J < n_local)


def select_row(L_row: np.ndarray, I: int, alpha: float, sink_tokens: int,
               local_tokens: int, block_size: int):
    """Kept block indices of query block I (ascending, R12) and in-band flags.

    keep J <=> forced(J) or Shat_IJ >= alpha, Shat_IJ = exp(L_IJ - max_J' L_IJ')
    (the threshold alpha * max over J' <= I of the score, [V1] 3.2).
    """
    L_row = np.asarray(L_row[:I + 1], dtype=np.float64)
    Shat = np.exp(L_row - L_row.max())
    forced = forced_blocks(I, sink_tokens, local_tokens, block_size)
    keep = forced | (Shat >= alpha)
    band = (~forced) & (np.abs(Shat - alpha) <= BAND_REL * alpha) if alpha > 0 \
        else np.zeros(I + 1, dtype=bool)
    return np.nonzero(keep)[0].astype(np.int64), band


def rank_order(L_row: np.ndarray, I: int) -> np.ndarray:
    """Causal blocks J <= I by descending score, ties toward the lower J."""
    L = np.asarray(L_row[:I + 1], dtype=np.float64)
    return np.array(sorted(range(I + 1), key=lambda J: (-L[J], J)), dtype=np.int64)


def select_row_topk(L_row: np.ndarray, I: int, k: int, sink_tokens: int,
                    local_tokens: int, block_size: int) -> np.ndarray:
    """Top-k selection, the prior methods' strategy that [V1] 二 and the 4.4
    ablation compare with the max-based threshold (reading R21): the forced
    blocks plus the k highest-scoring other causal blocks."""
    forced = forced_blocks(I, sink_tokens, local_tokens, block_size)
    ranked = [J for J in rank_order(L_row, I) if not forced[J]]
    keep = forced.copy()
    keep[np.asarray(ranked[:max(0, k)], dtype=np.int64)] = True
    return np.nonzero(keep)[0].astype(np.int64)


def select_row_topp(L_row: np.ndarray, I: int, p: float, sink_tokens: int,
                    local_tokens: int, block_size: int) -> np.ndarray:
    """Top-p selection ([V1] 二, 4.4; reading R21): the fewest highest-scoring
    causal blocks whose share of the row's total score sum_J e^{L_IJ} reaches
    p, plus the forced blocks.  p <= 0 keeps the forced blocks only."""
    forced = forced_blocks(I, sink_tokens, local_tokens, block_size)
    keep = forced.copy()
    if p > 0:
        L = np.asarray(L_row[:I + 1], dtype=np.float64)
        order = rank_order(L_row, I)
        w = np.exp(L[order] - L.max())
        cum = np.cumsum(w)
        n = int(np.searchsorted(cum, p * cum[-1], side="left"))  # first cum >= p * total
        keep[order[:min(n + 1, I + 1)]] = True
    return np.nonzero(keep)[0].astype(np.int64)


# ---------------------------------------------------------------------------
# step 4: sparse attention with mean correction    [V2] 4.1, [V2a] 均值修正
# ---------------------------------------------------------------------------

def attend_block(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                 k_means: np.ndarray, v_means: np.ndarray, counts: np.ndarray,
                 kept: Sequence[int], I: int, block_size: int, scale: float,
                 correction: bool):
    """Output rows of query block I for a group of heads.

    q: [G, nI, d] queries of block I (token positions I*B .. I*B+nI-1);
    keys/values: [L, d] the whole sequence of the KV head;
    k_means/v_means/counts: pooled blocks of that sequence.
    Softmax over E = {tokens j <= p of kept blocks} plus, with the correction,
    one pseudo-key per pruned block J <= I with logit scale*q.kbar_J + ln n_J
    and value vbar_J (R11).  Returns out [G, nI, d] and natural-log lse [G, nI].
    """
    G, nI, _ = q.shape
    B = block_size
    p = I * B + np.arange(nI)                                    # query positions
    kept = sorted(int(J) for J in kept)
    pos = np.concatenate([np.arange(J * B, J * B + counts[J]) for J in kept])
    y = scale * np.einsum("gtd,kd->gtk", q, keys[pos])
    y = np.where(pos[None, None, :] <= p[None, :, None], y, -np.inf)
    logit_parts = [y]
    val_parts = [values[pos]]
    if correction:
        pruned = [J for J in range(I + 1) if J not in set(kept)]
        if pruned:
            pr = np.asarray(pruned)
            z = scale * np.einsum("gtd,jd->gtj", q, k_means[pr]) + np.log(counts[pr])[None, None, :]
            logit_parts.append(z)
            val_parts.append(v_means[pr])
    logits = np.concatenate(logit_parts, axis=2)
    vals = np.concatenate(val_parts, axis=0)
    m = logits.max(axis=2, keepdims=True)
    w = np.exp(logits - m)
    ell = w.sum(axis=2, keepdims=True)
    out = np.einsum("gtk,kd->gtd", w, vals) / ell
    lse = (m + np.log(ell))[..., 0]
    return out, lse


# ---------------------------------------------------------------------------
# whole pipeline
# ---------------------------------------------------------------------------

def run_pipeline(prob: OracleProblem, alpha: float, sink_tokens: int = 256,
                 local_tokens: int = 512, correction: bool = True,
                 rows: Optional[Sequence] = None, attend: bool = True,
                 given_csr: Optional[tuple] = None, cache: Optional[dict] = None) -> dict:
    """Run pool -> score -> select -> attend.

    rows: optional list of (h, s, I) to evaluate (default: all); h is the
    list owner (the KV head, or the query head under R22).  For each
    evaluated row the result holds the L scores, the kept list, the band
    flags, and (if `attend`) out [G, nI, d] / lse [G, nI] for the owner's
    query heads (G = g, or 1 under R22).
    given_csr: optional (row_ptr, col_idx) in the library's row order
    (h, global block); when set, attention uses those lists instead of the
    oracle's own selection (to compare attention alone).
    cache: optional dict kept by the caller between calls; it holds the
    decoded keys/values and pooled blocks of the last (sequence, kv head).
    """
    B = prob.block_size
    if rows is None:
        rows = [(h, s, I) for h in range(prob.list_owners) for s in range(prob.num_seqs)
                for I in prob.query_blocks(s)]
    if cache is None:
        cache = {}

    def seq_data(s, h):
        key = (s, h)
        if key not in cache:
            cache.clear()
            K = prob.keys(s, h)
            V = prob.values(s, h)
            km, cnt = pool_blocks(K, B)
            vm, _ = pool_blocks(V, B)
            cache[key] = (K, V, km, vm, cnt)
        return cache[key]

    results = {}
    for (h, s, I) in sorted(rows, key=lambda r: (r[1], r[0], r[2])):
        K, V, km, vm, cnt = seq_data(s, prob.list_kv_head(h))
        nI = int(cnt[I])
        pos = I * B + np.arange(nI)
        qg = prob.queries(s, prob.list_heads(h), pos)             # [G, nI, d]
        sc = block_scores(qg.reshape(-1, prob.d), km[:I + 1], prob.scale)
        kept, band = select_row(sc["L"], I, alpha, sink_tokens, local_tokens, B)
        res = {"L": sc["L"], "M": sc["M"], "S": sc["S"], "Shat": sc["Shat"],
               "kept": kept, "band": band}
        if attend:
            use = kept
            if given_csr is not None:
                rp, ci = given_csr
                r = prob.row_index(h, s, I)
                use = np.asarray(ci[rp[r]:rp[r + 1]], dtype=np.int64)
            out, lse = attend_block(qg, K, V, km, vm, cnt, use, I, B, prob.scale, correction)
            res["out"], res["lse"] = out, lse
            res["used"] = use
        results[(h, s, I)] = res
    return results


def pooled_all(prob: OracleProblem):
    """k_mean / v_mean [Hkv, total_blocks, d] and counts [total_blocks]."""
    B = prob.block_size
    boff = prob.block_offsets()
    nblk = int(boff[-1])
    km = np.zeros((prob.hkv, nblk, prob.d))
    vm = np.zeros((prob.hkv, nblk, prob.d))
    cnt = np.zeros(nblk, dtype=np.int64)
    for s in range(prob.num_seqs):
        for h in range(prob.hkv):
            a, c = pool_blocks(prob.keys(s, h), B)
            b, _ = pool_blocks(prob.values(s, h), B)
            km[h, boff[s]:boff[s + 1]] = a
            vm[h, boff[s]:boff[s + 1]] = b
            cnt[boff[s]:boff[s + 1]] = c
    return km, vm, cnt


def csr_from_results(prob: OracleProblem, results: dict):
    """Library-order CSR (rows (owner, s, I)) from a full run_pipeline result."""
    nq = int(prob.query_block_offsets()[-1])
    counts = np.zeros(prob.list_owners * nq, dtype=np.int64)
    lists = {}
    for (h, s, I), r in results.items():
        row = prob.row_index(h, s, I)
        lists[row] = r["kept"]
        counts[row] = len(r["kept"])
    row_ptr = np.zeros(prob.list_owners * nq + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col = np.zeros(int(row_ptr[-1]), dtype=np.int64)
    for row, kept in lists.items():
        col[row_ptr[row]:row_ptr[row + 1]] = kept
    return row_ptr, col
