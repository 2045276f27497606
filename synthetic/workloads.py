"""Seeded synthetic prefill workloads (Q, paged K/V, page table, cu_seqlens).

The recipe follows the workload text the block-sparse prefill benchmarks are
quoted on: every 128-token block b of a sequence has a centroid
c_b ~ 1.5 N(0, I_d) shared by the queries of all heads in a GQA group and by
the keys of that group's KV head; each token is its block centroid plus
0.5 N(0, I_d) noise; for every query block I >= 1, min(m, I) distinct earlier
key blocks ("needles") get their key centroid replaced by c_I + 0.3 N(0, I_d)
(later picks overwrite earlier ones); the first 256 keys of every sequence get
3 x the unit mean-query direction of their group added ("sink" keys); values
are N(0, I_d).

Draw order: every (sequence s, KV head h, role) triple has its own PCG64
stream seeded by SeedSequence(seed, spawn_key=(s, h, role)), role 0 =
centroids then needles (ascending I, one `choice` then one normal draw per I),
1 = query noise [g, L, d], 2 = key noise [L, d], 3 = values [L, d].  The
streams are independent, so the arrays do not depend on how many threads fill
them.

Storage encodings (this module only produces the input bits; decoding them is
each consumer's own business):
  * "f32": IEEE float32 as drawn;
  * "bf16": bfloat16 bit patterns (uint16), round-to-nearest-even from float32;
  * "e4m3": OCP FP8 E4M3FN codes (uint8, bias 7, max 448, saturating,
    round-to-nearest-even) of x / scale with one fp32 scale per head equal to
    amax(|x|) / 448 over all tokens of that head.

K/V live in a paged cache [num_pages, page_size, Hkv, d]; token p of sequence
s sits at page page_table[s, p // page_size], slot p % page_size.  Unused
slots of partially filled pages hold NaN patterns so that any read of them
poisons the result.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

BLOCK = 128
HEAD_DIM = 128
E4M3_MAX = 448.0


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seqlens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = HEAD_DIM
    block_size: int = BLOCK
    qk_dtype: str = "bf16"  # "f32" | "bf16" | "e4m3"
    v_dtype: str = "bf16"  # "f32" | "bf16"
    out_dtype: str = "bf16"  # "f32" | "bf16"
    page_size: int = 64
    paging: str = "permute"  # "identity" | "permute" | "roundrobin"
    needles: int = 2
    alpha: float = 0.1
    sink_tokens: int = 256
    local_tokens: int = 512
    seed: int = 20261201

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


# The five benchmark workloads (sizes as quoted with the method's results).
CONFIGS = {
    "toy_2k": WorkloadSpec(
        name="toy_2k", seqlens=(2048,), num_q_heads=4, num_kv_heads=1,
        qk_dtype="f32", v_dtype="f32", out_dtype="f32", page_size=2048,
        paging="identity", seed=20261201),
    "gqa_32k": WorkloadSpec(
        name="gqa_32k", seqlens=(32768,), num_q_heads=32, num_kv_heads=4,
        page_size=64, paging="permute", seed=20261202),
    "sweep_128k": WorkloadSpec(
        name="sweep_128k", seqlens=(131072,), num_q_heads=32, num_kv_heads=4,
        page_size=64, paging="permute", seed=20261203),
    "varlen_4x": WorkloadSpec(
        name="varlen_4x", seqlens=(8192, 24576, 65536, 131072), num_q_heads=32,
        num_kv_heads=8, qk_dtype="e4m3", v_dtype="bf16", out_dtype="bf16",
        page_size=16, paging="roundrobin", seed=20261204),
    "long_256k": WorkloadSpec(
        name="long_256k", seqlens=(262144,), num_q_heads=32, num_kv_heads=4,
        qk_dtype="e4m3", v_dtype="bf16", out_dtype="bf16", page_size=64,
        paging="permute", needles=4, seed=20261205),
}

ALPHA_SWEEP = (0.2, 0.1, 0.05, 0.025, 0.0125)


def spec_for(name: str, **overrides) -> WorkloadSpec:
    return replace(CONFIGS[name], **overrides)


def custom_spec(seqlens, num_q_heads, num_kv_heads, **kw) -> WorkloadSpec:
    kw.setdefault("name", "custom")
    return WorkloadSpec(seqlens=tuple(int(x) for x in seqlens),
                        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, **kw)


@dataclass
class Workload:
    spec: WorkloadSpec
    q: np.ndarray  # [T, Hq, d] storage dtype
    k_cache: np.ndarray  # [num_pages, page_size, Hkv, d]
    v_cache: np.ndarray  # [num_pages, page_size, Hkv, d]
    page_table: np.ndarray  # int32 [num_seqs, max_pages_per_seq]
    cu_seqlens: np.ndarray  # int32 [num_seqs + 1]
    q_scale: Optional[np.ndarray] = None  # float32 [Hq] (e4m3 only)
    k_scale: Optional[np.ndarray] = None  # float32 [Hkv] (e4m3 only)
    extra: dict = field(default_factory=dict)
    # tokens per sequence already in the KV cache before q (chunked prefill);
    # None: q covers whole prompts
    ctx_lens: Optional[np.ndarray] = None

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])


def chunk_view(w: Workload, ctx_lens) -> Workload:
    """The same prompts served in a later chunk: the first ctx_lens[s] tokens
    of sequence s count as already cached (same K/V cache and page table),
    and q holds only the remaining tokens.  No values are changed."""
    ctx = np.asarray([int(x) for x in ctx_lens], dtype=np.int32)
    cu = w.cu_seqlens
    if len(ctx) != len(cu) - 1:
        raise ValueError("one ctx length per sequence")
    lens = np.diff(cu)
    if np.any(ctx < 0) or np.any(ctx > lens) or np.any(ctx % w.spec.block_size):
        raise ValueError("ctx lengths must be multiples of the block size within each sequence")
    rows = np.concatenate([np.arange(cu[s] + ctx[s], cu[s + 1]) for s in range(len(ctx))])
    qcu = np.zeros_like(cu)
    qcu[1:] = np.cumsum(lens - ctx)
    return Workload(spec=replace(w.spec, name=w.spec.name + "_chunk"),
                    q=np.ascontiguousarray(w.q[rows.astype(np.int64)]), k_cache=w.k_cache,
                    v_cache=w.v_cache, page_table=w.page_table, cu_seqlens=qcu.astype(np.int32),
                    q_scale=w.q_scale, k_scale=w.k_scale, ctx_lens=ctx)


# --------------------------------------------------------------------------
# encoders (input production only)
# --------------------------------------------------------------------------

def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite x)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def encode_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """float -> OCP E4M3FN codes of x/scale (saturating, round to nearest even)."""
    y = np.asarray(x, dtype=np.float64) / float(scale)
    sign = (y < 0).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # quantum: 2^(e-3) for normal binades (e >= -6), 2^-9 in the subnormal range
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.ldexp(1.0, (e - 3).astype(np.int32))
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)
    _, rex = np.frexp(r)
    re = np.maximum(rex.astype(np.int64) - 1, -6)
    mant_units = np.rint(r / np.ldexp(1.0, (re - 3).astype(np.int32))).astype(np.int64)
    normal = r >= 2.0 ** -6
    E = np.where(normal, re + 7, 0)
    M = np.where(normal, mant_units - 8, mant_units)
    code = (E << 3) | M
    code = np.where(r == 0, 0, code).astype(np.uint8)
    return code | sign


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------

def _stream(seed: int, s: int, h: int, role: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(s, h, role))))


def _page_layout(spec: WorkloadSpec, seqlens: List[int]):
    P = spec.page_size
    npages = [max(1, math.ceil(L / P)) for L in seqlens]
    total = int(sum(npages))
    max_pages = max(npages)
    table = np.zeros((len(seqlens), max_pages), dtype=np.int32)
    if spec.paging == "identity":
        off = 0
        for s, n in enumerate(npages):
            table[s, :n] = np.arange(off, off + n)
            off += n
    elif spec.paging == "permute":
        perm = np.random.Generator(
            np.random.PCG64(np.random.SeedSequence(spec.seed, spawn_key=(1 << 20,)))
        ).permutation(total).astype(np.int32)
        off = 0
        for s, n in enumerate(npages):
            table[s, :n] = perm[off:off + n]
            off += n
    elif spec.paging == "roundrobin":
        nxt = 0
        filled = [0] * len(seqlens)
        while nxt < total:
            for s, n in enumerate(npages):
                if filled[s] < n:
                    table[s, filled[s]] = nxt
                    filled[s] += 1
                    nxt += 1
    else:
        raise ValueError(f"unknown paging {spec.paging!r}")
    return table, total


def _nan_fill(dtype_name: str):
    return {"f32": np.float32(np.nan), "bf16": np.uint16(0xFFC0),
            "e4m3": np.uint8(0x7F)}[dtype_name]


def _storage_dtype(dtype_name: str):
    return {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[dtype_name]


def make_workload(spec: WorkloadSpec, threads: Optional[int] = None) -> Workload:
    """Draw and encode one workload.  Deterministic in `spec` alone."""
    if spec.num_q_heads % spec.num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    seqlens = [int(x) for x in spec.seqlens]
    S, Hq, Hkv, d, B, g = len(seqlens), spec.num_q_heads, spec.num_kv_heads, \
        spec.head_dim, spec.block_size, spec.group
    T = int(sum(seqlens))
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    q32 = np.empty((T, Hq, d), dtype=np.float32)
    k32 = np.empty((T, Hkv, d), dtype=np.float32)
    v32 = np.empty((T, Hkv, d), dtype=np.float32)
    sink = min(256, max(seqlens))

    def fill(task):
        s, h = task
        L, t0 = seqlens[s], int(cu[s])
        if L == 0:  # empty sequence: no tokens to draw
            return
        n = math.ceil(L / B)
        blk = np.arange(L) // B
        rs = _stream(spec.seed, s, h, 0)
        c = (1.5 * rs.standard_normal((n, d))).astype(np.float32)
        ck = c.copy()
        for I in range(1, n):
            m = min(spec.needles, I)
            picks = rs.choice(I, size=m, replace=False)
            ck[picks] = c[I] + (0.3 * rs.standard_normal((m, d))).astype(np.float32)
        qn = np.empty((g, L, d), dtype=np.float32)
        _stream(spec.seed, s, h, 1).standard_normal(out=qn, dtype=np.float32)
        qn *= np.float32(0.5)
        qn += c[blk][None]
        kn = np.empty((L, d), dtype=np.float32)
        _stream(spec.seed, s, h, 2).standard_normal(out=kn, dtype=np.float32)
        kn *= np.float32(0.5)
        kn += ck[blk]
        u = qn.reshape(-1, d).mean(axis=0, dtype=np.float64)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        kn[:min(sink, L)] += np.float32(3.0) * u
        vn = np.empty((L, d), dtype=np.float32)
        _stream(spec.seed, s, h, 3).standard_normal(out=vn, dtype=np.float32)
        q32[t0:t0 + L, h * g:(h + 1) * g, :] = qn.transpose(1, 0, 2)
        k32[t0:t0 + L, h, :] = kn
        v32[t0:t0 + L, h, :] = vn

    nthreads = threads or min(16, os.cpu_count() or 1)
    tasks = [(s, h) for s in range(S) for h in range(Hkv)]
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, tasks))

    q_scale = k_scale = None
    if spec.qk_dtype == "f32":
        q_store, k_store = q32, k32
    elif spec.qk_dtype == "bf16":
        q_store, k_store = _par_map_heads(encode_bf16, q32, nthreads), \
            _par_map_heads(encode_bf16, k32, nthreads)
    elif spec.qk_dtype == "e4m3":
        q_scale = (np.abs(q32).max(axis=(0, 2)) / E4M3_MAX).astype(np.float32)
        k_scale = (np.abs(k32).max(axis=(0, 2)) / E4M3_MAX).astype(np.float32)
        q_store = _par_map_heads(encode_e4m3, q32, nthreads, q_scale)
        k_store = _par_map_heads(encode_e4m3, k32, nthreads, k_scale)
    else:
        raise ValueError(spec.qk_dtype)
    if spec.v_dtype == "f32":
        v_store = v32
    elif spec.v_dtype == "bf16":
        v_store = _par_map_heads(encode_bf16, v32, nthreads)
    else:
        raise ValueError(spec.v_dtype)
    del q32

    table, num_pages = _page_layout(spec, seqlens)
    P = spec.page_size
    flat = np.empty(T, dtype=np.int64)
    for s, L in enumerate(seqlens):
        pos = np.arange(L)
        flat[cu[s]:cu[s] + L] = table[s, pos // P].astype(np.int64) * P + pos % P
    k_cache = np.full((num_pages * P, Hkv, d), _nan_fill(spec.qk_dtype),
                      dtype=_storage_dtype(spec.qk_dtype))
    v_cache = np.full((num_pages * P, Hkv, d), _nan_fill(spec.v_dtype),
                      dtype=_storage_dtype(spec.v_dtype))
    k_cache[flat] = k_store
    v_cache[flat] = v_store
    return Workload(
        spec=spec, q=np.ascontiguousarray(q_store),
        k_cache=k_cache.reshape(num_pages, P, Hkv, d),
        v_cache=v_cache.reshape(num_pages, P, Hkv, d),
        page_table=table, cu_seqlens=cu, q_scale=q_scale, k_scale=k_scale)


def _par_map_heads(fn, x, nthreads, scales=None):
    """Apply an encoder head by head ([T, H, d] arrays), in parallel."""
    H = x.shape[1]
    out = None
    parts = [None] * H

    def work(h):
        parts[h] = fn(x[:, h, :]) if scales is None else fn(x[:, h, :], scales[h])

    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(work, range(H)))
    out = np.empty(x.shape, dtype=parts[0].dtype)
    for h in range(H):
        out[:, h, :] = parts[h]
    return out
