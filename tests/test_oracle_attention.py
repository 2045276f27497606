"""Pins of the oracle's attention step (no GPU).

Reference routines: torch's scaled_dot_product_attention in float64 on the
CPU (dense causal softmax attention, a library routine), and explicit
augmented key sets in which every pruned block is replaced by n_J literal
copies of its mean token -- the mean correction's ln n_J bias must equal that
duplication exactly.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import OracleProblem, attend_block, pool_blocks, run_pipeline
from synthetic import custom_spec, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(torch, q, k, v, mask=None, causal=False, scale=None):
    """q [H, Lq, d], k/v [H, Lk, d] float64 numpy -> out, via torch SDPA."""
    F = torch.nn.functional
    out = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        is_causal=causal, scale=scale)
    return out[0].numpy()


def _problem(seqlens, hq, hkv, **kw):
    return OracleProblem.from_workload(make_workload(custom_spec(seqlens, hq, hkv, **kw)))


@pytest.mark.parametrize("qk,pg,ps", [("bf16", "permute", 16), ("e4m3", "roundrobin", 64),
                                      ("f32", "identity", 256)])
def test_alpha_zero_no_correction_is_dense_causal(torch_cpu, qk, pg, ps):
    """alpha = 0 keeps every causal block; without correction the result is
    textbook dense causal softmax attention (per sequence, GQA head map
    hq // g)."""
    prob = _problem((300, 129, 1), 4, 2, qk_dtype=qk,
                    v_dtype="f32" if qk == "f32" else "bf16", paging=pg, page_size=ps, seed=21)
    res = run_pipeline(prob, 0.0, correction=False)
    for s in range(prob.num_seqs):
        L = prob.seqlen(s)
        for h in range(prob.hkv):
            heads = prob.group_heads(h)
            q = prob.queries(s, heads, np.arange(L))
            K, V = prob.keys(s, h), prob.values(s, h)
            ref = _sdpa(torch_cpu, q, np.broadcast_to(K, (len(heads),) + K.shape).copy(),
                        np.broadcast_to(V, (len(heads),) + V.shape).copy(), causal=True,
                        scale=prob.scale)
            got = np.concatenate([res[(h, s, I)]["out"] for I in range(prob.nblocks(s))], axis=1)
            assert np.max(np.abs(got - ref)) < 1e-12


def test_alpha_zero_with_correction_is_dense(torch_cpu):
    """With every block kept there is nothing to correct."""
    prob = _problem((260,), 8, 2, seed=22)
    a = run_pipeline(prob, 0.0, correction=True)
    b = run_pipeline(prob, 0.0, correction=False)
    for key in a:
        assert np.array_equal(a[key]["out"], b[key]["out"])


def _blockwise_constant_keys(prob, B):
    """Overwrite K so that every token of a block equals its block's first
    token (then kbar_J = k_t for all t in J)."""
    kc = prob.k_cache.copy()
    P = kc.shape[1]
    for s in range(prob.num_seqs):
        L = prob.seqlen(s)
        for t in range(L):
            src = (t // B) * B
            ps, pd = prob.page_table[s, src // P], prob.page_table[s, t // P]
            kc[pd, t % P] = kc[ps, src % P]
    prob.k_cache = kc
    return prob


def test_identical_keys_make_correction_exact(torch_cpu):
    """Keys constant inside each block: e^{q.k} summed over a block equals
    n_J e^{q.kbar_J}, so the corrected sparse output equals dense causal
    attention for any alpha (while blocks really are pruned)."""
    B = 128
    prob = _blockwise_constant_keys(_problem((1100,), 4, 1, seed=23, needles=1), B)
    res = run_pipeline(prob, 0.3, sink_tokens=0, local_tokens=128, correction=True)
    pruned = sum((I + 1) - len(r["kept"]) for (h, s, I), r in res.items())
    assert pruned > 10
    L = prob.seqlen(0)
    heads = prob.group_heads(0)
    q = prob.queries(0, heads, np.arange(L))
    K, V = prob.keys(0, 0), prob.values(0, 0)
    ref = _sdpa(torch_cpu, q, np.broadcast_to(K, (4,) + K.shape).copy(),
                np.broadcast_to(V, (4,) + V.shape).copy(), causal=True, scale=prob.scale)
    got = np.concatenate([res[(0, 0, I)]["out"] for I in range(prob.nblocks(0))], axis=1)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_correction_equals_duplicated_mean_tokens(torch_cpu):
    """General keys: the corrected output equals softmax attention over the
    kept tokens plus n_J literal copies of (kbar_J, vbar_J) per pruned block."""
    prob = _problem((900, 333), 4, 2, seed=24, page_size=64)
    res = run_pipeline(prob, 0.2, sink_tokens=128, local_tokens=256, correction=True)
    B = prob.block_size
    checked = 0
    for (h, s, I), r in res.items():
        K, V = prob.keys(s, h), prob.values(s, h)
        km, cnt = pool_blocks(K, B)
        vm, _ = pool_blocks(V, B)
        pruned = [J for J in range(I + 1) if J not in set(r["kept"])]
        if not pruned:
            continue
        nI = int(cnt[I])
        p = I * B + np.arange(nI)
        keys, vals, kpos = [], [], []
        for J in range(I + 1):
            if J in set(r["kept"]):
                idx = np.arange(J * B, J * B + cnt[J])
                keys.append(K[idx]); vals.append(V[idx]); kpos.append(idx)
            else:
                keys.append(np.repeat(km[J][None], cnt[J], 0))
                vals.append(np.repeat(vm[J][None], cnt[J], 0))
                kpos.append(np.full(cnt[J], -1))          # always visible
        Ka, Va, kp = np.concatenate(keys), np.concatenate(vals), np.concatenate(kpos)
        visible = kp[None, :] <= p[:, None]
        q = prob.queries(s, prob.group_heads(h), p)
        G = q.shape[0]
        ref = _sdpa(torch_cpu, q, np.broadcast_to(Ka, (G,) + Ka.shape).copy(),
                    np.broadcast_to(Va, (G,) + Va.shape).copy(),
                    mask=np.broadcast_to(visible, (G,) + visible.shape).copy(), scale=prob.scale)
        assert np.max(np.abs(r["out"] - ref)) < 1e-12
        checked += 1
    assert checked >= 4


def test_correction_changes_output_only_when_blocks_are_pruned():
    prob = _problem((1000,), 4, 1, seed=25)
    a = run_pipeline(prob, 0.5, correction=True)
    b = run_pipeline(prob, 0.5, correction=False)
    for key in a:
        same = np.array_equal(a[key]["out"], b[key]["out"])
        assert same == (len(a[key]["kept"]) == key[2] + 1)


def test_golden_tiny_example():
    """Hand-worked example (B = 2, d = 2, L = 6, scale 1); expected values are
    closed forms derived in tests/golden/tiny_b2_example.json."""
    with open(os.path.join(GOLDEN, "tiny_b2_example.json")) as f:
        ex = json.load(f)
    B = ex["block_size"]
    q = np.array(ex["q"], dtype=np.float32)[:, None, :]
    k = np.array(ex["k"], dtype=np.float32)
    v = np.array(ex["v"], dtype=np.float32)
    L = q.shape[0]
    prob = OracleProblem(q=q, k_cache=k[None, :, None, :], v_cache=v[None, :, None, :],
                         page_table=np.zeros((1, 1), np.int32),
                         cu_seqlens=np.array([0, L], np.int32), qk_dtype="f32", v_dtype="f32",
                         block_size=B, softmax_scale=1.0)
    e2 = math.exp(2.0)
    env = {"e2": e2, "ln": math.log, "exp": math.exp}
    for corr in (True, False):
        res = run_pipeline(prob, ex["alpha"], sink_tokens=ex["sink_tokens"],
                           local_tokens=ex["local_tokens"], correction=corr)
        tag = "with_correction" if corr else "without_correction"
        for row in ex["rows"]:
            I = row["I"]
            assert list(res[(0, 0, I)]["kept"]) == row["kept"]
            assert np.allclose(res[(0, 0, I)]["L"], [eval(x, env) for x in row["L"]], atol=1e-14)
            for t, exp_row in enumerate(row[tag]):
                got = res[(0, 0, I)]
                want_o = [eval(x, env) for x in exp_row["out"]]
                assert np.allclose(got["out"][0, t], want_o, atol=1e-14), (I, t, tag)
                assert np.isclose(got["lse"][0, t], eval(exp_row["lse"], env), atol=1e-14)
