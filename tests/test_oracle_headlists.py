"""Per-query-head index lists in the oracle (reading R22: the alternative to
the per-KV-group lists of R4 that the index-memory figure in the CSR /
paged-KV section of the animattoys.com FlashPrefill V2 article suggests).

Pins, each independent of the oracle's own code path:
  * a constructed case whose answer is fixed by construction: two query heads
    of one KV group aim at different key blocks, so each head's own list
    holds its block and not the other's, while the group list holds both;
    the two KV heads place the blocks the other way round, so a wrong
    query-head -> KV-head map picks the wrong block;
  * with one query head per KV head the two readings are the same thing;
  * when every head of a group carries the same queries, each head's list is
    the group's list (the group sum is g times the head sum, the normalised
    scores are equal);
  * each head's corrected output equals softmax attention over its own kept
    tokens plus n_J literal copies of (kbar_J, vbar_J) for each block that
    head pruned (token-level, via torch SDPA in float64).
"""

import math

import numpy as np

from oracle import OracleProblem, pool_blocks, run_pipeline
from synthetic import custom_spec, make_workload

B = 128


def _constructed(head_lists: bool) -> OracleProblem:
    rng = np.random.default_rng(7)
    T, hq, hkv, d = 8 * B, 4, 2, 128
    q = 0.05 * rng.standard_normal((T, hq, d))
    k = 0.05 * rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    e0, e1 = np.eye(d)[0], np.eye(d)[1]
    blk = lambda J: slice(J * B, (J + 1) * B)
    # KV head 0: block 2 along e0, block 3 along e1; KV head 1 the other way
    k[blk(2), 0] += 6 * e0
    k[blk(3), 0] += 6 * e1
    k[blk(2), 1] += 6 * e1
    k[blk(3), 1] += 6 * e0
    # queries of block 7: heads 0 and 2 along e0, heads 1 and 3 along e1
    for h, u in ((0, e0), (1, e1), (2, e0), (3, e1)):
        q[blk(7), h] += 6 * u
    pages = 8
    kc = k.reshape(pages, B, hkv, d).astype(np.float32)
    vc = v.reshape(pages, B, hkv, d).astype(np.float32)
    return OracleProblem(q=q.astype(np.float32), k_cache=kc, v_cache=vc,
                         page_table=np.arange(pages, dtype=np.int32)[None],
                         cu_seqlens=np.array([0, T], np.int32), qk_dtype="f32",
                         v_dtype="f32", head_lists=head_lists)


def test_constructed_heads_keep_their_own_block():
    kw = dict(sink_tokens=256, local_tokens=512, correction=True)
    ph = _constructed(True)
    rh = run_pipeline(ph, 0.5, rows=[(h, 0, 7) for h in range(4)], **kw)
    want = {0: 2, 1: 3, 2: 3, 3: 2}          # the block each head aims at
    for h in range(4):
        kept = set(rh[(h, 0, 7)]["kept"].tolist())
        other = 5 - want[h]
        assert want[h] in kept and other not in kept, (h, sorted(kept))
        assert kept >= {0, 1, 4, 5, 6, 7}
        assert rh[(h, 0, 7)]["out"].shape == (1, B, 128)
    pg = _constructed(False)
    rg = run_pipeline(pg, 0.5, rows=[(h, 0, 7) for h in range(2)], **kw)
    for h in range(2):
        assert {2, 3} <= set(rg[(h, 0, 7)]["kept"].tolist())
        assert rg[(h, 0, 7)]["out"].shape == (2, B, 128)
    # row order of the library: (owner, sequence, query block)
    assert ph.row_index(3, 0, 7) == 3 * 8 + 7 and pg.row_index(1, 0, 7) == 8 + 7
    assert ph.list_owners == 4 and pg.list_owners == 2
    assert [ph.list_kv_head(o) for o in range(4)] == [0, 0, 1, 1]


def _workload_problem(seqlens, hq, hkv, seed, head_lists, same_heads=False):
    w = make_workload(custom_spec(seqlens, hq, hkv, seed=seed, page_size=64))
    p = OracleProblem.from_workload(w)
    if same_heads:
        g = hq // hkv
        q = p.q.copy()
        for h in range(hkv):
            for j in range(1, g):
                q[:, h * g + j] = q[:, h * g]
        p.q = q
    p.head_lists = head_lists
    return p


def test_group_of_one_makes_the_readings_equal():
    a = run_pipeline(_workload_problem((700, 300), 2, 2, 31, False), 0.1)
    b = run_pipeline(_workload_problem((700, 300), 2, 2, 31, True), 0.1)
    assert a.keys() == b.keys()
    for key in a:
        assert np.array_equal(a[key]["kept"], b[key]["kept"])
        assert np.array_equal(a[key]["out"], b[key]["out"])


def test_identical_heads_share_the_group_list():
    g, hkv = 4, 2
    grp = run_pipeline(_workload_problem((900,), g * hkv, hkv, 32, False, True), 0.1)
    hd = run_pipeline(_workload_problem((900,), g * hkv, hkv, 32, True, True), 0.1)
    checked = 0
    for (h, s, I), r in grp.items():
        for j in range(g):
            rh = hd[(h * g + j, s, I)]
            assert np.array_equal(rh["kept"], r["kept"])
            assert np.max(np.abs(rh["out"][0] - r["out"][j])) < 1e-12
            checked += 1
    assert checked == g * len(grp)


def test_each_head_corrects_with_its_own_pruned_blocks(torch_cpu):
    prob = _workload_problem((800, 400), 4, 2, 33, True)
    res = run_pipeline(prob, 0.2, sink_tokens=128, local_tokens=256, correction=True)
    F = torch_cpu.nn.functional
    checked = 0
    for (o, s, I), r in res.items():
        kv = o // prob.group
        K, V = prob.keys(s, kv), prob.values(s, kv)
        km, cnt = pool_blocks(K, B)
        vm, _ = pool_blocks(V, B)
        kept = set(r["kept"].tolist())
        if len(kept) == I + 1:
            continue
        nI = int(cnt[I])
        p = I * B + np.arange(nI)
        keys, vals, kpos = [], [], []
        for J in range(I + 1):
            if J in kept:
                idx = np.arange(J * B, J * B + cnt[J])
                keys.append(K[idx]); vals.append(V[idx]); kpos.append(idx)
            else:
                keys.append(np.repeat(km[J][None], cnt[J], 0))
                vals.append(np.repeat(vm[J][None], cnt[J], 0))
                kpos.append(np.full(cnt[J], -1))
        Ka, Va, kp = np.concatenate(keys), np.concatenate(vals), np.concatenate(kpos)
        mask = kp[None, :] <= p[:, None]
        q = prob.queries(s, [o], p)[0]
        ref = F.scaled_dot_product_attention(
            torch_cpu.from_numpy(q)[None], torch_cpu.from_numpy(Ka)[None],
            torch_cpu.from_numpy(Va)[None], attn_mask=torch_cpu.from_numpy(mask)[None],
            scale=1.0 / math.sqrt(prob.d))[0].numpy()
        assert np.max(np.abs(r["out"][0] - ref)) < 1e-12
        checked += 1
    assert checked >= 4
