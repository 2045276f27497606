"""Pins of the oracle's e4m3 dequantisation against the values that were
encoded (no GPU).

The e4m3 inputs are OCP E4M3FN codes of x / s_h with one fp32 scale s_h per
head (reading of the FP8 passage of "FlashPrefill V2 paper reading" 4.2 and
of the FP8 section of the V2 article: e4m3 codes plus scale handling).  A
decoded value must therefore lie within half an e4m3 step of x / s_h, times
the scale of the SAME head: |dec - x| <= s_h * step(x / s_h) / 2, where the
step of a value y is 2^(max(floor(log2|y|), -6) - 3) (3 mantissa bits, the
subnormal range below 2^-6).

The reference values x come from the generator itself: the same seed with
fp32 storage draws identical arrays (every (sequence, head, role) has its
own random stream), so the f32 workload holds exactly the x that the e4m3
workload encoded.  A second case gives every head a different magnitude (a
factor of 3 per head), so that a scale taken from the wrong head, or applied
twice, is far outside the half-step bound; the test plants both mistakes in
the oracle and checks that the pin then fails.
"""

import numpy as np
import pytest

from oracle import OracleProblem, pool_blocks
from oracle import flashprefill as ofp
from synthetic import custom_spec, make_workload
from synthetic.workloads import encode_e4m3


def half_step(x, s):
    """Half the e4m3 quantisation step at x / s, in the units of x."""
    y = np.abs(np.asarray(x, dtype=np.float64) / s)
    _, ex = np.frexp(y)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    return 0.5 * s * np.ldexp(1.0, (e - 3).astype(np.int32))


def _pair(seed):
    kw = dict(seqlens=(300, 129), num_q_heads=8, num_kv_heads=2, page_size=16,
              paging="permute", seed=seed)
    w8 = make_workload(custom_spec(name="e4m3", qk_dtype="e4m3", v_dtype="bf16", **kw))
    w32 = make_workload(custom_spec(name="f32", qk_dtype="f32", v_dtype="f32", **kw))
    return w8, w32


def _check_dequant(prob8, x_q, x_k):
    """Oracle queries / keys of every head of prob8 against the encoded
    values x_q ([T, Hq, d]) and x_k (per sequence, [Hkv] of [L, d])."""
    for s in range(prob8.num_seqs):
        L = prob8.seqlen(s)
        pos = np.arange(L)
        t = int(prob8.cu_seqlens[s]) + pos
        for hq in range(prob8.hq):
            got = prob8.queries(s, [hq], pos)[0]
            x = x_q[t, hq, :].astype(np.float64)
            sc = float(np.float32(prob8.q_scale[hq]))
            assert np.all(np.abs(got - x) <= half_step(x, sc) * (1 + 1e-6)), ("q", s, hq)
        for h in range(prob8.hkv):
            got = prob8.keys(s, h)
            x = x_k[s][h].astype(np.float64)
            sc = float(np.float32(prob8.k_scale[h]))
            assert np.all(np.abs(got - x) <= half_step(x, sc) * (1 + 1e-6)), ("k", s, h)
            # pooled means: the mean of the decoded keys stays within the mean
            # of the per-element bounds of the encoded keys' mean
            km, _ = pool_blocks(got, prob8.block_size)
            kx, _ = pool_blocks(x, prob8.block_size)
            hb, _ = pool_blocks(half_step(x, sc), prob8.block_size)
            assert np.all(np.abs(km - kx) <= hb * (1 + 1e-6)), ("kbar", s, h)


def _keys_f32(w32, prob32):
    return [[prob32._paged_rows(w32.k_cache, s, h, np.arange(prob32.seqlen(s)))
             for h in range(prob32.hkv)] for s in range(prob32.num_seqs)]


def test_e4m3_decode_matches_same_seed_f32_draws():
    w8, w32 = _pair(seed=41)
    p8, p32 = OracleProblem.from_workload(w8), OracleProblem.from_workload(w32)
    _check_dequant(p8, w32.q, _keys_f32(w32, p32))


def _scaled_heads_problem():
    """e4m3 problem whose heads differ in magnitude by 3x each, encoded with
    the generator's own encoder and per-head amax / 448 scales."""
    w32 = make_workload(custom_spec(name="f32", seqlens=(260, 140), num_q_heads=4,
                                    num_kv_heads=2, qk_dtype="f32", v_dtype="f32",
                                    page_size=32, paging="roundrobin", seed=43))
    qf = w32.q * (3.0 ** np.arange(4, dtype=np.float32))[None, :, None]
    kf = w32.k_cache * (1.5 * 3.0 ** np.arange(2, dtype=np.float32))[None, None, :, None]
    q_scale = (np.abs(qf).max(axis=(0, 2)) / 448.0).astype(np.float32)
    valid = np.isfinite(kf)
    k_scale = (np.where(valid, np.abs(kf), 0).max(axis=(0, 1, 3)) / 448.0).astype(np.float32)
    q8 = np.stack([encode_e4m3(qf[:, h, :], q_scale[h]) for h in range(4)], axis=1)
    k8 = np.stack([encode_e4m3(np.where(valid[:, :, h, :], kf[:, :, h, :], 0.0), k_scale[h])
                   for h in range(2)], axis=2)
    prob8 = OracleProblem(q=q8, k_cache=k8, v_cache=w32.v_cache, page_table=w32.page_table,
                          cu_seqlens=w32.cu_seqlens, qk_dtype="e4m3", v_dtype="f32",
                          q_scale=q_scale, k_scale=k_scale)
    p32 = OracleProblem.from_workload(w32)
    xk = [[prob8._paged_rows(kf, s, h, np.arange(p32.seqlen(s))) for h in range(2)]
          for s in range(p32.num_seqs)]
    return prob8, qf, xk


def test_e4m3_scales_follow_the_head():
    prob8, qf, xk = _scaled_heads_problem()
    assert np.min(np.diff(prob8.q_scale)) > 0 and prob8.k_scale[1] > 2 * prob8.k_scale[0]
    _check_dequant(prob8, qf, xk)


@pytest.mark.parametrize("mistake", ["k_wrong_head", "q_wrong_head", "k_twice", "q_twice"])
def test_planted_scale_mistakes_fail_the_pin(monkeypatch, mistake):
    """Each planted oracle mistake (a neighbouring head's scale, or the scale
    applied twice) must make the dequantisation pin fail."""
    prob8, qf, xk = _scaled_heads_problem()
    dec = ofp.decode_e4m3
    if mistake.startswith("k"):
        def keys(self, s, h, pos=None):
            if pos is None:
                pos = np.arange(self.seqlen(s))
            raw = self._paged_rows(self.k_cache, s, h, pos)
            sc = float(self.k_scale[(h + 1) % self.hkv]) if mistake == "k_wrong_head" \
                else float(self.k_scale[h]) ** 2
            return dec(raw) * sc
        monkeypatch.setattr(OracleProblem, "keys", keys)
    else:
        def queries(self, s, heads, pos):
            t = int(self.cu_seqlens[s]) + pos - self.ctx(s)
            raw = self.q[t][:, list(heads), :]
            if mistake == "q_wrong_head":
                sc = np.asarray([self.q_scale[(h + 1) % self.hq] for h in heads], np.float64)
            else:
                sc = np.asarray([self.q_scale[h] ** 2 for h in heads], np.float64)
            return (dec(raw) * sc[None, :, None]).transpose(1, 0, 2)
        monkeypatch.setattr(OracleProblem, "queries", queries)
    with pytest.raises(AssertionError):
        _check_dequant(prob8, qf, xk)
