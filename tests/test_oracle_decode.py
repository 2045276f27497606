"""Pins of the oracle's exact decoders against IEEE/OCP definitions and
against torch's own float8/bfloat16 conversions (library routines)."""

import numpy as np
import pytest

from oracle import bf16_round, decode_bf16, decode_e4m3
from synthetic.workloads import encode_bf16, encode_e4m3


def test_bf16_known_patterns():
    pats = np.array([0x3F80, 0xBF80, 0x4049, 0x0080, 0x0001, 0x7F7F, 0x0000, 0x8000],
                    dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -126, 2.0 ** -133,
            (2 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0]
    got = decode_bf16(pats)
    assert list(got) == want


def test_bf16_all_patterns_match_torch(torch_cpu):
    torch = torch_cpu
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(pats)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3_known_codes():
    codes = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x80, 0x3C], dtype=np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -448.0, -0.0, 1.5]
    assert list(decode_e4m3(codes)) == want
    assert np.isnan(decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_all_codes_match_torch(torch_cpu):
    torch = torch_cpu
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # positive codes 0..0x7E are strictly increasing (a mis-placed exponent
    # or mantissa bit breaks the ordering)
    assert np.all(np.diff(got[:0x7F]) > 0)


def test_bf16_round_matches_torch_including_ties(torch_cpu):
    torch = torch_cpu
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    # exact halfway cases: low 16 bits = 0x8000, both even and odd upper halves
    hi = rng.integers(0x0080, 0x7F00, 4096).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x), ref)


def test_generator_encoders_roundtrip(torch_cpu):
    """The generator's encoders agree with torch's conversions (so the stored
    bits are what a reader of the workload recipe expects)."""
    torch = torch_cpu
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    assert np.array_equal(decode_bf16(encode_bf16(x)),
                          torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())
    scale = float(np.float32(np.abs(x).max() / 448.0))
    codes = encode_e4m3(x, scale)
    ref = torch.from_numpy((x.astype(np.float64) / scale)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
