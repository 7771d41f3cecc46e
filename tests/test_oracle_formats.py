"""Pins for the oracle's number formats and for the input generator.

bf16 and OCP E4M3 decoding are checked against torch's own dtype conversions
(a library routine) and against the OFP8 spec table in tests/golden; bf16
rounding is checked against torch on values where torch rounds once, and
against hand-derived ties where a one-step rounding matters.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_philox_known_answers(syn):
    for row in _golden_rows("philox4x32_10_kat.txt"):
        vals = [int(v, 16) for v in row]
        out = syn.philox4x32_10(vals[0:4], vals[4:6])
        assert [int(v) for v in out] == vals[6:10]


def test_normal_generator_moments(syn):
    z = syn.normal_f32(7, 3, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    # tail mass of a standard normal beyond 3 sigma is 0.0027
    assert abs((np.abs(z) > 3).mean() - 0.0027) < 5e-4
    # counter-based: any sub-range regenerates identically
    assert np.array_equal(syn.normal_f32(7, 3, 1000, 64), z[1000:1064])


def test_bf16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.int32)
    ref = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([orc.bf16_to_f64(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_bf16_round_vs_torch(orc):
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # bf16/fp32 subnormals
        np.clip(rng.standard_normal(2000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),  # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0], np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    mine = np.array([orc.f64_to_bf16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_round_ties_and_single_rounding(orc):
    # 1 + 2^-8 is halfway between 1 (even mantissa) and 1 + 2^-7: ties to even -> 1.0
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert orc.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the first tie: must round up.  Rounding through binary32 first
    # would land exactly on the tie and go down; the oracle rounds once.
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert orc.f64_to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    assert orc.f64_to_bf16(float("inf")) == 0x7F80
    assert orc.f64_to_bf16(3.5e38) == 0x7F80


def test_fp8_decode_spec_table(orc):
    for code, val in _golden_rows("e4m3_spec_values.txt"):
        got = orc.fp8_to_f64(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_fp8_decode_all_codes_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([orc.fp8_to_f64(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])


def test_generator_e4m3_encoder_vs_torch(syn):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000) * 0.01,
                        np.array([0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11])]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(syn.encode_e4m3(v), ref)
    # saturation above the largest finite value instead of NaN
    assert syn.encode_e4m3(np.array([460.0, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def test_generator_bf16_encoder_vs_torch(syn):
    v = np.random.default_rng(2).standard_normal(100000).astype(np.float32) * 0.02
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(syn.encode_bf16(v), ref)


def test_record_sizes_agree(orc, syn):
    # the layout sizes each side computes on its own (no shared code)
    for wdt, H, F in [(0, 64, 128), (1, 2048, 768), (1, 4096, 14336), (2, 7168, 2048)]:
        assert orc.record_bytes(wdt, H, F) == syn.record_bytes(wdt, H, F)
    assert orc.record_bytes(1, 2048, 768) == 9437184
    assert orc.record_bytes(1, 4096, 14336) == 352321536
    assert orc.record_bytes(2, 7168, 2048) == 44050944


def test_e2m1_decode_all_codes(orc):
    # OCP MX v1.0 FP4: sign, 2 exponent bits with bias 1, 1 mantissa bit; no inf/NaN.
    # Closed form written from the bit fields, separately from the oracle's expression.
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        want = sign * (0.5 * m if e == 0 else (1 + 0.5 * m) * 2.0 ** (e - 1))
        got = orc.e2m1_to_f64(code)
        assert got == want and math.copysign(1.0, got) == sign, code
    mags = sorted({abs(orc.e2m1_to_f64(c)) for c in range(16)})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # largest normal 6, smallest subnormal 0.5


def test_e8m0_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        got = orc.e8m0_to_f64(c)
        if c == 255:
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c] == 2.0 ** (c - 127)


def test_mxfp4_record_size_and_generator(orc, syn):
    for H, F in ((256, 512), (2048, 768), (7168, 2048)):
        n = 3 * H * F
        assert orc.record_bytes(3, H, F) == syn.record_bytes(3, H, F) == n // 2 + n // 32
    H, F = 512, 256
    rec = syn.records(3, 1, 1, H, F, 3)[0]
    n = H * F
    codes = np.frombuffer(rec[:3 * n // 2].tobytes(), np.uint8)
    scales = rec[3 * n // 2:3 * n // 2 + 3 * n // 32]
    lut = np.array([orc.e2m1_to_f64(c) for c in range(16)])
    vals = lut[np.stack([codes & 15, codes >> 4], axis=1).reshape(-1)].reshape(-1, 32)
    # OCP conversion: X = 2^(floor(log2 amax) - 2), so each block's largest |w| / X lies in [4, 8)
    # and rounds to 4 or 6 (saturating); the dequantized weights keep sigma = 0.02
    assert set(np.abs(vals).max(axis=1).tolist()) <= {4.0, 6.0}
    deq = vals * np.array([orc.e8m0_to_f64(int(e)) for e in scales])[:, None]
    assert abs(deq.std() - 0.02) < 0.002 and abs(deq.mean()) < 5e-4
