"""Pins for the oracle's codecs: format tables, a library decoder, brute force.

Each check is independent of the oracle's own code path: torch's CPU dtype
conversions (a library routine), the OCP spec tables stored under
tests/golden/, and nearest-value searches over every code.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 0), float(v)))
    return rows


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


# ---------------------------------------------------------------- decoders

def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(F.e4m3_decode(codes), ref)


def test_e4m3_decode_landmarks_golden():
    for code, val in _golden("e4m3_landmarks.txt"):
        got = F.e4m3_decode(np.array([code]))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(F.e8m0_decode(codes), ref)


def test_e2m1_decode_all_codes_golden():
    table = _golden("e2m1_table.txt")
    assert len(table) == 16
    for code, val in table:
        got = F.e2m1_decode(np.array([code]))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_bf16_decode_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(F.bf16_decode(bits), ref)


# ---------------------------------------------------------------- encoders

def _torch_e4m3(v):
    """torch's fp32 -> float8_e4m3fn cast is RNE but not saturating: clamp first."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_decode(bits)
    vals = vals[np.isfinite(vals)]
    for shift in (0, -3, -7, 4, 9):
        v = np.ldexp(vals, shift).astype(np.float32)
        v = v[np.isfinite(v)]
        assert np.array_equal(F.e4m3_encode(v.astype(np.float64)), _torch_e4m3(v)), shift


def test_e4m3_encode_random_fp32_vs_torch():
    g = np.random.default_rng(123)
    bits = g.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # concentrate on the representable range too
    v2 = (g.standard_normal(1_000_000) * np.exp2(g.integers(-14, 10, 1_000_000))).astype(np.float32)
    for arr in (v, v2):
        assert np.array_equal(F.e4m3_encode(arr.astype(np.float64)), _torch_e4m3(arr))


def test_e4m3_encode_midpoints_and_neighbours():
    pos = F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))      # 0 .. 448
    mids = (pos[:-1] + pos[1:]) / 2                                # exact in fp32
    m32 = mids.astype(np.float32)
    cases = np.concatenate([m32, np.nextafter(m32, np.float32(0)),
                            np.nextafter(m32, np.float32(1e9)),
                            np.float32([448.0, 449.0, 463.9, 464.0, 465.0, 1e30])])
    cases = np.concatenate([cases, -cases])
    assert np.array_equal(F.e4m3_encode(cases.astype(np.float64)), _torch_e4m3(cases))


def _nearest_code_bruteforce(v, decode, codes):
    """Nearest finite code by exhaustive search; ties -> even mantissa LSB;
    beyond the range -> the largest magnitude; sign of v kept."""
    vals = decode(codes)
    out = []
    for x in v:
        best = None
        for c, y in zip(codes, vals):
            if not np.isfinite(y) or np.signbit(y) != np.signbit(x):
                continue
            d = abs(y - x)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        out.append(best[1])
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_bruteforce_nearest():
    g = np.random.default_rng(7)
    v = np.concatenate([g.standard_normal(300) * 100, g.standard_normal(300) * 0.01,
                        g.uniform(-500, 500, 100), [0.0, -0.0, 1e-9, -1e-9, 600, -600]])
    v = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(F.e4m3_encode(v),
                          _nearest_code_bruteforce(v, F.e4m3_decode, np.arange(256)))


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e2m1_encode_ties_and_saturation():
    # round half to even on the E2M1 grid; saturate at 6
    table = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0,
             5.0: 4.0, 6.0: 6.0, 7.0: 6.0, 100.0: 6.0, 0.2: 0.0, 0.3: 0.5}
    for x, y in table.items():
        assert F.e2m1_decode(F.e2m1_encode(np.array([x])))[0] == y, x
        assert F.e2m1_decode(F.e2m1_encode(np.array([-x])))[0] == -y, -x
    assert F.e2m1_encode(np.array([-0.0]))[0] == 8
    assert F.e2m1_encode(np.array([-0.1]))[0] == 8


def test_e2m1_encode_bruteforce_nearest():
    g = np.random.default_rng(11)
    v = np.concatenate([g.uniform(-8, 8, 2000), np.arange(-7, 7.01, 0.25)])
    assert np.array_equal(F.e2m1_encode(v),
                          _nearest_code_bruteforce(v, F.e2m1_decode, np.arange(16)))


def test_e2m1_pack_low_nibble_first():
    n = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    p = F.e2m1_pack(n)
    assert p.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.e2m1_unpack(p), n)


def test_bf16_round_vs_torch_on_fp32_inputs():
    g = np.random.default_rng(5)
    bits = g.integers(0, 2**32, size=500_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3e38)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_round(v.astype(np.float64))
    assert _same(got, ref)
