"""Pins for the oracle's FP8 quantizers: invariants, closed forms, brute force.

The brute-force references below loop over single groups in plain Python and
pick codes by exhaustive nearest-value search, so they share no step with
the vectorised oracle except the fp32 division that defines the reading.
"""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import quant as Q

ALL_CODES = np.arange(256)
DEC = F.e4m3_decode(ALL_CODES)
FINITE = np.isfinite(DEC)


def _nearest_e4m3(x):
    """Exhaustive nearest finite E4M3 code; ties to even; sign kept; saturates."""
    best = None
    for c in range(256):
        y = DEC[c]
        if not FINITE[c] or np.signbit(y) != np.signbit(x):
            continue
        d = abs(y - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def _bf(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _brute_group(vals, fmt):
    """One group, pure Python: returns (codes, stored scale)."""
    amax = max(abs(float(v)) for v in vals)
    if fmt == Q.SCALE_FLOAT:
        s = np.float32(1.0) if amax == 0 else np.float32(np.float32(amax) / np.float32(448.0))
        codes = [_nearest_e4m3(float(np.float32(np.float32(v) / s))) for v in vals]
        return codes, s
    # ue8m0: smallest e with 448 * 2^e >= amax, by search
    if amax == 0:
        e = 0
    else:
        e = -200
        while 448.0 * 2.0 ** e < amax:
            e += 1
    e = max(-127, min(127, e))
    codes = [_nearest_e4m3(float(v) * 2.0 ** (-e)) for v in vals]
    return codes, e + 127


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
@pytest.mark.parametrize("K,gk", [(128, 128), (200, 128), (48, 128), (200, 32), (48, 32)])
def test_quant_act_bruteforce(fmt, K, gk):
    x = synth.deepseek_acts(3, K, seed=4)
    xq, s = Q.quant_act(x, gk, fmt)
    xv = F.bf16_decode(x)
    G = -(-K // gk)
    assert xq.shape == (3, K) and s.shape == (3, G)
    for m in range(3):
        for g in range(G):
            vals = xv[m, g * gk:(g + 1) * gk]
            codes, sc = _brute_group(vals, fmt)
            assert list(xq[m, g * gk:(g + 1) * gk]) == codes
            assert s[m, g] == sc


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
def test_quant_weight_bruteforce_partial_blocks(fmt):
    N, K = 130, 272          # partial block on both axes
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=9)
    wq, s = Q.quant_weight(w, 128, 128, fmt)
    assert wq.shape == (N, K) and s.shape == (2, 3)
    wv = F.bf16_decode(w)
    for nb in range(2):
        for kb in range(3):
            blk = wv[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            codes, sc = _brute_group(blk.reshape(-1), fmt)
            got = wq[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].reshape(-1)
            assert list(got) == codes, (nb, kb)
            assert s[nb, kb] == sc


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
def test_quant_weight_bruteforce_block32(fmt):
    N, K = 70, 80            # (32, 32) blocks, partial on both axes
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=8)
    wq, s = Q.quant_weight(w, 32, 32, fmt)
    assert wq.shape == (N, K) and s.shape == (3, 3)
    wv = F.bf16_decode(w)
    for nb in range(3):
        for kb in range(3):
            blk = wv[nb * 32:(nb + 1) * 32, kb * 32:(kb + 1) * 32]
            codes, sc = _brute_group(blk.reshape(-1), fmt)
            got = wq[nb * 32:(nb + 1) * 32, kb * 32:(kb + 1) * 32].reshape(-1)
            assert list(got) == codes, (nb, kb)
            assert s[nb, kb] == sc


def test_float_amax_maps_to_448():
    x = synth.llama_acts(64, 512, seed=1)
    xq, s = Q.quant_act(x, 128, Q.SCALE_FLOAT)
    xv = F.bf16_decode(x).reshape(64, 4, 128)
    codes = xq.reshape(64, 4, 128)
    idx = np.argmax(np.abs(xv), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_ue8m0_scales_pow2_and_amax_in_range():
    x = synth.deepseek_acts(64, 512, seed=2)
    xq, s = Q.quant_act(x, 128, Q.SCALE_UE8M0)
    assert s.dtype == np.uint8 and np.all(s < 255)
    xv = F.bf16_decode(x).reshape(64, 4, 128)
    codes = xq.reshape(64, 4, 128)
    idx = np.argmax(np.abs(xv), axis=-1)
    top = np.abs(F.e4m3_decode(np.take_along_axis(codes, idx[..., None], -1)[..., 0]))
    assert np.all((top >= 224) & (top <= 448))
    # dequantized amax within one e4m3 half-quantum of the true amax
    amax = np.max(np.abs(xv), axis=-1)
    deq = top * np.exp2(s.astype(np.float64) - 127)
    assert np.all(np.abs(deq - amax) <= amax * 2.0 ** -4)


def test_ue8m0_exponent_closed_forms():
    # e = ceil(log2(amax / 448)): 3.5 * 2^7 = 448 exactly; 3.6 needs one more
    cases = {3.5: -7, 3.6: -6, 448.0: 0, 449.0: 1, 224.0: -1, 1.0: -8, 1.75: -8,
             1.76: -7, 0.0: 0, 2.0 ** -140: -127, 3e38: 120}
    for a, e in cases.items():
        assert int(Q.ue8m0_exponent(np.array([a]))[0]) == e, a


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
def test_dequant_error_half_quantum(fmt):
    x = synth.llama_acts(32, 1024, seed=3)
    xq, s = Q.quant_act(x, 128, fmt)
    xv = F.bf16_decode(x)
    sc = np.repeat(Q.dequant_scale(s, fmt), 128, axis=1)
    y = xv / sc                                         # exact-ish ratio
    d = F.e4m3_decode(xq)
    a = np.abs(y)
    _, ex = np.frexp(a)
    quantum = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(ex - 1.0 - 3))
    assert np.all(np.abs(d - y) <= 0.5 * quantum * (1 + 2.0 ** -20) + 1e-30)


def test_row_permutation_commutes():
    x = synth.deepseek_acts(40, 384, seed=5)
    p = np.random.default_rng(0).permutation(40)
    for fmt in (Q.SCALE_FLOAT, Q.SCALE_UE8M0):
        a, sa = Q.quant_act(x, 128, fmt)
        b, sb = Q.quant_act(x[p], 128, fmt)
        assert np.array_equal(a[p], b) and np.array_equal(sa[p], sb)


def test_constant_and_zero_groups():
    c = np.float32(0.3)
    x = _bf(np.full((2, 256), c))
    x[1, 128:] = 0
    xq, s = Q.quant_act(x, 128, Q.SCALE_FLOAT)
    cv = F.bf16_decode(x[0, 0])
    assert np.all(xq[0] == 0x7E) and s[0, 0] == np.float32(np.float32(cv) / np.float32(448))
    assert np.all(xq[1, 128:] == 0) and s[1, 1] == 1.0
    xq, s = Q.quant_act(x, 128, Q.SCALE_UE8M0)
    assert np.all(xq[1, 128:] == 0) and s[1, 1] == 127


def test_negative_zero_and_tiny_negatives_keep_sign():
    x = _bf(np.array([[-0.0, -1e-30, 1e-30, 0.0] + [1.0] * 124]))
    xq, _ = Q.quant_act(x, 128, Q.SCALE_FLOAT)
    assert list(xq[0, :4]) == [0x80, 0x80, 0x00, 0x00]
