"""Pins of oracle/mxfp4.py: the block exponent against a search for the
smallest power of two that fits the group under 6, codes against a
brute-force nearest-value search over the pinned E2M1 table, the
round-trip error bound, and the GEMM against explicit loops."""

import numpy as np

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import mxfp4 as X
from oracle import quant as Q


def _table():
    return np.array([F.e2m1_decode(c) for c in range(16)])


def test_exponent_is_smallest_fitting_power():
    rng = np.random.default_rng(0)
    amax = np.concatenate([rng.random(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           6.0 * np.exp2(np.arange(-20, 20)), [1e-40, 3.0, 6.0, 6.0000001, 12.0]])
    e = X.mx_exponent(amax)
    for a, ee in zip(amax, e):
        k = -127
        while 6.0 * 2.0 ** k < a:
            k += 1
        assert ee == max(-127, min(127, k)), (a, ee, k)
    assert X.mx_exponent(0.0) == 0


def test_codes_brute_force():
    w = synth.normal_bf16((8, 256), 0.015, "nvfp4", "w", seed=3)
    w[0, :32] = 0                                          # zero group
    w[1, 32:64] = synth.f32_to_bf16_bits(np.float32([6.0, -3.0, 1.5, 0.25] * 8))
    packed, sc = X.quant_weight_mxfp4(w)
    codes = F.e2m1_unpack(packed)
    vals = F.bf16_decode(w)
    tab = _table()
    for n in range(8):
        for g in range(8):
            grp = vals[n, 32 * g:32 * g + 32]
            amax = np.max(np.abs(grp))
            k = 0 if amax == 0 else next(k for k in range(-127, 128) if 6.0 * 2.0 ** k >= amax)
            assert sc[n, g] == k + 127
            for j, v in enumerate(grp):
                y = v * 2.0 ** -k
                d = np.abs(tab[:8] - abs(y))
                best = np.flatnonzero(d == d.min())
                # ties: the even code (mantissa bit 0)
                mag = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                want = mag | (8 if np.signbit(y) else 0)
                assert codes[n, 32 * g + j] == want, (n, g, j, v, y)
    assert sc[0, 0] == 127 and not codes[0, :32].any()
    # the hand group: amax 6 -> e = 0, codes exact
    assert sc[1, 1] == 127
    assert np.array_equal(F.e2m1_decode(codes[1, 32:64]), np.array([6.0, -3.0, 1.5, 0.0] * 8))


def test_roundtrip_bound():
    w = synth.normal_bf16((64, 512), 0.015, "nvfp4", "w", seed=4)
    packed, sc = X.quant_weight_mxfp4(w)
    back = X.dequant_mxfp4(packed, sc)
    orig = F.bf16_decode(w)
    s = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    # E2M1 quanta: 0.5 below 2, 1 below 4, 2 up to 6 (times the scale)
    q = np.where(np.abs(orig) / s < 2, 0.5, np.where(np.abs(orig) / s < 4, 1.0, 2.0)) * s
    assert np.all(np.abs(back - orig) <= q / 2 + 1e-30)
    assert np.all(np.max(np.abs(orig).reshape(64, -1, 32), axis=-1) <= 6 * s[:, ::32])


def test_gemm_loops():
    M, N, K = 3, 5, 256
    x = synth.normal_bf16((M, K), 1.0, "nvfp4", "x", seed=5)
    w = synth.normal_bf16((N, K), 0.015, "nvfp4", "w", seed=6)
    for fmt in (0, 1):
        xq, xs = Q.quant_act(x, 128, fmt)
        wq, ws = X.quant_weight_mxfp4(w)
        ref = X.fp8_fp4_gemm(xq, xs, wq, ws, fmt=fmt)
        wc = F.e2m1_unpack(wq)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    sa = float(xs[m, k // 128]) if fmt == 0 else 2.0 ** (int(xs[m, k // 128]) - 127)
                    sw = 2.0 ** (int(ws[n, k // 32]) - 127)
                    acc += F.e4m3_decode(xq[m, k]) * sa * F.e2m1_decode(wc[n, k]) * sw
                assert abs(acc - ref[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_grouped_matches_per_row_loops():
    """Grouped FP8 x MXFP4 experts: each row against an explicit loop over
    its own expert's dequantized weights (empty experts included); swapping
    two experts' weights changes exactly their rows."""
    E, N, K = 4, 3, 64
    counts = np.array([2, 0, 3, 1])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.normal_bf16((T, K), 1.0, "moe", "x", seed=7)
    wq = np.empty((E, N, K // 2), np.uint8)
    ws = np.empty((E, N, K // 32), np.uint8)
    for e in range(E):
        wq[e], ws[e] = X.quant_weight_mxfp4(synth.normal_bf16((N, K), 0.01, "moe", "w", e, seed=7))
    for fmt in (0, 1):
        xq, xs = Q.quant_act(x, 128, fmt)
        Y = X.grouped_fp8_fp4_gemm(xq, xs, wq, ws, off, fmt=fmt)
        for r in range(T):
            e = int(np.searchsorted(off, r, side="right") - 1)
            wc = F.e2m1_unpack(wq[e])
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    sa = float(xs[r, k // 128]) if fmt == 0 else 2.0 ** (int(xs[r, k // 128]) - 127)
                    sw = 2.0 ** (int(ws[e, n, k // 32]) - 127)
                    acc += F.e4m3_decode(xq[r, k]) * sa * F.e2m1_decode(wc[n, k]) * sw
                assert abs(acc - Y[r, n]) <= 1e-12 * max(1.0, abs(acc)), (fmt, r, n)
        sw_ = wq.copy()
        sw_[[0, 2]] = sw_[[2, 0]]
        ss_ = ws.copy()
        ss_[[0, 2]] = ss_[[2, 0]]
        Y2 = X.grouped_fp8_fp4_gemm(xq, xs, sw_, ss_, off, fmt=fmt)
        changed = np.flatnonzero(np.any(Y2 != Y, axis=1))
        assert set(changed) <= set(range(off[0], off[1])) | set(range(off[2], off[3]))
        assert len(changed) == counts[0] + counts[2]
