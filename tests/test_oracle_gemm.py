"""Pins for the oracle's GEMMs: brute-force loops in the per-K-block form,
closed forms, and the bf16 output-rounding floor."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from oracle import fp4 as P


def _brute_block_gemm(xq, xs, wq, ws, bias, fmt, blk=128):
    """Y[m,n] = sum_kb S_a[m,kb] S_w[n//blk,kb] sum_{k in kb} dec(xq) dec(wq),
    plain Python loops over every index (the block-by-block form)."""
    M, K = xq.shape
    N = wq.shape[0]
    dx = F.e4m3_decode(xq)
    dw = F.e4m3_decode(wq)
    sa = Q.dequant_scale(xs, fmt)
    sw = Q.dequant_scale(ws, fmt)
    Y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for kb in range(-(-K // blk)):
                part = 0.0
                for k in range(kb * blk, min(K, kb * blk + blk)):
                    part += float(dx[m, k]) * float(dw[n, k])
                tot += float(sa[m, kb]) * float(sw[n // blk, kb]) * part
            Y[m, n] = tot + (0.0 if bias is None else float(bias[n]))
    return Y


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
@pytest.mark.parametrize("shape", [(3, 5, 256), (2, 130, 144)])
def test_block_gemm_bruteforce(fmt, shape):
    M, N, K = shape
    x = synth.deepseek_acts(M, K, seed=1)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=1)
    xq, xs = Q.quant_act(x, 128, fmt)
    wq, ws = Q.quant_weight(w, 128, 128, fmt)
    bias = F.bf16_decode(synth.normal_bf16((N,), 0.5, "llama", "bias", seed=1))
    Y = G.block_gemm(xq, xs, wq, ws, bias, fmt=fmt)
    R = _brute_block_gemm(xq, xs, wq, ws, bias, fmt)
    assert np.allclose(Y, R, rtol=1e-12, atol=1e-12 * np.abs(R).max())


@pytest.mark.parametrize("fmt", [Q.SCALE_FLOAT, Q.SCALE_UE8M0])
def test_block_gemm_bruteforce_block32(fmt):
    """(32, 32) weight blocks with 1 x 32 act groups, partial on every axis."""
    M, N, K = 3, 40, 80
    x = synth.deepseek_acts(M, K, seed=2)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=2)
    xq, xs = Q.quant_act(x, 32, fmt)
    wq, ws = Q.quant_weight(w, 32, 32, fmt)
    assert xs.shape == (M, 3) and ws.shape == (2, 3)
    Y = G.block_gemm(xq, xs, wq, ws, None, 32, 32, fmt=fmt)
    R = _brute_block_gemm(xq, xs, wq, ws, None, fmt, blk=32)
    assert np.allclose(Y, R, rtol=1e-12, atol=1e-12 * np.abs(R).max())


def test_block_gemm_rows_matches_full():
    M, N, K = 6, 260, 384
    x = synth.llama_acts(M, K, seed=2)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=2)
    xq, xs = Q.quant_act(x)
    wq, ws = Q.quant_weight(w)
    Y = G.block_gemm(xq, xs, wq, ws)
    rows = np.array([0, 5, 3, 1])
    cols = np.array([0, 259, 128, 7])
    assert np.allclose(G.block_gemm_rows(xq, xs, wq, ws, rows, cols), Y[rows, cols],
                       rtol=1e-12)


def test_block_gemm_constant_closed_form():
    # X = c everywhere, W = d everywhere: every group/block is constant, codes
    # are all 0x7E (448) and Y = K * (448 s_a) * (448 s_w).
    M, N, K = 4, 256, 384
    c, d = np.float32(1.3), np.float32(-0.07)
    x = synth.f32_to_bf16_bits(np.full((M, K), c))
    w = synth.f32_to_bf16_bits(np.full((N, K), d))
    xq, xs = Q.quant_act(x)
    wq, ws = Q.quant_weight(w)
    assert np.all(xq == 0x7E) and np.all(wq == 0xFE)
    Y = G.block_gemm(xq, xs, wq, ws)
    expect = K * (448.0 * float(xs[0, 0])) * (-448.0 * float(ws[0, 0]))
    assert np.allclose(Y, expect, rtol=1e-15)


def test_block_gemm_ue8m0_pow2_exact():
    # Powers of two are exact under UE8M0 scaling, so Y is the exact integer
    # combination of the inputs.
    g = np.random.default_rng(0)
    M, N, K = 3, 128, 256
    xv = np.ldexp(np.where(g.random((M, K)) < 0.5, -1.0, 1.0), g.integers(-6, 3, (M, K)))
    wv = np.ldexp(np.where(g.random((N, K)) < 0.5, -1.0, 1.0), g.integers(-9, -3, (N, K)))
    x = synth.f32_to_bf16_bits(xv.astype(np.float32))
    w = synth.f32_to_bf16_bits(wv.astype(np.float32))
    xq, xs = Q.quant_act(x, fmt=Q.SCALE_UE8M0)
    wq, ws = Q.quant_weight(w, fmt=Q.SCALE_UE8M0)
    Y = G.block_gemm(xq, xs, wq, ws, fmt=Q.SCALE_UE8M0)
    assert np.array_equal(Y, xv @ wv.T)


def test_grouped_gemm_matches_per_row_lookup():
    E, N, K = 5, 128, 256
    counts = np.array([3, 0, 1, 6, 2])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.normal_bf16((T, K), 1.0, "moe", "x", seed=3)
    xq, xs = Q.quant_act(x)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, 1, 2), np.float32)
    for e in range(E):
        wq[e], ws[e] = Q.quant_weight(synth.normal_bf16((N, K), 0.02, "moe", "w", e, seed=3))
    Y = G.grouped_gemm(xq, xs, wq, ws, off)
    ref = np.empty((T, N))
    for r in range(T):
        e = int(np.searchsorted(off, r, side="right") - 1)
        ref[r] = _brute_block_gemm(xq[r:r + 1], xs[r:r + 1], wq[e], ws[e], None, 0)[0]
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-13)


def test_bf16_output_floor_below_budget():
    # Rounding the exact product to bf16 must leave room inside the 2e-3
    # relative-Frobenius acceptance budget.
    M, N, K = 16, 256, 256
    x = synth.normal_bf16((M, K), 1.0, "single", "x")
    w = synth.normal_bf16((N, K), 0.02, "single", "w")
    xq, xs = Q.quant_act(x)
    wq, ws = Q.quant_weight(w)
    Y = G.block_gemm(xq, xs, wq, ws)
    err = np.linalg.norm(F.bf16_round(Y) - Y) / np.linalg.norm(Y)
    assert 1e-3 < err < 2e-3


# ---------------------------------------------------------------- FP4

def test_fp4_invariants():
    x = synth.normal_bf16((8, 256), 1.0, "nvfp4", "x")
    q, sg, g = P.quant_fp4(x)
    xv = F.bf16_decode(x).astype(np.float32)
    assert g == np.float32(np.float32(np.abs(xv).max()) / np.float32(2688.0))
    # the group holding the tensor amax gets the largest E4M3 scale
    r, c = np.unravel_index(np.argmax(np.abs(xv)), xv.shape)
    assert sg[r, c // 16] == 0x7E
    # every group with a normal scale maps its amax element to +-6
    codes = F.e2m1_unpack(q).reshape(8, 16, 16)
    idx = np.argmax(np.abs(xv.reshape(8, 16, 16)), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    normal = (sg & 0x78) != 0
    assert np.all((top[normal] & 0x7) == 0x7)


def test_fp4_bruteforce_codes():
    x = synth.normal_bf16((3, 64), 1.0, "nvfp4", "x", seed=4)
    q, sg, g = P.quant_fp4(x)
    xv = F.bf16_decode(x)
    dec2 = F.e2m1_decode(np.arange(16))
    nib = F.e2m1_unpack(q)
    for r in range(3):
        for j in range(4):
            grp = [float(np.float32(v)) for v in xv[r, j * 16:(j + 1) * 16]]
            a = max(abs(v) for v in grp)
            den = np.float32(np.float32(6.0) * g)
            sc = _nearest_scale(float(np.float32(np.float32(a) / den)))
            assert sg[r, j] == sc
            eff = np.float32(np.float32(F.e4m3_decode(np.array([sc]))[0]) * g)
            for i, v in enumerate(grp):
                y = float(np.float32(np.float32(v) / eff))
                best = None
                for c in range(16):
                    if np.signbit(dec2[c]) != np.signbit(y):
                        continue
                    d = abs(dec2[c] - y)
                    if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                        best = (d, c)
                assert nib[r, j * 16 + i] == best[1]


def _nearest_scale(v):
    dec = F.e4m3_decode(np.arange(128))
    best = None
    for c in range(127):
        d = abs(dec[c] - v)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def test_fp4_zero_tensor_and_zero_group():
    x = np.zeros((2, 32), np.uint16)
    q, sg, g = P.quant_fp4(x)
    assert g == 1.0 and not q.any() and not sg.any()
    x = synth.normal_bf16((2, 32), 1.0, "nvfp4", "x", seed=1)
    x[1, 16:] = 0
    q, sg, g = P.quant_fp4(x)
    assert sg[1, 1] == 0 and not F.e2m1_unpack(q)[1, 16:].any()


def test_fp4_gemm_bruteforce():
    M, N, K = 3, 4, 64
    x = synth.normal_bf16((M, K), 1.0, "nvfp4", "x", seed=6)
    w = synth.normal_bf16((N, K), 0.015, "nvfp4", "w", seed=6)
    xq, xs, xg = P.quant_fp4(x)
    wq, ws, wg = P.quant_fp4(w)
    Y = P.fp4_gemm(xq, xs, xg, wq, ws, wg)
    ax = F.e2m1_decode(F.e2m1_unpack(xq))
    aw = F.e2m1_decode(F.e2m1_unpack(wq))
    sx = F.e4m3_decode(xs)
    sw = F.e4m3_decode(ws)
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for gi in range(K // 16):
                part = sum(float(ax[m, k]) * float(aw[n, k]) for k in range(gi * 16, gi * 16 + 16))
                tot += float(sx[m, gi]) * float(sw[n, gi]) * part
            assert np.isclose(Y[m, n], tot * float(xg) * float(wg), rtol=1e-12)
