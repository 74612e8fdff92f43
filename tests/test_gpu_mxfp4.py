"""GPU parity of the MXFP4 weight quantizer (codes and UE8M0 group scales
bit-exact) and of the FP8 x FP4 GEMM (within 2e-3 relative Frobenius error
of the oracle's fp64 product of the dequantized operands)."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import mxfp4 as X
from oracle import quant as Q

from gpu_util import to_dev, to_dev_bf16, bf16_bits, u8, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _quant_dev(w_bits):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    N, K = w_bits.shape
    wd = to_dev_bf16(w_bits)
    q = torch.full((N, K // 2), 0xEE, dtype=torch.uint8, device=wd.device)
    s = torch.full((N, K // 32), 0xEE, dtype=torch.uint8, device=wd.device)
    L.mxfp4_quant_weight(wd, q, s)
    torch.cuda.synchronize()
    return u8(q), u8(s)


@pytest.mark.parametrize("N,K,sigma,seed", [(1, 32, 0.015, 0), (37, 4096, 0.015, 1),
                                            (300, 1056, 1.0, 2), (8, 28672, 0.015, 3)])
def test_mxfp4_quant_parity(N, K, sigma, seed):
    say(f"mxfp4 quant N={N} K={K}")
    w = synth.normal_bf16((N, K), sigma, "nvfp4", "w", seed=seed)
    q, s = _quant_dev(w)
    rq, rs = X.quant_weight_mxfp4(w)
    assert np.array_equal(s, rs), f"{np.count_nonzero(s != rs)} scale mismatches"
    assert np.array_equal(q, rq), f"{np.count_nonzero(q != rq)} code-byte mismatches"


def test_mxfp4_quant_edges():
    w = synth.normal_bf16((4, 128), 0.015, "nvfp4", "w", seed=4)
    w[0, :32] = 0                                             # zero group
    w[0, 32:64] = 0x8000                                      # negative zeros
    w[1, :32] = np.arange(1, 33, dtype=np.uint16)             # bf16 subnormals
    w[1, 32:64] = synth.f32_to_bf16_bits(np.float32([3e38, -1e38] * 16))
    w[2, :32] = synth.f32_to_bf16_bits(np.float32([6.0, -0.25, 0.75, 2.5] * 8))   # ties at e = 0
    q, s = _quant_dev(w)
    rq, rs = X.quant_weight_mxfp4(w)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


def _gemm(M, N, K, fmt, bias=False, seed=0):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    x = synth.deepseek_acts(M, K, seed=seed) if fmt else synth.llama_acts(M, K, seed=seed)
    w = synth.normal_bf16((N, K), 0.015, "nvfp4", "w", seed=seed + 1)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=seed) if bias else None
    xq, xs = Q.quant_act(x, 128, fmt)
    wq, ws = X.quant_weight_mxfp4(w)
    yf = torch.full((M * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yf[:M * N].view(M, N)
    L.fp8_fp4_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), y,
                   bias=None if b is None else to_dev_bf16(b), scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(yf[M * N:].float()).all(), "wrote past the output"
    got = F.bf16_decode(bf16_bits(y))
    ref = X.fp8_fp4_gemm(xq, xs, wq, ws, bias=None if b is None else F.bf16_decode(b), fmt=fmt)
    return got, ref


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,bias", [
    (1, 256, 256, False), (5, 264, 288, True), (16, 1000, 1024, False), (17, 520, 4128, True),
    (64, 256, 2048, False), (130, 520, 640, True), (300, 1000, 1056, False), (1024, 1024, 1024, True),
    (4100, 4104, 384, True),     # 256 x 256 tiles, ragged in M, N and K
    (4100, 4104, 512, False),    # 256 x 256 tiles, dword-aligned UE8M0 scale rows (staged)
])
def test_fp8_fp4_gemm_parity(M, N, K, bias, fmt):
    say(f"fp8 x fp4 gemm M={M} N={N} K={K} fmt={fmt}")
    got, ref = _gemm(M, N, K, fmt, bias, seed=M + N)
    assert np.isfinite(got).all(), "unwritten outputs"
    err = rel_fro(got, ref)
    say(f"  rel fro {err:.3e}  vs bf16(ref) {rel_fro(got, F.bf16_round(ref)):.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,K,N,fmt", [(1, 7168, 18432, 1), (16, 4096, 28672, 0), (4096, 7168, 4096, 1)])
def test_fp8_fp4_gemm_full_size_sampled(M, K, N, fmt):
    """Full-size shapes; the oracle recomputes 2048 sampled outputs."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"fp8 x fp4 full-size M={M} K={K} N={N} fmt={fmt}")
    x = synth.deepseek_acts(M, K, seed=2) if fmt else synth.llama_acts(M, K, seed=2)
    wdev = synth.device_normal_bf16((N, K), 0.015, "nvfp4", "w", index=N)
    xd = to_dev_bf16(x)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=sdt, device="cuda")
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.mxfp4_quant_weight(wdev, wq, ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_fp4_gemm(xq, xs, wq, ws, y, scale_fmt=fmt)
    torch.cuda.synchronize()
    g = np.random.default_rng(M + N)
    rows, cols = g.integers(0, M, 2048), g.integers(0, N, 2048)
    ur, uc = np.unique(rows), np.unique(cols)
    hx, hxs = Q.quant_act(x[ur], 128, fmt)
    hw, hws = X.quant_weight_mxfp4(bf16_bits(wdev)[uc])
    from oracle import gemm as G
    A = G.dequant_act(hx, hxs, 128, fmt)
    B = X.dequant_mxfp4(hw, hws)
    ref = np.einsum("ik,ik->i", A[np.searchsorted(ur, rows)], B[np.searchsorted(uc, cols)])
    got = F.bf16_decode(bf16_bits(y))[rows, cols]
    err = rel_fro(got, ref)
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL
    # the device-quantized weights of the sampled rows equal the oracle's
    assert np.array_equal(u8(wq)[uc], hw) and np.array_equal(u8(ws)[uc], hws)


def _grouped_w4_case(counts, N, K, fmt, seed):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.deepseek_acts(T, K, seed=seed) if fmt else synth.llama_acts(T, K, seed=seed)
    xq, xs = Q.quant_act(x, 128, fmt)
    wq = np.empty((E, N, K // 2), np.uint8)
    ws = np.empty((E, N, K // 32), np.uint8)
    for e in range(E):
        wq[e], ws[e] = X.quant_weight_mxfp4(synth.normal_bf16((N, K), 0.01, "moe", "w", e,
                                                              seed=seed))
    yf = torch.full((T * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yf[:T * N].view(T, N)
    L.fp8_fp4_grouped_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off), y,
                           scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(yf[T * N:].float()).all(), "wrote past the output"
    got = F.bf16_decode(bf16_bits(y))
    assert np.isfinite(got).all(), "unwritten rows"
    return rel_fro(got, X.grouped_fp8_fp4_gemm(xq, xs, wq, ws, off, fmt=fmt))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("counts,N,K", [
    ([3, 0, 1, 6, 2], 256, 256),
    ([0, 0, 130, 0, 1, 257, 64, 0], 512, 640),     # both tile classes, K % 128 == 0
    ([300], 264, 1056),                            # ragged N, K % 128 != 0 (per-block scales)
    ([0, 300, 5, 140], 384, 1024),                 # large experts, dword-aligned UE8M0 rows
    ([0, 129, 0, 0], 256, 288),                    # one large expert, ragged K
    (list(np.random.default_rng(5).integers(0, 40, 33)), 384, 512),
])
def test_fp8_fp4_grouped_gemm_parity(counts, N, K, fmt):
    """MoE experts with MXFP4 weights against the oracle's per-expert
    FP8 x FP4 product; both expert classes (more / at most 128 rows), empty
    experts, ragged N and K."""
    say(f"fp8 x fp4 grouped E={len(counts)} T={sum(counts)} N={N} K={K} fmt={fmt}")
    err = _grouped_w4_case(counts, N, K, fmt, seed=len(counts) + K)
    say(f"  rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_fp4_grouped_moe_shape_sampled(fmt):
    """The MoE gate/up shape (256 experts, 7168 -> 4096, 4096 tokens x top-8
    Zipf routing) with MXFP4 expert weights; the oracle recomputes sampled
    rows of the largest, the smallest and two other experts."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E, N, K, TOK, TOPK = 256, 4096, 7168, 4096, 8
    tok, off = synth.moe_routing(TOK, E, TOPK)
    T = len(tok)
    say(f"fp8 x fp4 moe shape T={T} fmt={fmt}")
    x = synth.deepseek_acts(TOK, K, seed=9) if fmt else synth.normal_bf16((TOK, K), 1.0, "moe", "x")
    xd = to_dev_bf16(x)[torch.from_numpy(tok).cuda()]
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 128), dtype=sdt, device="cuda")
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    wq = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
    for e in range(E):
        wb = synth.device_normal_bf16((N, K), 0.01, "moe", "w", e)
        L.mxfp4_quant_weight(wb, wq[e], ws[e])
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_fp4_grouped_gemm(xq, xs, wq, ws, to_dev(off), y, scale_fmt=fmt)
    torch.cuda.synchronize()
    counts = np.diff(off)
    experts = [int(np.argmax(counts)), int(np.argmin(counts)), 17, 200]
    g = np.random.default_rng(fmt)
    from oracle import gemm as G
    got_all, ref_all = [], []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = g.integers(lo, hi, 8)
        cols = g.integers(0, N, 64)
        hx, hxs = Q.quant_act(x[tok[rows]], 128, fmt)            # the oracle's own codes
        wb = synth.device_normal_bf16((N, K), 0.01, "moe", "w", e)
        hw, hws = X.quant_weight_mxfp4(bf16_bits(wb)[cols])
        assert np.array_equal(u8(wq[e])[cols], hw) and np.array_equal(u8(ws[e])[cols], hws)
        ref = G.dequant_act(hx, hxs, 128, fmt) @ X.dequant_mxfp4(hw, hws).T
        got = F.bf16_decode(bf16_bits(y[torch.from_numpy(rows).cuda()]))[:, cols]
        got_all.append(got.ravel())
        ref_all.append(ref.ravel())
    err = rel_fro(np.concatenate(got_all), np.concatenate(ref_all))
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL
