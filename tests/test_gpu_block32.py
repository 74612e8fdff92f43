"""GPU parity at (32, 32) weight blocks with 1 x 32 activation groups (a
non-default weight_block_size the fine-grained FP8 guide lists, section 九):
quantizer codes and scales bit-exact, dequantization bit-exact, and the GEMM
(its own kernel, one promotion per 32-wide K group) within 2e-3 relative
Frobenius error of the oracle's fp64 block-by-block product."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import convert as C
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q

from gpu_util import to_dev, to_dev_bf16, bf16_bits, u8, empty_u8, guard_intact, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _sdt(fmt):
    import torch
    return torch.float32 if fmt == 0 else torch.uint8


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K", [(1, 48), (7, 208), (33, 4096), (300, 1040)])
def test_quant_act_group32(M, K, fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"act quant 1x32 M={M} K={K} fmt={fmt}")
    x = synth.deepseek_acts(M, K, seed=K) if fmt else synth.llama_acts(M, K, seed=K)
    x[0, :32] = 0                                         # a zero group
    xq, full = empty_u8((M, K))
    xs = torch.full((M, -(-K // 32)), 3, dtype=_sdt(fmt), device="cuda")
    L.fp8_quant_act(to_dev_bf16(x), xq, xs, group_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    rq, rs = Q.quant_act(x, 32, fmt)
    assert guard_intact(full, M * K)
    assert np.array_equal(u8(xq), rq) and np.array_equal(xs.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("N,K", [(70, 80), (300, 1040), (4096, 4096)])
def test_quant_weight_block32(N, K, fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"weight quant 32x32 N={N} K={K} fmt={fmt}")
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N)
    w[:32, :32] = 0                                       # a zero block
    wq, full = empty_u8((N, K))
    ws = torch.full((-(-N // 32), -(-K // 32)), 3, dtype=_sdt(fmt), device="cuda")
    L.fp8_quant_weight(to_dev_bf16(w), wq, ws, block_n=32, block_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    rq, rs = Q.quant_weight(w, 32, 32, fmt)
    assert guard_intact(full, N * K)
    assert np.array_equal(u8(wq), rq), f"{np.count_nonzero(u8(wq) != rq)} code mismatches"
    assert np.array_equal(ws.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequant_block32(fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    N, K = 100, 208
    wq, ws = Q.quant_weight(synth.normal_bf16((N, K), 0.02, "llama", "w", seed=5), 32, 32, fmt)
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    L.fp8_dequant_weight(to_dev(wq), to_dev(ws), out, block_n=32, block_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), C.dequant_weight_bf16(wq, ws, 32, 32, fmt))


def _gemm(M, N, K, fmt, bias, seed):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    x = synth.deepseek_acts(M, K, seed=seed) if fmt else synth.llama_acts(M, K, seed=seed)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=seed + 1)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=seed) if bias else None
    xq, xs = Q.quant_act(x, 32, fmt)
    wq, ws = Q.quant_weight(w, 32, 32, fmt)
    yf = torch.full((M * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yf[:M * N].view(M, N)
    L.fp8_block_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), y,
                     bias=None if b is None else to_dev_bf16(b), block_n=32, block_k=32,
                     scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(yf[M * N:].float()).all(), "wrote past the output"
    got = F.bf16_decode(bf16_bits(y))
    ref = G.block_gemm(xq, xs, wq, ws, None if b is None else F.bf16_decode(b), 32, 32, fmt)
    return got, ref, (x, w, b)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,bias", [
    (1, 256, 256, False), (16, 264, 400, True), (130, 520, 640, False), (300, 1000, 1040, True),
    (257, 136, 4112, False), (5, 136, 4112, True),
    (260, 264, 2048, True),    # two staged chunks of UE8M0 scales (K a multiple of 128)
])
def test_block32_gemm_parity(M, N, K, bias, fmt):
    say(f"gemm 32x32 M={M} N={N} K={K} fmt={fmt}")
    got, ref, _ = _gemm(M, N, K, fmt, bias, seed=M + K)
    assert np.isfinite(got).all(), "unwritten outputs"
    err = rel_fro(got, ref)
    say(f"  rel fro {err:.3e}  vs bf16(ref) {rel_fro(got, F.bf16_round(ref)):.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
def test_block32_linear_equals_quant_then_gemm(fmt):
    """fp8_linear with (32, 32) blocks returns the same bf16 bits as
    fp8_quant_act (1 x 32) followed by fp8_block_gemm."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, N, K = 40, 264, 528
    got, _, (x, w, b) = _gemm(M, N, K, fmt, True, seed=9)
    wq, ws = Q.quant_weight(w, 32, 32, fmt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_linear(to_dev_bf16(x), to_dev(wq), to_dev(ws), y, bias=to_dev_bf16(b), block_n=32,
                 block_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(F.bf16_decode(bf16_bits(y)), got)


@pytest.mark.parametrize("fmt", [0, 1])
def test_block32_gemm_full_size_sampled(fmt):
    """Llama-3-8B o_proj shape at M = 2048 with (32, 32) blocks (fp32 scales;
    UE8M0 scales run the scaled-MFMA form); the oracle recomputes 2048
    sampled outputs."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, N, K = 2048, 4096, 4096
    say(f"gemm 32x32 full size M={M} N={N} K={K} fmt={fmt}")
    x = synth.llama_acts(M, K, seed=1)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=2)
    sdt = torch.uint8 if fmt else torch.float32
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 32), dtype=sdt, device="cuda")
    wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((N // 32, K // 32), dtype=sdt, device="cuda")
    L.fp8_quant_act(to_dev_bf16(x), xq, xs, group_k=32, scale_fmt=fmt)
    L.fp8_quant_weight(to_dev_bf16(w), wq, ws, block_n=32, block_k=32, scale_fmt=fmt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_block_gemm(xq, xs, wq, ws, y, block_n=32, block_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    rows, cols = g.integers(0, M, 2048), g.integers(0, N, 2048)
    hxq, hxs = Q.quant_act(x, 32, fmt)
    hwq, hws = Q.quant_weight(w, 32, 32, fmt)
    assert np.array_equal(u8(xq), hxq) and np.array_equal(u8(wq), hwq)
    ref = G.block_gemm_rows(hxq, hxs, hwq, hws, rows, cols, block_n=32, block_k=32, fmt=fmt)
    got = F.bf16_decode(bf16_bits(y))[rows, cols]
    err = rel_fro(got, ref)
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("counts,N,K", [
    ([3, 0, 1, 6, 2], 128, 256),
    ([0, 0, 130, 0, 1, 257, 64, 0], 200, 1040),   # ragged N and K, partial M tiles
    ([300], 264, 512),
    (list(np.random.default_rng(6).integers(0, 40, 33)), 384, 640),
])
def test_grouped_gemm_block32(counts, N, K, fmt):
    """MoE experts with (32, 32) weight blocks and 1 x 32 activation groups
    against the oracle's per-expert block-by-block product; empty experts,
    ragged N and K."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    say(f"grouped (32, 32) E={E} T={T} N={N} K={K} fmt={fmt}")
    x = synth.deepseek_acts(T, K, seed=K) if fmt else synth.llama_acts(T, K, seed=K)
    xq, xs = Q.quant_act(x, 32, fmt)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, -(-N // 32), -(-K // 32)), np.float32 if fmt == 0 else np.uint8)
    for e in range(E):
        wq[e], ws[e] = Q.quant_weight(synth.normal_bf16((N, K), 0.02, "moe", "w", e, seed=K),
                                      32, 32, fmt)
    yf = torch.full((T * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yf[:T * N].view(T, N)
    L.fp8_grouped_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off), y,
                       block_n=32, block_k=32, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(yf[T * N:].float()).all(), "wrote past the output"
    got = F.bf16_decode(bf16_bits(y))
    assert np.isfinite(got).all(), "unwritten rows"
    err = rel_fro(got, G.grouped_gemm(xq, xs, wq, ws, off, 32, 32, fmt))
    say(f"  rel fro {err:.3e}")
    assert err <= TOL
