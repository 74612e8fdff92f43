"""GPU parity of the static activation scheme, weight dequantization and the
fp32 -> UE8M0 scale conversion against oracle/convert.py (bit-exact)."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import convert as C
from oracle import gemm as G
from oracle import quant as Q

from gpu_util import to_dev, to_dev_bf16, bf16_bits, u8, rel_fro, say

pytestmark = pytest.mark.gpu


def _static_dev(x_bits, scale, fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, K = x_bits.shape
    G_ = -(-K // 128)
    xd = to_dev_bf16(x_bits)
    xq = torch.full((M, K), 0xEE, dtype=torch.uint8, device=xd.device)
    if fmt == 0:
        xs = torch.full((M, G_), float("nan"), dtype=torch.float32, device=xd.device)
        xs.view(-1)[0] = float(scale)
    else:
        xs = torch.full((M, G_), 0xEE, dtype=torch.uint8, device=xd.device)
        xs.view(-1)[0] = int(scale)
    L.fp8_quant_act(xd, xq, xs, act_scheme=L.ACT_STATIC, scale_fmt=fmt)
    torch.cuda.synchronize()
    return u8(xq), xs.cpu().numpy()


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K,seed", [(1, 128, 0), (37, 272, 1), (300, 4096, 2), (8, 14336, 3)])
def test_static_quant_parity(M, K, seed, fmt):
    say(f"static quant M={M} K={K} fmt={fmt}")
    x = synth.llama_acts(M, K, seed=seed)
    scale = np.float32(0.0123) if fmt == 0 else np.uint8(122)
    q, s = _static_dev(x, scale, fmt)
    rq, rs = C.quant_act_static(x, scale, fmt=fmt)
    assert np.array_equal(q, rq), f"{np.count_nonzero(q != rq)} code mismatches"
    assert np.array_equal(s.view(np.uint8) if fmt else s.view(np.uint32),
                          rs.view(np.uint8) if fmt else rs.view(np.uint32))


def test_static_quant_edges():
    x = synth.f32_to_bf16_bits(np.float32([[1000.0, -1000.0, 0.0, -0.0, 448.0, 0.5] + [1e-30] * 10]))
    for fmt, scale in ((0, np.float32(1.0)), (0, np.float32(3.7)), (1, np.uint8(128)), (1, np.uint8(100))):
        q, _ = _static_dev(x, scale, fmt)
        rq, _ = C.quant_act_static(x, scale, fmt=fmt)
        assert np.array_equal(q, rq)


@pytest.mark.parametrize("fmt", [0, 1])
def test_static_quant_feeds_gemm(fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, K, N = 64, 640, 264
    x = synth.llama_acts(M, K, seed=9)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=9)
    scale = np.float32(0.35) if fmt == 0 else np.uint8(126)
    q, s = _static_dev(x, scale, fmt)
    wq, ws = Q.quant_weight(w, fmt=fmt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_block_gemm(to_dev(q), to_dev(s), to_dev(wq), to_dev(ws), y, scale_fmt=fmt)
    torch.cuda.synchronize()
    from oracle import formats as F
    rq, rs = C.quant_act_static(x, scale, fmt=fmt)
    ref = G.block_gemm(rq, rs, wq, ws, fmt=fmt)
    assert rel_fro(F.bf16_decode(bf16_bits(y)), ref) <= 2e-3


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("N,K", [(1, 16), (130, 272), (256, 4096), (4096, 14336)])
def test_dequant_weight_parity(N, K, fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"dequant N={N} K={K} fmt={fmt}")
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N)
    wq, ws = Q.quant_weight(w, fmt=fmt)
    if N == 130:                           # every finite code, scales spread wide
        rng = np.random.default_rng(1)
        wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
        wq[(wq & 0x7F) == 0x7F] = 0x7E
        ws = (rng.random(ws.shape).astype(np.float32) * 4 + 1e-3) if fmt == 0 else \
            rng.integers(0, 255, ws.shape).astype(np.uint8)
    out = torch.full((N * K + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    L.fp8_dequant_weight(to_dev(wq), to_dev(ws), out[:N * K].view(torch.bfloat16).view(N, K),
                         scale_fmt=fmt)
    torch.cuda.synchronize()
    assert (out[N * K:] == 0x5A5A).all(), "wrote past the output"
    got = out[:N * K].cpu().numpy().view(np.uint16).reshape(N, K)
    ref = C.dequant_weight_bf16(wq, ws, fmt=fmt)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} mismatches"


def test_scale_to_ue8m0_parity():
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    k = np.arange(-127, 128)
    pw = np.ldexp(np.float32(1.0), k).astype(np.float32)
    rng = np.random.default_rng(2)
    other = np.concatenate([np.float32([0.0, -0.0, -2.0, np.inf, -np.inf, np.nan, 2.0 ** -128,
                                        2.0 ** -149, 3.0, 1.5]),
                            rng.standard_normal(5000).astype(np.float32),
                            rng.integers(0, 2 ** 32, 5000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    s = np.concatenate([pw, other]).astype(np.float32)
    out = torch.full((s.size,), 0x33, dtype=torch.uint8, device="cuda")
    L.fp8_scale_to_ue8m0(to_dev(s), out)
    torch.cuda.synchronize()
    assert np.array_equal(u8(out), C.pow2_to_ue8m0(s))
