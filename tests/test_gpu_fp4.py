"""GPU parity of the NVFP4-style path against the oracle: E2M1 codes, E4M3
group scales and the fp32 tensor scale bit-exact; the FP4 GEMM within 2e-3
relative Frobenius error of the fp64 product of the dequantized operands."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import fp4 as P

from gpu_util import to_dev, to_dev_bf16, bf16_bits, u8, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _quant_dev(x_bits, g=None):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    R, K = x_bits.shape
    xd = to_dev_bf16(x_bits)
    q = torch.full((R, K // 2), 0xEE, dtype=torch.uint8, device=xd.device)
    s = torch.full((R, K // 16), 0xEE, dtype=torch.uint8, device=xd.device)
    if g is None:
        t = torch.full((1,), float("nan"), dtype=torch.float32, device=xd.device)
        L.fp4_quant(xd, q, s, t, dynamic_tscale=1)
    else:
        t = torch.tensor([g], dtype=torch.float32, device=xd.device)
        L.fp4_quant(xd, q, s, t, dynamic_tscale=0)
    torch.cuda.synchronize()
    return u8(q), u8(s), np.float32(t.cpu().numpy()[0])


@pytest.mark.parametrize("R,K,sigma,seed", [
    (4, 64, 1.0, 0), (33, 12288, 1.0, 1), (1000, 1024, 0.015, 2), (7, 28672, 1.0, 3),
    (1, 32, 1.0, 4), (129, 96, 0.015, 5),
    # decode-sized activations (one or two tokens of the MLP's K)
    (1, 28672, 1.0, 6), (2, 12288, 0.015, 7), (2, 32768, 1.0, 8), (1, 65568, 1.0, 9),
])
def test_fp4_quant_parity(R, K, sigma, seed):
    say(f"fp4 quant R={R} K={K}")
    x = synth.normal_bf16((R, K), sigma, "nvfp4", "x" if sigma == 1.0 else "w", seed=seed)
    q, s, g = _quant_dev(x)
    rq, rs, rg = P.quant_fp4(x)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32)
    assert np.array_equal(s, rs), f"{np.count_nonzero(s != rs)} group-scale mismatches"
    assert np.array_equal(q, rq), f"{np.count_nonzero(q != rq)} code-byte mismatches"


def test_fp4_quant_static_scale_and_edges():
    x = synth.normal_bf16((6, 256), 1.0, "nvfp4", "x", seed=9)
    x[1] = 0                                   # zero row
    x[2, :16] = 0x8000                         # negative zeros
    x[3, 16:32] = np.arange(1, 17, dtype=np.uint16)   # subnormal group
    x[4, 32:48] = synth.f32_to_bf16_bits(np.float32([3e4, -3e4] * 8))  # saturating group
    g = np.float32(0.02)
    q, s, gg = _quant_dev(x, g)
    rq, rs, _ = P.quant_fp4(x, g)
    assert gg == g
    assert np.array_equal(s, rs) and np.array_equal(q, rq)
    q, s, gg = _quant_dev(np.zeros((3, 64), np.uint16))
    assert gg == 1.0 and not q.any() and not s.any()


def _gemm_dev(h, M, N):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    xq, xs, xg, wq, ws, wg = h
    y_full = torch.full((M * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = y_full[: M * N].view(M, N)
    L.fp4_group_gemm(to_dev(xq), to_dev(xs), to_dev(np.float32([xg])), to_dev(wq), to_dev(ws),
                     to_dev(np.float32([wg])), y)
    torch.cuda.synchronize()
    assert torch.isnan(y_full[M * N:].float()).all(), "wrote past the output"
    return F.bf16_decode(bf16_bits(y))


@pytest.mark.parametrize("M,N,K", [
    (1, 256, 256), (5, 264, 288), (16, 1000, 1024), (33, 512, 640), (64, 256, 2048),
    (65, 256, 256), (130, 520, 640), (300, 1000, 1056), (256, 256, 128),
    (200, 264, 2144), (129, 136, 96),     # K blocks ending after 96 of 128 values
    # K % 128 == 0, M > 64: codes staged through the four-stage LDS pipeline
    (384, 1024, 4096), (300, 1000, 1152), (129, 136, 128), (4100, 264, 640),
    # enough 128 x 128 tiles for two rounds, one round of 256 x 256 tiles:
    # the 256 x 256 tile, ragged in M and N, with 1 and 5 K blocks
    (1536, 6144, 128), (1300, 8200, 256), (1100, 8296, 640),
])
def test_fp4_gemm_parity(M, N, K):
    say(f"fp4 gemm M={M} N={N} K={K}")
    x = synth.normal_bf16((M, K), 1.0, "nvfp4", "x", seed=M)
    w = synth.normal_bf16((N, K), 0.015, "nvfp4", "w", seed=N)
    xq, xs, xg = P.quant_fp4(x)
    wq, ws, wg = P.quant_fp4(w)
    y = _gemm_dev((xq, xs, xg, wq, ws, wg), M, N)
    assert np.isfinite(y).all(), "unwritten outputs"
    ref = P.fp4_gemm(xq, xs, xg, wq, ws, wg)
    err = rel_fro(y, ref)
    say(f"  rel fro {err:.3e}  vs bf16(ref) {rel_fro(y, F.bf16_round(ref)):.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,K,N", [(32, 12288, 28672), (4096, 12288, 28672), (1, 28672, 12288)])
def test_fp4_mlp_full_size_sampled(M, K, N):
    """Mistral MLP shapes with device-side quantization of both operands (the
    launch configuration the bench uses); the oracle quantizes the sampled
    rows itself with the full tensors' scales and recomputes 2048 outputs."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"fp4 full-size M={M} K={K} N={N}")
    x = synth.normal_bf16((M, K), 1.0, "nvfp4", "x", seed=11)
    wdev = synth.device_normal_bf16((N, K), 0.015, "nvfp4", "w", index=N)
    xd = to_dev_bf16(x)
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    tx = torch.empty((1,), dtype=torch.float32, device="cuda")
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    tw = torch.empty((1,), dtype=torch.float32, device="cuda")
    L.fp4_quant(xd, qx, sx, tx)
    L.fp4_quant(wdev, qw, sw, tw)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.fp4_group_gemm(qx, sx, tx, qw, sw, tw, y)
    torch.cuda.synchronize()
    wh = bf16_bits(wdev)
    gx, gw = P.tensor_scale(x), P.tensor_scale(wh)
    g = np.random.default_rng(M)
    rows = g.integers(0, M, 2048)
    cols = g.integers(0, N, 2048)
    ur, uc = np.unique(rows), np.unique(cols)
    hx = P.quant_fp4(x[ur], gx)
    hw = P.quant_fp4(wh[uc], gw)
    A = P.dequant_fp4(*hx)
    B = P.dequant_fp4(*hw)
    ri = np.searchsorted(ur, rows)
    ci = np.searchsorted(uc, cols)
    ref = np.einsum("ik,ik->i", A[ri], B[ci])
    got = F.bf16_decode(bf16_bits(y))[rows, cols]
    err = rel_fro(got, ref)
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL
    # and the device tensor scales equal the oracle's
    assert np.float32(tx.item()) == gx and np.float32(tw.item()) == gw
