"""GPU parity of the block-scaled FP8 GEMM, the fused linear and the MoE
grouped GEMM against the oracle's fp64 product (relative Frobenius error
<= 2e-3, bf16 output rounding included)."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G

from gpu_util import to_dev, to_dev_bf16, bf16_bits, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _quant_dev(x_bits, w_bits, fmt):
    """Quantize on the host with the oracle; upload codes and scales."""
    xq, xs = Q.quant_act(x_bits, 128, fmt)
    wq, ws = Q.quant_weight(w_bits, 128, 128, fmt)
    return (xq, xs, wq, ws), (to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws))


def _gemm_dev(d, M, N, bias_bits=None, fmt=0):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    xq, xs, wq, ws = d
    y_full = torch.full((M * N + 64,), float("nan"), dtype=torch.bfloat16, device=xq.device)
    y = y_full[: M * N].view(M, N)
    bias = None if bias_bits is None else to_dev_bf16(bias_bits)
    L.fp8_block_gemm(xq, xs, wq, ws, y, bias=bias, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(y_full[M * N:].float()).all(), "wrote past the output"
    return F.bf16_decode(bf16_bits(y))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,bias", [
    (16, 256, 256, False),        # the single-linear case
    (1, 512, 384, True), (16, 264, 400, False), (37, 1000, 1024, True),
    (64, 256, 2048, False), (128, 384, 640, True),
    (130, 520, 640, False), (300, 1000, 1040, True), (256, 256, 128, False),
    (513, 768, 2048, True), (1024, 1024, 1024, False),
    (4100, 4104, 384, True),      # enough tiles for the 256 x 256 tile, ragged in M and N
    (5, 16400, 1040, True),       # decode, N past 16K, ragged N and K
    (16, 16384, 256, False),      # decode, N = 16K
])
def test_block_gemm_parity(M, N, K, bias, fmt):
    say(f"block gemm M={M} N={N} K={K} bias={bias} fmt={fmt}")
    if (M, N) == (4100, 4104):
        from block_scaled_precision_fp8_amd import lib as L
        assert L.gemm_kernel(M, N, K)[0] == L.GEMM_TILE_256x256
    x = synth.deepseek_acts(M, K, seed=M) if fmt else synth.llama_acts(M, K, seed=M)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=N) if bias else None
    h, d = _quant_dev(x, w, fmt)
    y = _gemm_dev(d, M, N, b, fmt)
    ref = G.block_gemm(*h, bias=None if b is None else F.bf16_decode(b), fmt=fmt)
    assert np.isfinite(y).all(), "unwritten outputs"
    err = rel_fro(y, ref)
    diag = rel_fro(y, F.bf16_round(ref))
    say(f"  rel fro {err:.3e}  vs bf16(ref) {diag:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,N,K,fmt", [
    (4100, 4104, 1040, 0),   # 256 x 256 tiles; the second scale chunk runs past ragged K
    (4100, 4104, 1040, 1),   # UE8M0 rows of 9 bytes: per-block scale loads
    (4100, 4104, 1024, 1),   # UE8M0 rows of 8 bytes: staged scale chunks
    (512, 512, 2688, 0),     # 7 K splits of 3 blocks: chunks start at every split
    (640, 1024, 6400, 0),    # 8 splits of 7 blocks
    (512, 512, 2560, 1),     # UE8M0, splits of 3 blocks: per-block loads
    (384, 1024, 4096, 1),    # UE8M0, 8 splits of 4 blocks: staged chunks
])
def test_block_gemm_scale_staging(M, N, K, fmt):
    """The activation-scale chunks the large-M kernel stages through LDS
    (fp32 always, UE8M0 when every row and split is dword-aligned), at
    chunk, split and ragged-K boundaries, against the oracle."""
    from block_scaled_precision_fp8_amd import lib as L
    kind, splits = L.gemm_kernel(M, N, K)
    say(f"scale staging M={M} N={N} K={K} fmt={fmt} kind={kind} splits={splits}")
    assert kind in (L.GEMM_TILE_256x256, L.GEMM_TILE_128x256)
    x = synth.deepseek_acts(M, K, seed=K) if fmt else synth.llama_acts(M, K, seed=K)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=K + 1)
    h, d = _quant_dev(x, w, fmt)
    y = _gemm_dev(d, M, N, None, fmt)
    ref = G.block_gemm(*h, fmt=fmt)
    assert np.isfinite(y).all(), "unwritten outputs"
    err = rel_fro(y, ref)
    say(f"  rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,K,N,fmt,gen", [
    (2048, 4096, 28672, 0, "llama"), (16, 14336, 4096, 0, "llama"),
    (128, 4096, 6144, 0, "llama"), (4096, 7168, 18432, 1, "deepseek"),
    (1, 18432, 7168, 1, "deepseek"), (64, 1536, 24576, 1, "deepseek"),
    (8192, 14336, 4096, 0, "llama"),
])
def test_block_gemm_full_size_sampled(M, K, N, fmt, gen):
    """Full-size shapes in the launch configuration the bench uses; the
    oracle recomputes 4096 sampled outputs one by one."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    say(f"full-size gemm M={M} K={K} N={N} fmt={fmt}")
    x = synth.llama_acts(M, K, seed=1) if gen == "llama" else synth.deepseek_acts(M, K, seed=1)
    sigma = 0.02 if gen == "llama" else 0.01
    w = synth.normal_bf16((N, K), sigma, gen, "w", seed=1)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xs = torch.empty((M, -(-K // 128)), dtype=sdt, device=xd.device)
    ws = torch.empty((-(-N // 128), -(-K // 128)), dtype=sdt, device=xd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    L.fp8_block_gemm(xq, xs, wq, ws, y, scale_fmt=fmt)
    y2 = torch.empty_like(y)
    L.fp8_linear(xd, wq, ws, y2, scale_fmt=fmt)
    torch.cuda.synchronize()
    yb = bf16_bits(y)
    assert np.array_equal(yb, bf16_bits(y2)), "fp8_linear differs from quant + gemm"
    g = np.random.default_rng(M + N)
    rows = g.integers(0, M, 4096)
    cols = g.integers(0, N, 4096)
    # the oracle quantizes the sampled rows itself (per-row act quant) and
    # the weight rows' blocks
    hx, hxs = Q.quant_act(x[np.unique(rows)], 128, fmt)
    rmap = {r: i for i, r in enumerate(np.unique(rows))}
    hw, hws = Q.quant_weight(w, 128, 128, fmt)
    ref = G.block_gemm_rows(hx, hxs, hw, hws, np.array([rmap[r] for r in rows]), cols, fmt=fmt)
    got = F.bf16_decode(yb[rows, cols])
    err = rel_fro(got, ref)
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_fused_quant_every_bf16_pattern(fmt):
    """The decode kernel's in-launch activation quantization against the
    standalone quantizer: every finite bf16 bit pattern, in a seeded order,
    as 16 tokens x 4096 channels; outputs must agree bit for bit."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, K, N = 16, 4096, 512
    pats = np.arange(65536, dtype=np.uint32)
    finite = ((pats >> 7) & 0xFF) != 0xFF
    pats = np.where(finite, pats, 0).astype(np.uint16)
    x = pats[np.random.default_rng(3).permutation(65536)].reshape(M, K)
    assert L.workspace_size(L.OP_LINEAR, M, N, K) == 0          # the fused path
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=8)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    xs = torch.empty((M, K // 128), dtype=sdt, device=xd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((N // 128, K // 128), dtype=sdt, device=xd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    y2 = torch.empty_like(y1)
    L.fp8_block_gemm(xq, xs, wq, ws, y1, scale_fmt=fmt)
    L.fp8_linear(xd, wq, ws, y2, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (16, 520, 384), (200, 512, 1040),
                                   (1, 8200, 256), (5, 264, 4112),
                                   # either side of the fused-quantization bound
                                   # (N K <= 2^24, K <= 6144)
                                   (1, 2728, 6144), (16, 4104, 4096), (4, 1536, 7168)])
def test_linear_matches_two_calls(M, N, K, fmt):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    x = synth.llama_acts(M, K, seed=7)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=7)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=7)
    xd, wd, bd = to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(b)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    xs = torch.empty((M, -(-K // 128)), dtype=sdt, device=xd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((-(-N // 128), -(-K // 128)), dtype=sdt, device=xd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    y2 = torch.empty_like(y1)
    L.fp8_block_gemm(xq, xs, wq, ws, y1, bias=bd, scale_fmt=fmt)
    L.fp8_linear(xd, wq, ws, y2, bias=bd, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2))
    ref = G.block_gemm(*Q.quant_act(x, 128, fmt), *Q.quant_weight(w, 128, 128, fmt),
                       bias=F.bf16_decode(b), fmt=fmt)
    assert rel_fro(F.bf16_decode(bf16_bits(y2)), ref) <= TOL


def _grouped_case(counts, N, K, fmt, seed):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.normal_bf16((T, K), 1.0, "moe", "x", seed=seed)
    xq, xs = Q.quant_act(x, 128, fmt)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, -(-N // 128), -(-K // 128)), np.float32 if fmt == 0 else np.uint8)
    for e in range(E):
        wq[e], ws[e] = Q.quant_weight(synth.normal_bf16((N, K), 0.02, "moe", "w", e, seed=seed),
                                      128, 128, fmt)
    y_full = torch.full((T * N + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = y_full[: T * N].view(T, N)
    L.fp8_grouped_gemm(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), to_dev(off), y,
                       scale_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.isnan(y_full[T * N:].float()).all()
    got = F.bf16_decode(bf16_bits(y))
    assert np.isfinite(got).all(), "unwritten rows"
    ref = G.grouped_gemm(xq, xs, wq, ws, off, fmt=fmt)
    return rel_fro(got, ref)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("counts,N,K", [
    ([3, 0, 1, 6, 2], 256, 256),
    ([0, 0, 130, 0, 1, 257, 64, 0], 512, 640),
    ([300], 264, 1040),
    ([0, 300, 5, 140], 384, 1024),   # large experts with dword-aligned UE8M0 scale rows
    (list(np.random.default_rng(5).integers(0, 40, 33)), 384, 512),
])
def test_grouped_gemm_parity(counts, N, K, fmt):
    say(f"grouped E={len(counts)} T={sum(counts)} N={N} K={K} fmt={fmt}")
    err = _grouped_case(counts, N, K, fmt, seed=len(counts))
    say(f"  rel fro {err:.3e}")
    assert err <= TOL


def test_grouped_gemm_moe_shape_sampled():
    """Full MoE gate/up shape (256 experts, 7168 -> 4096, 4096 tokens x top-8
    Zipf routing); the oracle checks sampled rows of a few experts."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E, N, K, TOK, TOPK = 256, 4096, 7168, 4096, 8
    tok, off = synth.moe_routing(TOK, E, TOPK)
    T = len(tok)
    say(f"moe full shape T={T}")
    x = synth.normal_bf16((TOK, K), 1.0, "moe", "x")
    xd = to_dev_bf16(x)[torch.from_numpy(tok).cuda()]
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 128), dtype=torch.float32, device="cuda")
    L.fp8_quant_act(xd, xq, xs)
    wq = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        wb = synth.device_normal_bf16((N, K), 0.02, "moe", "w", e)
        L.fp8_quant_weight(wb, wq[e], ws[e])
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    L.fp8_grouped_gemm(xq, xs, wq, ws, to_dev(off), y)
    torch.cuda.synchronize()
    counts = np.diff(off)
    experts = [int(np.argmax(counts)), int(np.argmin(counts)), 17, 200]
    g = np.random.default_rng(0)
    got_all, ref_all = [], []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = g.integers(lo, hi, 8)
        cols = g.integers(0, N, 64)
        hxq, hxs = Q.quant_act(x[tok[rows]], 128, 0)   # oracle's own codes
        # weights re-derived by the oracle from the same bf16 draw
        wb = synth.device_normal_bf16((N, K), 0.02, "moe", "w", e)
        hwq, hws = Q.quant_weight(bf16_bits(wb), 128, 128, 0)
        rr, cc = np.meshgrid(np.arange(8), cols, indexing="ij")
        ref = G.block_gemm_rows(hxq, hxs, hwq, hws, rr.ravel(), cc.ravel())
        got = F.bf16_decode(bf16_bits(y[torch.from_numpy(rows).cuda()]))[rr.ravel(), cc.ravel()]
        got_all.append(got)
        ref_all.append(ref)
    err = rel_fro(np.concatenate(got_all), np.concatenate(ref_all))
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL
