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
    # decode with M x K codes too large to stage in LDS (the one-launch
    # weight-streaming kernel): long and ragged rows
    (16, 4104, 14336, True), (12, 1040, 14352, False), (4, 1032, 32784, True),
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


@pytest.mark.parametrize("M,N,K,fmt,bias", [
    (4, 6144, 1792, 0, True),     # 384 tiles over the resident workgroups; one block per wave
    (16, 6400, 4096, 1, False),   # 400 tiles: some workgroups one tile (an all-zero chunk)
    (8, 6160, 6160, 0, False),    # ragged K and N; two chunks of two blocks per tile
    (4, 2056, 14352, 0, True),    # long ragged rows: 113 blocks, four chunks of two
    (6, 1032, 18432, 1, False),   # 144 blocks: three chunks of three, ragged last tile
])
def test_decode_persistent_parity(M, N, K, fmt, bias):
    """Decode shapes (4 <= M <= 16) on the persistent kernel: the M x K codes
    staged in LDS, chunks prefetched across tiles, chunk slots past a tile's
    blocks, a final all-zero chunk, ragged K and N, against the oracle."""
    from block_scaled_precision_fp8_amd import lib as L
    say(f"persistent decode M={M} N={N} K={K} fmt={fmt} bias={bias}")
    assert L.gemm_kernel(M, N, K)[0] == L.GEMM_DECODE
    x = synth.deepseek_acts(M, K, seed=K) if fmt else synth.llama_acts(M, K, seed=K)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=N) if bias else None
    h, d = _quant_dev(x, w, fmt)
    y = _gemm_dev(d, M, N, b, fmt)
    ref = G.block_gemm(*h, bias=None if b is None else F.bf16_decode(b), fmt=fmt)
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
                                   (1, 2728, 6144), (16, 4104, 4096), (4, 1536, 7168),
                                   # fused kernel against the persistent decode kernel
                                   (8, 2048, 6144),
                                   # the persistent kernel quantizing X itself
                                   (1, 1536, 7168), (2, 8192, 4096), (1, 1032, 14352),
                                   (16, 6144, 1536), (4, 1032, 7168)])
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


def _tiny_amax_acts(M, K, seed=11):
    """bf16 activations whose 1x128 groups have tiny amaxes: row r takes the
    r-th magnitude class below for every group (a few groups zero), so the
    fp32 scale fl32(amax / 448) runs from 0 through subnormal values (1 / s
    overflows below 2^-128) up to normal ones.  Values are uniform in
    [-amax, amax] (bf16 subnormals included) with one element = +-amax."""
    # 448 = 1.75 * 2^8, so amax = 1.75 * 2^k gives s = 2^(k - 8) exactly
    mags = [0.0, 2.0**-133, 2.0**-130, 2.0**-127,
            1.75 * 2.0**-121,          # s = 2^-129
            1.75 * 2.0**-120,          # s = 2^-128 exactly: 1 / s overflows
            1.7578125 * 2.0**-120,     # s just above 2^-128, still subnormal
            1.75 * 2.0**-119,          # s = 2^-127
            1.7421875 * 2.0**-118,     # s just below the smallest normal
            1.75 * 2.0**-118,          # s = 2^-126, the smallest normal
            2.0**-110, 1.0,
            "alt0", "alt1", "single", 2.0**-126]
    g = np.random.default_rng(seed)
    G = K // 128
    x = np.zeros((M, K), np.float32)
    for r in range(M):
        kind = mags[r % len(mags)]
        for gi in range(G):
            if isinstance(kind, str):
                if kind == "alt0":
                    a = 2.0**-125 if gi % 2 else 0.0
                elif kind == "alt1":
                    a = 2.0**-125 if gi % 2 else 2.0**-120
                else:
                    a = -1.0                       # one nonzero element, 2^-128
            else:
                a = kind if gi % 7 != 3 else 0.0   # a few zero groups per row
            seg = x[r, gi * 128:(gi + 1) * 128]
            if a == -1.0:
                seg[g.integers(0, 128)] = (2.0**-128) * (1 if gi % 2 else -1)
                continue
            if a == 0.0:
                continue
            seg[:] = (g.random(128) * 2 - 1) * a
            seg[g.integers(0, 128)] = a if g.random() < 0.5 else -a
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N", [(16, 512), (5, 512), (1, 512),
                                 # the persistent decode kernel's in-launch form
                                 (1, 8192), (2, 8192), (5, 8192)])
def test_linear_fused_quant_tiny_scales(fmt, M, N):
    """fp8_linear's in-launch quantization on groups whose scale is subnormal
    (amax below, at and above 448 * 2^-128, where 1 / s overflows, and
    around 448 * 2^-126), all-zero and mixed groups: bit-identical to
    fp8_quant_act + fp8_block_gemm, whose codes and scales match the oracle
    bit for bit; each row's output within the acceptance bound of the
    oracle's product."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    K = 4096
    assert L.workspace_size(L.OP_LINEAR, M, N, K) == 0          # the fused path
    # 16 tokens: every class; 5: the subnormal-scale classes; 1: s = 2^-128
    rows = {16: list(range(16)), 5: [1, 3, 5, 6, 8], 2: [3, 5], 1: [5]}[M]
    x = np.ascontiguousarray(_tiny_amax_acts(16, K)[rows])
    # large weights keep the products of the tiny activations normal
    w = synth.normal_bf16((N, K), 2.0**100, "llama", "w", seed=12)
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
    hq, hs = Q.quant_act(x, 128, fmt)
    assert np.array_equal(xq.cpu().numpy(), hq), "act codes differ from the oracle"
    assert np.array_equal(xs.cpu().numpy().view(np.uint8), hs.view(np.uint8)), \
        "act scales differ from the oracle"
    b1, b2 = bf16_bits(y1), bf16_bits(y2)
    bad = np.argwhere(b1 != b2)
    assert bad.size == 0, f"fused linear differs from quant + gemm at rows {np.unique(bad[:, 0])}"
    ref = G.block_gemm(hq, hs, *Q.quant_weight(w, 128, 128, fmt), fmt=fmt)
    got = F.bf16_decode(b2)
    assert np.isfinite(got).all()
    for r in range(M):
        if not np.any(ref[r]):
            assert not np.any(got[r]), f"row {r}: zero activations, nonzero output"
            continue
        e = rel_fro(got[r], ref[r])
        assert e <= TOL, f"row {r}: rel fro {e:.3e}"


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 512, 4096), (16, 1024, 4096), (16, 4104, 4096),
                                   (1, 8192, 4096), (2, 1032, 14352),
                                   (64, 1024, 1536), (300, 520, 640)])
@pytest.mark.parametrize("scale", ["plain", "tiny"])
def test_linear_static_matches_two_calls(M, N, K, fmt, scale):
    """fp8_linear with the static scheme (one calibrated per-tensor scale
    passed by pointer) equals fp8_quant_act with that static scale followed
    by fp8_block_gemm, bit for bit, on the fused decode path and the staged
    one; the static codes match the oracle's static quantizer."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    from oracle import convert as C
    x = synth.llama_acts(M, K, seed=21)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=21)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    if fmt == 0:
        sval = np.float32(0.05 if scale == "plain" else 2.0**-130)
        stat = torch.tensor([sval], dtype=torch.float32, device=xd.device)
    else:
        sval = np.uint8(120 if scale == "plain" else 1)
        stat = torch.tensor([int(sval)], dtype=torch.uint8, device=xd.device)
    G = -(-K // 128)
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    xs = torch.empty((M, G), dtype=sdt, device=xd.device)
    xs.view(-1)[0] = stat[0]
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((-(-N // 128), G), dtype=sdt, device=xd.device)
    L.fp8_quant_act(xd, xq, xs, act_scheme=L.ACT_STATIC, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    y2 = torch.empty_like(y1)
    L.fp8_block_gemm(xq, xs, wq, ws, y1, scale_fmt=fmt)
    L.fp8_linear(xd, wq, ws, y2, act_scheme=L.ACT_STATIC, scale_fmt=fmt, act_scale=stat)
    torch.cuda.synchronize()
    hq, _ = C.quant_act_static(x, sval, 128, fmt)
    assert np.array_equal(xq.cpu().numpy(), hq), "static codes differ from the oracle"
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2)), "static fp8_linear differs"


@pytest.mark.parametrize("M", [1, 32, 4096])
def test_attention_projection_12288_sampled(M):
    """The FP8 attention projection of the NVFP4-style model (12288 x 12288,
    1x128 / 128x128, fp32 scales) in the launch configuration the bench
    times; the oracle recomputes sampled outputs in three weight blocks."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    K = N = 12288
    say(f"attention projection M={M}")
    x = synth.normal_bf16((M, K), 1.0, "nvfp4", "x", index=M, seed=3)
    xd = to_dev_bf16(x)
    wd = synth.device_normal_bf16((N, K), 0.015, "nvfp4", "w", index=7, seed=3)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=xd.device)
    L.fp8_quant_weight(wd, wq, ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    L.fp8_linear(xd, wq, ws, y)
    torch.cuda.synchronize()
    g = np.random.default_rng(M)
    blocks = g.choice(N // 128, 3, replace=False)
    wrows = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
    wsub = bf16_bits(wd[torch.from_numpy(wrows).cuda()])       # the same bf16 draw
    hw, hws = Q.quant_weight(wsub, 128, 128, 0)                  # whole blocks
    rows = np.unique(g.integers(0, M, min(M, 64)))
    hx, hxs = Q.quant_act(x[rows], 128, 0)
    rr, cc = np.meshgrid(np.arange(len(rows)), np.arange(len(wrows)), indexing="ij")
    ref = G.block_gemm_rows(hx, hxs, hw, hws, rr.ravel(), cc.ravel())
    got = F.bf16_decode(bf16_bits(y)[rows][:, wrows]).ravel()
    err = rel_fro(got, ref)
    say(f"  sampled rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,ldx", [
    (17, 256, 256, 256),          # one K block, one tile, ragged M
    (40, 1024, 1536, 1536),       # K split in 4
    (200, 520, 1040, 1040),       # ragged M, N and K (partial last K block), 3 splits
    (32, 4096, 4096, 4096),       # 16 K splits: the largest problem the rule fuses
    (150, 1000, 2048, 2560),      # a strided X view (row stride > K)
    (520, 512, 512, 512),         # five M tiles
])
def test_linear_fused_large_m(M, N, K, ldx, fmt):
    """fp8_linear with M > 16 on 128 x 256 tiles quantizes the activations in
    the GEMM's K loop: bit-identical to fp8_quant_act + fp8_block_gemm (same
    tile and K splits), within the bound of the oracle's product."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    assert L.gemm_kernel(M, N, K)[0] == L.GEMM_TILE_128x256
    assert M * K * -(-N // 256) <= 2**21                         # the rule that fuses
    assert L.workspace_size(L.OP_LINEAR, M, N, K) == L.workspace_size(L.OP_BLOCK_GEMM, M, N, K)
    say(f"fused large-M linear M={M} N={N} K={K} ldx={ldx} fmt={fmt}")
    xfull = synth.deepseek_acts(M, ldx, seed=M + K) if fmt else synth.llama_acts(M, ldx, seed=M + K)
    x = np.ascontiguousarray(xfull[:, :K])
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N + K)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=N)
    xd = to_dev_bf16(xfull)[:, :K]
    wd, bd = to_dev_bf16(w), to_dev_bf16(b)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    G_ = -(-K // 128)
    xq = torch.empty((M, K), dtype=torch.uint8, device=wd.device)
    xs = torch.empty((M, G_), dtype=sdt, device=wd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=wd.device)
    ws = torch.empty((-(-N // 128), G_), dtype=sdt, device=wd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=wd.device)
    y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=wd.device)
    L.fp8_block_gemm(xq, xs, wq, ws, y1, bias=bd, scale_fmt=fmt)
    L.fp8_linear(xd, wq, ws, y2, bias=bd, scale_fmt=fmt)
    torch.cuda.synchronize()
    b1, b2 = bf16_bits(y1), bf16_bits(y2)
    assert np.array_equal(b1, b2), f"{np.count_nonzero(b1 != b2)} outputs differ from quant + gemm"
    hq, hs = Q.quant_act(x, 128, fmt)
    assert np.array_equal(xq.cpu().numpy(), hq)
    ref = G.block_gemm(hq, hs, *Q.quant_weight(w, 128, 128, fmt), bias=F.bf16_decode(b), fmt=fmt)
    err = rel_fro(F.bf16_decode(b2), ref)
    say(f"  rel fro {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_fused_large_m_tiny_scales(fmt):
    """The large-M in-loop quantization on rows whose groups have subnormal
    scales (1 / s overflowing at 2^-128), zero and mixed groups, and the
    static scheme with a subnormal scale: bit-identical to the two calls."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    M, K, N = 48, 4096, 512
    assert L.gemm_kernel(M, N, K)[0] == L.GEMM_TILE_128x256
    x = np.concatenate([_tiny_amax_acts(16, K)] * 3)
    w = synth.normal_bf16((N, K), 2.0**100, "llama", "w", seed=13)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    xs = torch.empty((M, K // 128), dtype=sdt, device=xd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((N // 128, K // 128), dtype=sdt, device=xd.device)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    ws_ = L.workspace_size(L.OP_LINEAR, M, N, K)
    work = torch.empty(max(ws_, 16), dtype=torch.uint8, device=xd.device)
    for stat in (None, "tiny"):
        if stat is None:
            L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
            sc = None
        else:
            sc = (torch.tensor([2.0**-130], dtype=torch.float32, device=xd.device) if fmt == 0
                  else torch.tensor([3], dtype=torch.uint8, device=xd.device))
            xs.view(-1)[0] = sc[0]
            L.fp8_quant_act(xd, xq, xs, act_scheme=L.ACT_STATIC, scale_fmt=fmt)
        y1 = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
        y2 = torch.empty_like(y1)
        L.fp8_block_gemm(xq, xs, wq, ws, y1, scale_fmt=fmt, workspace=work)
        L.fp8_linear(xd, wq, ws, y2, scale_fmt=fmt, workspace=work,
                     act_scheme=L.ACT_DYNAMIC if stat is None else L.ACT_STATIC, act_scale=sc)
        torch.cuda.synchronize()
        b1, b2 = bf16_bits(y1), bf16_bits(y2)
        bad = np.argwhere(b1 != b2)
        assert bad.size == 0, f"{stat}: rows {np.unique(bad[:, 0])} differ"


@pytest.mark.parametrize("M,fmt", [(1, 1), (17, 1), (1, 0), (17, 0)])
def test_block_gemm_max_k(M, fmt):
    """The largest K the entry points accept, 2^22 (32768 K blocks), through
    the device quantizers and fp8_block_gemm: the decode kernel (M = 1) and
    the split-K tile kernel (M = 17).  The activations are zero except in 24
    K blocks spread over the whole range, both ends included; each of those
    1 x 128 groups holds one power-of-two magnitude 2^a (a in -2..2, a third
    of the signs negative), and the 24-row weights hold 2^-(3 + j) with j in
    0..5 varying by row and block.  Both quantizers are then lossless: with
    UE8M0 scales a group gets 2^(a - 8) and codes +-256 and every weight
    block gets 2^-11 and codes 2^(8 - j), so dequantized operands equal the
    inputs; with fp32 scales they differ from them by one fp32 rounding of
    the scale.  The product is then the plain sum over the 24 blocks, exact
    in fp64 and in the kernels' fp32 accumulation (multiples of 2^-10 below
    2^11): UE8M0 must give its bf16 rounding bit for bit (a dropped, doubled
    or mispaired K block, or a wrong far-end offset, moves the sum by at
    least 2^-3), fp32 scales must be within the acceptance bound."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    K, N = 1 << 22, 24
    KB = K // 128
    say(f"max-K block gemm M={M} N={N} K={K} fmt={fmt}")
    g = np.random.default_rng(22 + M)
    blocks = np.array(sorted({0, 1, 2, 127, 128, 4095, 4096, 16383, 16384, KB - 2, KB - 1}
                             | set(int(b) for b in g.choice(np.arange(3, KB - 2), 13, replace=False))))
    assert len(blocks) == 24
    kk = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)      # the nonzero columns
    x = np.zeros((M, K), dtype=np.float32)
    for i, b in enumerate(blocks):
        for m in range(M):
            a = (i + m) % 5 - 2
            k = b * 128 + np.arange(128)
            x[m, k] = np.where(k % 3 == 0, -1.0, 1.0) * np.float32(2.0 ** a)
    j = (np.arange(KB)[None, :] + np.arange(N)[:, None]) % 6                # (N, KB)
    w = np.repeat(np.exp2(-(3.0 + j)).astype(np.float32), 128, axis=1)     # (N, K)
    ref = x[:, kk].astype(np.float64) @ w[:, kk].astype(np.float64).T        # the 24 blocks
    xd = to_dev_bf16(synth.f32_to_bf16_bits(x))
    wd = to_dev_bf16(synth.f32_to_bf16_bits(w))
    del x, w
    sdt = torch.float32 if fmt == 0 else torch.uint8
    xq = torch.empty((M, K), dtype=torch.uint8, device=xd.device)
    xs = torch.empty((M, KB), dtype=sdt, device=xd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((1, KB), dtype=sdt, device=xd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=xd.device)
    L.fp8_block_gemm(xq, xs, wq, ws, y, scale_fmt=fmt)
    torch.cuda.synchronize()
    got = F.bf16_decode(bf16_bits(y))
    assert np.isfinite(got).all(), "unwritten outputs"
    if fmt == 1:
        bad = np.argwhere(got != F.bf16_round(ref))
        assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[0]}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    else:
        err = rel_fro(got, ref)
        say(f"  rel fro {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("M,N,K,ldx,fmt", [
    (16, 4088, 4096, 4160, 0),    # branch-free loads (8+ tokens), ragged N
    (8, 520, 1024, 1096, 1),      # the smallest token count on those loads
    (5, 264, 640, 648, 0),        # below 8 tokens: the branch-guarded loads
    (16, 2048, 6144, 6208, 1),    # the longest row the fused form takes
])
def test_linear_fused_decode_row_stride(M, N, K, ldx, fmt):
    """fp8_linear's one-launch decode form on activations with a row stride
    above K (a view of wider rows): bit-identical to fp8_quant_act +
    fp8_block_gemm on the same view, codes equal to the oracle's, the
    product within the bound of the oracle's."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    assert L.gemm_kernel(M, N, K)[0] == L.GEMM_DECODE
    assert L.workspace_size(L.OP_LINEAR, M, N, K) == 0            # fused in the decode launch
    say(f"fused decode linear M={M} N={N} K={K} ldx={ldx} fmt={fmt}")
    xfull = synth.deepseek_acts(M, ldx, seed=M + K) if fmt else synth.llama_acts(M, ldx, seed=M + K)
    x = np.ascontiguousarray(xfull[:, :K])
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=N + K)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=N)
    xd = to_dev_bf16(xfull)[:, :K]
    assert xd.stride(0) == ldx
    wd, bd = to_dev_bf16(w), to_dev_bf16(b)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    G_ = -(-K // 128)
    xq = torch.empty((M, K), dtype=torch.uint8, device=wd.device)
    xs = torch.empty((M, G_), dtype=sdt, device=wd.device)
    wq = torch.empty((N, K), dtype=torch.uint8, device=wd.device)
    ws = torch.empty((-(-N // 128), G_), dtype=sdt, device=wd.device)
    L.fp8_quant_act(xd, xq, xs, scale_fmt=fmt)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=wd.device)
    y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=wd.device)
    L.fp8_block_gemm(xq, xs, wq, ws, y1, bias=bd, scale_fmt=fmt)
    L.fp8_linear(xd, wq, ws, y2, bias=bd, scale_fmt=fmt)
    torch.cuda.synchronize()
    b1, b2 = bf16_bits(y1), bf16_bits(y2)
    assert np.array_equal(b1, b2), f"{np.count_nonzero(b1 != b2)} outputs differ from quant + gemm"
    hq, hs = Q.quant_act(x, 128, fmt)
    assert np.array_equal(xq.cpu().numpy(), hq)
    ref = G.block_gemm(hq, hs, *Q.quant_weight(w, 128, 128, fmt), bias=F.bf16_decode(b), fmt=fmt)
    err = rel_fro(F.bf16_decode(b2), ref)
    say(f"  rel fro {err:.3e}")
    assert err <= TOL
