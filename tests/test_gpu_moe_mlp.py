"""GPU parity of the MoE gate/up grouped GEMM with the fused SiLU-mul and
1 x 128 requantization: h against the oracle's fp64 silu(g) u (relative
Frobenius error <= 2e-3, the bf16 rounding of h included), and the codes and
scales bit-exact against the oracle's activation quantizer applied to the
kernel's own bf16 h."""

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import moe_mlp as MM
from oracle import quant as Q

from gpu_util import to_dev, to_dev_bf16, bf16_bits, u8, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def dsilu(g):
    sig = MM.silu(g) / np.where(g == 0, 1.0, g)
    sig = np.where(g == 0, 0.5, sig)
    return sig * (1.0 + g * (1.0 - sig))


def bound_ratio(got, g, u, sg, su, K):
    """max over elements of |got - h| / bound, h = silu(g) u from the fp64
    GEMM values g, u.  The bound is one bf16 ulp of h (2^-7 |h| covers it)
    plus the fp32 accumulation error carried through silu(g) u: recursive
    summation of K products errs by at most K 2^-24 sum|a b| (sg, su: the
    same GEMMs on sign-cleared codes), and 2^-20 |h| for the fp32 silu and
    product.  At most 1 for a correct kernel."""
    h = MM.silu(g) * u
    gam = K * 2.0 ** -24
    bnd = (2.0 ** -7 + 2.0 ** -20) * np.abs(h) + gam * (np.abs(dsilu(g) * u) * sg +
                                                       np.abs(MM.silu(g)) * su) + 1e-30
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - h) / bnd))


def _run(xq, xs, wq, ws, off, I, fmt, with_h):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    T = xq.shape[0]
    hq_full = torch.full((T * I + 256,), 0xA5, dtype=torch.uint8, device="cuda")
    hq = hq_full[:T * I].view(T, I)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    hs = torch.full((T, I // 128), 7, dtype=sdt, device="cuda")
    hb_full = torch.full((T * I + 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    hb = hb_full[:T * I].view(T, I) if with_h else None
    L.fp8_grouped_gemm_silu_mul_quant(xq, xs, wq, ws, off, hq, hs, h_bf16=hb, scale_fmt=fmt)
    torch.cuda.synchronize()
    assert (hq_full[T * I:] == 0xA5).all(), "wrote past the codes"
    if with_h:
        assert torch.isnan(hb_full[T * I:].float()).all(), "wrote past h"
    return hq, hs, hb


def _case(counts, I, K, fmt, seed):
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.normal_bf16((T, K), 1.0, "moe", "x", seed=seed)
    xq, xs = Q.quant_act(x, 128, fmt)
    wq = np.empty((E, 2 * I, K), np.uint8)
    ws = np.empty((E, 2 * I // 128, -(-K // 128)), np.float32 if fmt == 0 else np.uint8)
    for e in range(E):
        wq[e], ws[e] = Q.quant_weight(synth.normal_bf16((2 * I, K), 0.02, "moe", "w", e, seed=seed),
                                      128, 128, fmt)
    dev = [to_dev(a) for a in (xq, xs, wq, ws, off)]
    hq, hs, hb = _run(*dev, I, fmt, True)
    h_bits = bf16_bits(hb)
    got = F.bf16_decode(h_bits)
    assert np.isfinite(got).all(), "unwritten rows of h"
    ref = MM.gate_up_silu(xq, xs, wq, ws, off, fmt)
    err = rel_fro(got, ref)
    Y = G.grouped_gemm(xq, xs, wq, ws, off, fmt=fmt)
    S = G.grouped_gemm(xq & 0x7F, xs, wq & 0x7F, ws, off, fmt=fmt)   # sum |a b|
    r = bound_ratio(got, Y[:, :I], Y[:, I:], S[:, :I], S[:, I:], K)
    say(f"  h rel fro {err:.3e}  vs bf16(ref) {rel_fro(got, F.bf16_round(ref)):.3e}  bound ratio {r:.3f}")
    assert err <= TOL and r <= 1.0
    # the requantization is the activation quantizer applied to that bf16 h
    rq, rs = Q.quant_act(h_bits, 128, fmt)
    assert np.array_equal(u8(hq), rq), f"{np.count_nonzero(u8(hq) != rq)} code mismatches"
    assert np.array_equal(hs.cpu().numpy(), rs), "scale mismatches"
    # without the optional bf16 h the codes and scales are the same
    hq2, hs2, _ = _run(*dev, I, fmt, False)
    assert np.array_equal(u8(hq2), rq) and np.array_equal(hs2.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("counts,I,K", [
    ([3, 0, 1, 6, 2], 128, 256),
    ([0, 130, 0, 1, 257, 64], 256, 640),
    ([300], 384, 1040),
    (list(np.random.default_rng(7).integers(0, 40, 33)), 256, 512),
])
def test_silu_mul_quant_parity(counts, I, K, fmt):
    say(f"gate/up silu-mul quant E={len(counts)} T={sum(counts)} I={I} K={K} fmt={fmt}")
    _case(counts, I, K, fmt, seed=len(counts) + I)


def test_silu_mul_quant_feeds_down_gemm():
    """The codes and scales go straight into the down projection."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    counts, I, K, H = [5, 140, 0, 33], 256, 384, 264
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = synth.normal_bf16((T, K), 1.0, "moe", "x", seed=1)
    xq, xs = Q.quant_act(x, 128, 1)
    w1 = np.stack([Q.quant_weight(synth.normal_bf16((2 * I, K), 0.02, "moe", "w", e), 128, 128, 1)[0]
                   for e in range(4)])
    s1 = np.stack([Q.quant_weight(synth.normal_bf16((2 * I, K), 0.02, "moe", "w", e), 128, 128, 1)[1]
                   for e in range(4)])
    q2 = [Q.quant_weight(synth.normal_bf16((H, I), 0.02, "moe", "w2", e), 128, 128, 1) for e in range(4)]
    w2 = np.stack([a for a, _ in q2]); s2 = np.stack([b for _, b in q2])
    hq, hs, _ = _run(to_dev(xq), to_dev(xs), to_dev(w1), to_dev(s1), to_dev(off), I, 1, False)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    L.fp8_grouped_gemm(hq, hs, to_dev(w2), to_dev(s2), to_dev(off), y, scale_fmt=1)
    torch.cuda.synchronize()
    ref = G.grouped_gemm(u8(hq), hs.cpu().numpy(), w2, s2, off, fmt=1)
    err = rel_fro(F.bf16_decode(bf16_bits(y)), ref)
    say(f"  down rel fro {err:.3e}")
    assert err <= TOL


def test_silu_mul_quant_moe_shape_sampled():
    """Full MoE shape (256 experts, 7168 -> 2 x 2048, 4096 tokens x top-8
    Zipf routing, UE8M0): h sampled per expert against the oracle, and whole
    rows' codes and scales against the oracle quantizer of the kernel's h."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    E, I, K, TOK, TOPK = 256, 2048, 7168, 4096, 8
    tok, off = synth.moe_routing(TOK, E, TOPK)
    T = len(tok)
    say(f"moe gate/up silu-mul full shape T={T}")
    x = synth.normal_bf16((TOK, K), 1.0, "moe", "x")
    xd = to_dev_bf16(x)[torch.from_numpy(tok).cuda()]
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 128), dtype=torch.uint8, device="cuda")
    L.fp8_quant_act(xd, xq, xs, scale_fmt=1)
    wq = torch.empty((E, 2 * I, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((E, 2 * I // 128, K // 128), dtype=torch.uint8, device="cuda")
    for e in range(E):
        wb = synth.device_normal_bf16((2 * I, K), 0.02, "moe", "w", e)
        L.fp8_quant_weight(wb, wq[e], ws[e], scale_fmt=1)
    hq, hs, hb = _run(xq, xs, wq, ws, to_dev(off), I, 1, True)
    counts = np.diff(off)
    experts = [int(np.argmax(counts)), int(np.argmin(counts)), 17, 200]
    g = np.random.default_rng(0)
    got_all, ref_all, ratios = [], [], []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = g.integers(lo, hi, 16)
        cols = g.integers(0, I, 128)
        hxq, hxs = Q.quant_act(x[tok[rows]], 128, 1)
        wb = synth.device_normal_bf16((2 * I, K), 0.02, "moe", "w", e)
        hwq, hws = Q.quant_weight(bf16_bits(wb), 128, 128, 1)
        rr, cc = np.meshgrid(np.arange(16), cols, indexing="ij")
        gate = G.block_gemm_rows(hxq, hxs, hwq, hws, rr.ravel(), cc.ravel(), fmt=1)
        up = G.block_gemm_rows(hxq, hxs, hwq, hws, rr.ravel(), I + cc.ravel(), fmt=1)
        sg = G.block_gemm_rows(hxq & 0x7F, hxs, hwq & 0x7F, hws, rr.ravel(), cc.ravel(), fmt=1)
        su = G.block_gemm_rows(hxq & 0x7F, hxs, hwq & 0x7F, hws, rr.ravel(), I + cc.ravel(),
                               fmt=1)
        ridx = torch.from_numpy(rows).cuda()
        hrows = bf16_bits(hb[ridx])
        got_all.append(F.bf16_decode(hrows)[rr.ravel(), cc.ravel()])
        ref_all.append(MM.silu(gate) * up)
        ratios.append(bound_ratio(got_all[-1], gate, up, sg, su, K))
        rq, rs = Q.quant_act(hrows, 128, 1)
        assert np.array_equal(u8(hq[ridx]), rq) and np.array_equal(u8(hs[ridx]), rs)
    got, ref = np.concatenate(got_all), np.concatenate(ref_all)
    err, r = rel_fro(got, ref), max(ratios)
    say(f"  sampled h rel fro {err:.3e}  bound ratio {r:.3f}")
    assert err <= TOL and r <= 1.0
