"""fp8_linear_noalloc (the entry point for callers that cannot allocate: its
workspace is a library-owned device array) against fp8_linear with a caller
workspace: bit-identical outputs on two calls in a row, the second with a
smaller problem, on the staged-quantization path (which uses the array) and
the fused decode path; a problem whose workspace exceeds the array is
refused on the host."""

import ctypes

import numpy as np
import pytest

from block_scaled_precision_fp8_amd import synth

from gpu_util import to_dev_bf16, bf16_bits, say

pytestmark = pytest.mark.gpu


def _noalloc(L, x, wq, ws, y, bias=None, fmt=0, scheme=0, act_scale=None, stream=None):
    """Direct C-ABI call (no workspace argument exists)."""
    M = x.shape[0]
    N, K = wq.shape
    return L.load().fp8_linear_noalloc(
        L._ptr(x), x.stride(0), L._ptr(wq), L._ptr(ws), L._ptr(bias), L._ptr(y), M, N, K,
        128, 128, scheme, fmt, L._ptr(act_scale), L._stream(stream))


def _case(M, N, K, fmt, seed):
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    x = synth.llama_acts(M, K, seed=seed)
    w = synth.normal_bf16((N, K), 0.02, "llama", "w", seed=seed)
    b = synth.normal_bf16((N,), 0.5, "llama", "bias", seed=seed)
    xd, wd, bd = to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(b)
    sdt = torch.float32 if fmt == 0 else torch.uint8
    wq = torch.empty((N, K), dtype=torch.uint8, device=xd.device)
    ws = torch.empty((-(-N // 128), -(-K // 128)), dtype=sdt, device=xd.device)
    L.fp8_quant_weight(wd, wq, ws, scale_fmt=fmt)
    y_ref = torch.empty((M, N), dtype=torch.bfloat16, device=xd.device)
    L.fp8_linear(xd, wq, ws, y_ref, bias=bd, scale_fmt=fmt)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=xd.device)
    st = _noalloc(L, xd, wq, ws, y, bias=bd, fmt=fmt)
    assert st == L.OK, L.status_string(st)
    torch.cuda.synchronize()
    return bf16_bits(y_ref), bf16_bits(y)


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_matches_linear_two_calls(fmt):
    from block_scaled_precision_fp8_amd import lib as L
    # first call: staged codes + scales and split-K partials in the array;
    # second, smaller: the array holds the first call's bytes on entry
    for (M, N, K) in ((128, 4096, 4096), (40, 1024, 1536)):
        need = L.workspace_size(L.OP_LINEAR, M, N, K)
        assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
        say(f"noalloc M={M} N={N} K={K} fmt={fmt} workspace={need}")
        a, b = _case(M, N, K, fmt, seed=M)
        assert np.array_equal(a, b), "fp8_linear_noalloc differs from fp8_linear"


def test_noalloc_decode_and_static():
    """The fused decode path (no workspace) and the static scheme."""
    import torch
    from block_scaled_precision_fp8_amd import lib as L
    a, b = _case(16, 512, 1024, 0, seed=3)
    assert np.array_equal(a, b)
    M, N, K = 96, 768, 2048
    x = to_dev_bf16(synth.llama_acts(M, K, seed=5))
    wq = torch.randint(0, 126, (N, K), dtype=torch.uint8, device=x.device)
    ws = torch.rand((N // 128, K // 128), device=x.device) * 1e-3
    s = torch.tensor([0.07], dtype=torch.float32, device=x.device)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    y2 = torch.empty_like(y1)
    L.fp8_linear(x, wq, ws, y1, act_scheme=L.ACT_STATIC, act_scale=s)
    assert _noalloc(L, x, wq, ws, y2, scheme=L.ACT_STATIC, act_scale=s) == L.OK
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2))


def test_noalloc_refuses_beyond_the_array():
    from block_scaled_precision_fp8_amd import lib as L
    M, N, K = 8192, 4096, 14336
    assert L.workspace_size(L.OP_LINEAR, M, N, K) > L.NOALLOC_SCRATCH_BYTES
    FAKE = 0x100000
    st = L.load().fp8_linear_noalloc(FAKE, K, FAKE, FAKE, None, FAKE, M, N, K, 128, 128, 0, 0,
                                     None, None)
    assert st == L.ENOSPC
