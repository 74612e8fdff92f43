"""FP4-packed weights with UE8M0 block scales, and the FP8-activation x
FP4-weight linear (test infrastructure: only tests/, the smoke check and the
benchmark's CPU baseline use this package).

What the pages fix ([FG-FP8] §一 and §6.1): V4-style checkpoints carry
FP4-packed expert weights, and the fast backend has an FP8-activation x
FP4-weight linear next to the FP8 x FP8 one; V4-style scales are UE8M0
([FG-FP8] §七).

Readings where the pages are silent:
 16. weight values are E2M1 (the 4-bit float of the NVFP4 page), two per
     byte, element 2i in the low nibble;
 17. one UE8M0 scale per 1 x 32 group along K of each weight row (the
     microscaling block of 32); the exponent is the smallest power of two
     that brings the group's amax within the E2M1 maximum 6 --
     e = ceil(log2(amax / 6)), the same round-up rule the pages give for
     UE8M0 FP8 scales -- clamped to [-127, 127], stored as e + 127; codes
     E2M1(w * 2^-e) rounded to nearest even; amax = 0 gives e = 0;
 18. activations are the FP8 1 x 128 groups of the FP8 path (fp32 or UE8M0
     scales); Y = sum_k dec(xq) s_a dec(wq) s_w in fp64, bf16 output
     rounding held to the usual 2e-3 relative Frobenius bound.
"""

import numpy as np

from .formats import bf16_decode, e2m1_decode, e2m1_encode, e2m1_pack, e2m1_unpack
from .gemm import dequant_act

E2M1_MAX = 6.0


def mx_exponent(amax):
    """e = ceil(log2(amax / 6)) from exact frexp; 0 where amax == 0.

    amax = f * 2^E with f in [1, 2): 6 = 1.5 * 2^2, so amax / 6 =
    (f / 1.5) * 2^(E - 2) with f / 1.5 in [0.67, 1.34): ceil gives E - 2
    when f <= 1.5 and E - 1 otherwise.
    """
    a = np.asarray(amax, dtype=np.float64)
    fr, ex = np.frexp(a)
    f = fr * 2.0
    E = ex.astype(np.int64) - 1
    e = np.where(f <= 1.5, E - 2, E - 1)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127)


def quant_weight_mxfp4(w_bf16, group=32):
    """w_bf16 uint16 (N, K), K % 32 == 0.  Returns (packed uint8 (N, K/2),
    scales uint8 (N, K/32) E8M0 bytes)."""
    w = bf16_decode(w_bf16)
    N, K = w.shape
    g = w.reshape(N, K // group, group)
    e = mx_exponent(np.max(np.abs(g), axis=-1))
    codes = e2m1_encode(np.ldexp(g, -e[..., None]))            # exact scaling
    return e2m1_pack(codes.reshape(N, K)), (e + 127).astype(np.uint8)


def dequant_mxfp4(packed, scales, group=32):
    """(N, K/2) codes + (N, K/32) E8M0 bytes -> float64 (N, K)."""
    v = e2m1_decode(e2m1_unpack(packed))
    s = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return v * np.repeat(s, group, axis=1)


def fp8_fp4_gemm(xq, x_scale, wq4, w_scale, bias=None, fmt=0):
    """Y (M, N) float64 = dequant(X, 1x128, fp32 or UE8M0) @ dequant(W, MXFP4)^T."""
    A = dequant_act(xq, x_scale, 128, fmt)
    B = dequant_mxfp4(wq4, w_scale)
    Y = A @ B.T
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    return Y


def grouped_fp8_fp4_gemm(xq, x_scale, wq4, w_scale, seg_offsets, fmt=0):
    """MoE experts with FP4-packed (MXFP4) weights over contiguous row
    segments ([FG-FP8] §一: V4-style FP4-packed expert weights): for every
    expert e, rows [off[e], off[e+1]) of Y are fp8_fp4_gemm of those rows of
    (xq, x_scale) with (wq4[e], w_scale[e]).

    xq (T, K) E4M3, x_scale (T, K/128), wq4 (E, N, K/2), w_scale (E, N, K/32),
    seg_offsets (E + 1,).  Returns Y (T, N) float64; rows of an empty
    segment do not exist.
    """
    off = np.asarray(seg_offsets, dtype=np.int64)
    E, N = wq4.shape[0], wq4.shape[1]
    Y = np.zeros((xq.shape[0], N))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            Y[lo:hi] = fp8_fp4_gemm(xq[lo:hi], x_scale[lo:hi], wq4[e], w_scale[e], fmt=fmt)
    return Y
