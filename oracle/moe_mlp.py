"""The step between the MoE experts' gate/up and down GEMMs, fused onto the
gate/up GEMM (test infrastructure: only tests/, the smoke check and the
benchmark's CPU baseline use this package).

What the pages fix: the MLP is made of gate_proj, up_proj and down_proj
([NVFP4], the layer-wise quantization section); MoE experts run their
matmuls on the FP8 path ([FG-FP8] §一 FP8Experts, §6.4); the down
projection's input is an activation like any other, quantized per token in
1 x 128 groups along its input channels ([FG-FP8] §一).

Readings where the pages are silent:
 19. expert e's gate and up projections are the two halves of one (2I, K)
     weight -- rows [0, I) gate, [I, 2I) up -- with I a multiple of 128, so
     each half starts on a 128-row weight block; both halves use the same
     1 x 128 activation groups;
 20. the activation is SiLU: h = silu(g) * u with silu(g) = g / (1 + e^-g),
     taken on the unrounded GEMM values g and u (no bf16 round trip);
 21. h is rounded to bf16, the linears' activation type, and quantized by
     the 1 x 128 activation quantizer with the scale format of the GEMM
     (fp32 or UE8M0), so the down GEMM reads it as any quantized activation.
"""

import numpy as np

from .gemm import grouped_gemm
from .quant import SCALE_FLOAT


def silu(x):
    """x * sigmoid(x) in float64, without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))                 # in (0, 1]
    sig = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return x * sig


def gate_up_silu(xq, x_scale, wq, w_scale, seg_offsets, fmt=SCALE_FLOAT):
    """h (T, I) float64 = silu(X Wg^T) * (X Wu^T) per expert segment.

    xq (T, K) codes, x_scale (T, ceil(K/128)); wq (E, 2I, K) with gate rows
    first, w_scale (E, 2I/128, ceil(K/128)); seg_offsets (E + 1,).
    """
    I = wq.shape[1] // 2
    Y = grouped_gemm(xq, x_scale, wq, w_scale, seg_offsets, 128, 128, fmt)
    return silu(Y[:, :I]) * Y[:, I:]
