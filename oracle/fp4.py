"""NVFP4-style quantization and GEMM (test infrastructure).

[NVFP4] (config_groups group_1; hf_quant_config quantized_layers): weights
*and* input activations of the MLP projections are 4-bit floats quantized in
groups of 16 elements (``group_size: 16``), while attention projections stay
FP8.  The pages give nothing more; the scale structure (an E4M3 scale per
16-element group times one fp32 scale per tensor) is the one the task states.

Readings taken (pages silent):
 1. tensor scale g = fl32(A_t / 2688), A_t = max |x| over the tensor,
    2688 = 6 * 448, so that the largest group scale is the E4M3 maximum;
    g = 1.0 when A_t = 0.  For activations g is recomputed on every call
    (dynamic); for weights once.
 2. group scale code sg = E4M3(fl32(a / fl32(6 * g))) with a = the group's
    max |x|; the effective group multiplier is eff = fl32(dec(sg) * g).
 3. codes q = E2M1(fl32(x / eff)); a group whose eff is 0 (all-zero group,
    or a scale that underflows E4M3) gets all-zero codes.
 4. two codes per byte, element 2i in the low nibble.
 5. the value represented is dec(q) * dec(sg) * g.
"""

import numpy as np

from .formats import bf16_decode, e4m3_encode, e4m3_decode, e2m1_encode, \
    e2m1_decode, e2m1_pack, e2m1_unpack, E4M3_MAX, E2M1_MAX

GROUP = 16


def tensor_scale(x_bf16):
    """fp32 tensor scale g = fl32(max|x| / 2688); 1.0 for an all-zero tensor."""
    x = bf16_decode(x_bf16).astype(np.float32)
    at = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if at == 0:
        return np.float32(1.0)
    return np.float32(at / np.float32(E2M1_MAX * E4M3_MAX))


def quant_fp4(x_bf16, g=None):
    """x_bf16 uint16 (R, K), K % 16 == 0.  Returns (packed uint8 (R, K/2),
    group scale codes uint8 (R, K/16), tensor scale float32)."""
    x = bf16_decode(x_bf16).astype(np.float32)
    R, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 16")
    g = tensor_scale(x_bf16) if g is None else np.float32(g)
    xg = x.reshape(R, K // GROUP, GROUP)
    a = np.max(np.abs(xg), axis=-1)                            # float32
    den = np.float32(np.float32(E2M1_MAX) * g)
    sg = e4m3_encode((a / den).astype(np.float32).astype(np.float64))
    eff = (e4m3_decode(sg).astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xg / eff[..., None]).astype(np.float32)
    codes = e2m1_encode(y.astype(np.float64))
    codes = np.where(eff[..., None] > 0, codes, 0).astype(np.uint8)
    return e2m1_pack(codes.reshape(R, K)), sg, g


def dequant_fp4(packed, gscale, g):
    """-> float64 (R, K) = dec(q) * dec(sg) * g."""
    q = e2m1_decode(e2m1_unpack(packed))
    s = np.repeat(e4m3_decode(gscale), GROUP, axis=-1)
    return q * s * np.float64(np.float32(g))


def fp4_gemm(xq4, xs, xg, wq4, ws, wg):
    """Y (M, N) float64 = dequant(X) @ dequant(W)^T, fp64 accumulation."""
    return dequant_fp4(xq4, xs, xg) @ dequant_fp4(wq4, ws, wg).T
