"""Static activation quantization, weight dequantization and the fp32 ->
UE8M0 scale conversion (test infrastructure: only tests/, the smoke check and
the benchmark's CPU baseline use this package).

What the pages fix ([FG-FP8] §四, §五, §七):
* ``activation_scheme`` is "dynamic" or "static";
* a pre-quantized checkpoint loaded with ``dequantize=True`` has its block
  scales folded into the weights (Fp8Dequantize);
* power-of-two UE8M0 scales stored in float32 containers are converted
  exactly to the float8_e8m0fnu dtype the kernels read.

Readings where the pages are silent:
 12. static: one calibrated per-tensor activation scale supplied by the
     caller; float: codes = E4M3(fl32(x / s)); ue8m0: the scale is the byte b
     (s = 2^(b-127)) and codes = E4M3(x * 2^-(b-127)); every 1 x 128 group's
     stored scale is that one scale, so the GEMM is unchanged;
 13. dequantized weight = bf16_rne(fl32(dec(code) * scale)) -- the float32
     product, then one round-to-nearest-even into bf16;
 14. fp32 -> UE8M0: an exact power of two 2^k with -127 <= k <= 127 becomes
     the byte k + 127; every other value (not a power of two, <= 0, out of
     range, Inf, NaN) becomes 0xFF, the E8M0 NaN encoding.
"""

import numpy as np

from .formats import bf16_decode, bf16_round, e4m3_decode, e4m3_encode
from .quant import SCALE_FLOAT, SCALE_UE8M0, dequant_scale


def quant_act_static(x_bf16, act_scale, group_k=128, fmt=SCALE_FLOAT):
    """x_bf16 uint16 (M, K); act_scale a float32 (float) or a uint8 byte
    (ue8m0).  Returns (codes uint8 (M, K), scales (M, ceil(K/group_k)))."""
    x = bf16_decode(x_bf16).astype(np.float32)
    M, K = x.shape
    G = -(-K // group_k)
    if fmt == SCALE_FLOAT:
        s = np.float32(act_scale)
        y = (x / s).astype(np.float32)
        return e4m3_encode(y.astype(np.float64)), np.full((M, G), s, dtype=np.float32)
    if fmt == SCALE_UE8M0:
        b = np.uint8(act_scale)
        y = np.ldexp(x.astype(np.float64), -(int(b) - 127))   # exact
        return e4m3_encode(y), np.full((M, G), b, dtype=np.uint8)
    raise ValueError("scale_fmt must be 0 (float) or 1 (ue8m0)")


def dequant_weight_bf16(wq, w_scale, block_n=128, block_k=128, fmt=SCALE_FLOAT):
    """(N, K) E4M3 codes + (ceil(N/bn), ceil(K/bk)) scales -> uint16 bf16 bits
    of fl32(dec(code) * scale), rounded to nearest even."""
    q = e4m3_decode(wq).astype(np.float32)
    s = dequant_scale(w_scale, fmt).astype(np.float32)
    N, K = q.shape
    full = np.repeat(np.repeat(s, block_n, axis=0), block_k, axis=1)[:N, :K]
    prod = (q * full).astype(np.float32)
    r = bf16_round(prod.astype(np.float64)).astype(np.float32)   # a bf16 value, exact in fp32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def pow2_to_ue8m0(scale_f32):
    """float32 array -> uint8 E8M0 bytes (see reading 14)."""
    s = np.asarray(scale_f32, dtype=np.float32).astype(np.float64)
    out = np.full(s.shape, 255, dtype=np.uint8)
    with np.errstate(divide="ignore", invalid="ignore"):
        fin = np.isfinite(s) & (s > 0)
        fr, ex = np.frexp(np.where(fin, s, 1.0))        # s = fr * 2^ex, fr in [0.5, 1)
    k = ex.astype(np.int64) - 1
    ok = fin & (fr == 0.5) & (k >= -127) & (k <= 127)
    out[ok] = (k[ok] + 127).astype(np.uint8)
    return out
