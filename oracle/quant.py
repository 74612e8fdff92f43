"""Fine-grained FP8 quantization (test infrastructure).

What the pages fix ([FG-FP8] §一; [HF-PT] opening list):
* weights are quantized per 2D block, ``weight_block_size=(128, 128)``: every
  128x128 sub-matrix of W (N x K, nn.Linear orientation) shares one scale, and
  ``weight_scale_inv`` has shape (ceil(N/128), ceil(K/128));
* activations are quantized per token in groups whose width equals the
  weight block along the input channels (128 by default), so that act groups
  and weight blocks line up along K;
* values are stored as float8_e4m3fn; scales as fp32, or as packed
  float8_e8m0fnu when ``scale_fmt="ue8m0"`` ([FG-FP8] §七).

Readings taken where the pages are silent:
 1. a scale maps the group's largest magnitude onto the E4M3 maximum 448;
 2. ``float``: s = fl32(amax / 448), codes = E4M3(fl32(x / s)) with IEEE fp32
    division and one round-to-nearest-even into E4M3; the stored scale is the
    dequantization multiplier (hence the name ``weight_scale_inv``);
 3. amax = 0 gives s = 1.0 (float) or exponent 0 (ue8m0);
 4. ``ue8m0``: the scale is the smallest power of two 2^e with 448*2^e >= amax,
    i.e. e = ceil(log2(amax/448)) -- the pages say fp32 scales are rounded
    *up* when turned into UE8M0 ([FG-FP8] §七, closing note); e is clamped to
    [-127, 127] and stored as the byte e + 127; codes = E4M3(x * 2^-e);
 5. a partial last block/group (ceil in the scale shape) takes its amax over
    the in-range elements only;
 6. activation scales are laid out row-major (M, ceil(K/128)).
"""

import numpy as np

from .formats import bf16_decode, e4m3_encode, E4M3_MAX

SCALE_FLOAT = 0
SCALE_UE8M0 = 1


def ue8m0_exponent(amax):
    """e = ceil(log2(amax / 448)) from exact frexp; 0 where amax == 0.

    amax = f * 2^E with f in [1, 2).  448 = 1.75 * 2^8, so amax / 448 =
    (f / 1.75) * 2^(E - 8): the ratio f / 1.75 lies in (0.57, 1] when
    f <= 1.75 (ceil gives E - 8) and in (1, 1.15) otherwise (E - 7).
    """
    a = np.asarray(amax, dtype=np.float64)
    fr, ex = np.frexp(a)                  # a = fr * 2^ex, fr in [0.5, 1)
    f = fr * 2.0
    E = ex.astype(np.int64) - 1
    e = np.where(f <= 1.75, E - 8, E - 7)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127)


def _scale_and_codes(blocks, valid, fmt):
    """blocks: float32 array (..., n) of one scale group each (last axis),
    valid: same shape bool mask.  Returns (codes uint8 (..., n), scale)."""
    amax = np.max(np.where(valid, np.abs(blocks), np.float32(0)), axis=-1)
    if fmt == SCALE_FLOAT:
        s = np.where(amax == 0, np.float32(1.0),
                     (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32))
        s = s.astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            y = (blocks.astype(np.float32) / s[..., None]).astype(np.float32)
        codes = e4m3_encode(y.astype(np.float64))
        return codes, s
    if fmt == SCALE_UE8M0:
        e = ue8m0_exponent(amax)
        y = np.ldexp(blocks.astype(np.float64), -e[..., None])   # exact
        codes = e4m3_encode(y)
        return codes, (e + 127).astype(np.uint8)
    raise ValueError("scale_fmt must be 0 (float) or 1 (ue8m0)")


def quant_act(x_bf16, group_k=128, fmt=SCALE_FLOAT):
    """Per-token 1 x group_k dynamic activation quantization.

    x_bf16: uint16 (M, K) bf16 bits.  Returns (xq uint8 (M, K) E4M3 codes,
    scale (M, ceil(K/group_k)) float32 or uint8 E8M0 bytes).
    """
    x = bf16_decode(x_bf16).astype(np.float32)
    M, K = x.shape
    G = -(-K // group_k)
    pad = G * group_k - K
    xp = np.pad(x, ((0, 0), (0, pad)))
    vp = np.pad(np.ones_like(x, dtype=bool), ((0, 0), (0, pad)))
    codes, s = _scale_and_codes(xp.reshape(M, G, group_k), vp.reshape(M, G, group_k), fmt)
    return codes.reshape(M, G * group_k)[:, :K].copy(), s


def quant_weight(w_bf16, block_n=128, block_k=128, fmt=SCALE_FLOAT):
    """Per 2D block (block_n x block_k) weight quantization.

    w_bf16: uint16 (N, K) bf16 bits.  Returns (wq uint8 (N, K),
    scale_inv (ceil(N/bn), ceil(K/bk)) float32 or uint8 E8M0 bytes).
    """
    w = bf16_decode(w_bf16).astype(np.float32)
    N, K = w.shape
    NB, KB = -(-N // block_n), -(-K // block_k)
    wp = np.pad(w, ((0, NB * block_n - N), (0, KB * block_k - K)))
    vp = np.pad(np.ones_like(w, dtype=bool), ((0, NB * block_n - N), (0, KB * block_k - K)))
    # (NB, bn, KB, bk) -> (NB, KB, bn*bk)
    wb = wp.reshape(NB, block_n, KB, block_k).transpose(0, 2, 1, 3).reshape(NB, KB, -1)
    vb = vp.reshape(NB, block_n, KB, block_k).transpose(0, 2, 1, 3).reshape(NB, KB, -1)
    codes, s = _scale_and_codes(wb, vb, fmt)
    codes = codes.reshape(NB, KB, block_n, block_k).transpose(0, 2, 1, 3)
    codes = codes.reshape(NB * block_n, KB * block_k)[:N, :K].copy()
    return codes, s


def dequant_scale(scale, fmt):
    """Stored scale -> float64 multiplier."""
    if fmt == SCALE_FLOAT:
        return np.asarray(scale, dtype=np.float32).astype(np.float64)
    return np.exp2(np.asarray(scale, dtype=np.uint8).astype(np.float64) - 127.0)
