"""Element codecs, written from the format definitions (test infrastructure).

The pages name the storage dtypes only: weights and activations in
``torch.float8_e4m3fn`` ([FG-FP8] §一), scales in ``torch.float8_e8m0fnu``
when ``scale_fmt="ue8m0"`` ([FG-FP8] §七, [HF-PT] "Formato de escala UE8M0"),
and 4-bit floats in 16-element groups for NVFP4 ([NVFP4], config_groups
group_1).  The bit layouts below are the OCP ones ([OFP8] E4M3, [MX] E8M0 and
E2M1).  All arithmetic is exact: values are held in float64, which represents
every code of these formats and every quotient by a power of two used here.

Rounding readings (pages silent): every encoder rounds to nearest, ties to
even, and saturates to the largest finite magnitude; the sign of a value that
rounds to zero is kept (so -0 and tiny negatives give the negative-zero code).
NaN / Inf inputs are outside the contract.
"""

import numpy as np

E4M3_MAX = 448.0   # largest finite E4M3FN magnitude ([OFP8]: S.1111.110)
E2M1_MAX = 6.0     # largest E2M1 magnitude ([MX]: S.11.1)


# --------------------------------------------------------------------------
# E4M3FN: s eeee mmm, bias 7, no infinities, S.1111.111 is NaN
# --------------------------------------------------------------------------

def e4m3_decode(codes):
    """uint8 codes -> float64 values ([OFP8] E4M3 table)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _round_quantum(a, q):
    """Round a/q to the nearest integer, ties to even; a/q is exact (q = 2^k)."""
    return np.rint(a / q)  # numpy rint rounds half to even


def e4m3_encode(values):
    """Finite float values -> uint8 E4M3FN codes, RNE, saturating to +-448.

    Step by step: clamp |v| to 448; the quantum is 2^-9 below 2^-6 (the
    subnormal range) and 2^(floor(log2|v|) - 3) above; round |v| / quantum
    to an integer with ties to even; re-assemble sign, exponent and mantissa
    (a carry into the next binade falls out of the re-assembly).
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    flo = ex.astype(np.int64) - 1             # floor(log2 a) for a > 0
    q = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.maximum(flo, -6) - 3.0))
    r = _round_quantum(a, q) * q              # rounded magnitude, exact
    r = np.minimum(r, E4M3_MAX)               # cannot exceed 448 after rounding
    # encode the rounded magnitude
    _, ex2 = np.frexp(r)
    e_unb = ex2.astype(np.int64) - 1          # floor(log2 r)
    normal = r >= 2.0 ** -6
    e_field = np.where(normal, e_unb + 7, 0)
    mant = np.where(normal, r / np.exp2(e_unb.astype(np.float64)) * 8 - 8, r / 2.0 ** -9)
    code = (e_field << 3) | mant.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# E8M0: unsigned exponent only, bias 127, 0xFF is NaN, no zero
# --------------------------------------------------------------------------

def e8m0_decode(codes):
    """uint8 -> float64 power of two 2^(b-127) ([MX] E8M0); 255 -> NaN."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


# --------------------------------------------------------------------------
# E2M1: s ee m, bias 1, values {0, .5, 1, 1.5, 2, 3, 4, 6}
# --------------------------------------------------------------------------

def e2m1_decode(nibbles):
    """4-bit codes (0..15, any integer dtype) -> float64 ([MX] FP4 E2M1)."""
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (2 + m) * np.exp2(e.astype(np.float64) - 2))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(values):
    """Finite values -> E2M1 nibble codes (uint8 0..15), RNE, saturating to 6.

    Quantum 0.5 on [0, 2), 1 on [2, 4), 2 on [4, 6]; ties to even.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(_round_quantum(a, q) * q, E2M1_MAX)
    # magnitude -> code: table position of the value
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    idx = np.searchsorted(mags, r)
    code = np.where(neg, idx | 0x8, idx)
    return code.astype(np.uint8)


def e2m1_pack(nibbles):
    """(..., 2k) nibbles -> (..., k) bytes; element 2i in the LOW nibble."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] & 0xF) | ((n[..., 1::2] & 0xF) << 4)


def e2m1_unpack(packed):
    """(..., k) bytes -> (..., 2k) nibbles (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# BF16: the upper half of an IEEE binary32
# --------------------------------------------------------------------------

def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(values):
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    Used only to describe the rounding of the final bf16 output for
    diagnostics.  Computed directly from float64 (no intermediate fp32
    rounding): quantum 2^(floor(log2|v|) - 7), subnormal quantum 2^-133.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    flo = ex.astype(np.int64) - 1
    q = np.exp2(np.maximum(flo, -126) - 7.0)
    r = np.rint(a / q) * q
    return np.copysign(r, v)
