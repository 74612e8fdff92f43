"""Block-scaled FP8 GEMM, dense and MoE-grouped (test infrastructure).

[FG-FP8] §一: because activation groups and weight blocks line up along the
input channels, the matmul runs block by block; weights are (out, in) as in
nn.Linear, so Y = X W^T, and the bias is not quantized ([FG-FP8] §三).

The plain definition used here: dequantize both operands exactly,

    A[m, k] = dec(Xq[m, k]) * S_a[m, k // bk]
    B[n, k] = dec(Wq[n, k]) * S_w[n // bn, k // bk]
    Y[m, n] = sum_k A[m, k] * B[n, k]  (+ bias[n])

and accumulate in float64.  This equals the per-K-block form
sum_kb S_a S_w * sum_{k in kb} dec(Xq) dec(Wq) up to rounding order.  The
result is returned unrounded (float64); the GPU writes bf16, and the
acceptance budget counts that rounding.

MoE experts ([FG-FP8] §一 FP8Experts, §6.4): the rows of X are arranged in
contiguous per-expert segments given by ``seg_offsets`` (E + 1 entries,
nondecreasing, first 0, last T); segment e is multiplied by expert e's
weights.  The segment layout is the reading taken (the pages do not fix it).
"""

import numpy as np

from .formats import e4m3_decode
from .quant import dequant_scale, SCALE_FLOAT


def dequant_act(xq, x_scale, group_k=128, fmt=SCALE_FLOAT):
    """(M, K) codes + (M, G) scales -> float64 (M, K)."""
    a = e4m3_decode(xq)
    s = dequant_scale(x_scale, fmt)
    K = a.shape[1]
    return a * np.repeat(s, group_k, axis=1)[:, :K]


def dequant_weight(wq, w_scale, block_n=128, block_k=128, fmt=SCALE_FLOAT):
    """(N, K) codes + (NB, KB) scales -> float64 (N, K)."""
    b = e4m3_decode(wq)
    s = dequant_scale(w_scale, fmt)
    N, K = b.shape
    return b * np.repeat(np.repeat(s, block_n, axis=0), block_k, axis=1)[:N, :K]


def block_gemm(xq, x_scale, wq, w_scale, bias=None, block_n=128, block_k=128,
               fmt=SCALE_FLOAT):
    """Y (M, N) float64 = dequant(X) @ dequant(W)^T (+ bias as float64)."""
    A = dequant_act(xq, x_scale, block_k, fmt)
    B = dequant_weight(wq, w_scale, block_n, block_k, fmt)
    Y = A @ B.T
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    return Y


def block_gemm_rows(xq, x_scale, wq, w_scale, rows, cols, bias=None,
                    block_n=128, block_k=128, fmt=SCALE_FLOAT):
    """Y[rows[i], cols[i]] for sampled output positions (full-size checks)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = dequant_act(xq[rows], x_scale[rows], block_k, fmt)
    K = xq.shape[1]
    out = np.empty(len(rows))
    for i, (m, n) in enumerate(zip(rows, cols)):
        b = e4m3_decode(wq[n]) * np.repeat(dequant_scale(w_scale[n // block_n], fmt),
                                           block_k)[:K]
        out[i] = float(np.dot(A[i], b))
        if bias is not None:
            out[i] += float(bias[n])
    return out


def grouped_gemm(xq, x_scale, wq, w_scale, seg_offsets, block_n=128, block_k=128,
                 fmt=SCALE_FLOAT):
    """Per-expert block GEMM over contiguous row segments.

    xq (T, K), x_scale (T, G), wq (E, N, K), w_scale (E, NB, KB),
    seg_offsets (E + 1,).  Returns Y (T, N) float64.  Rows of an empty
    segment do not exist; every row belongs to exactly one segment.
    """
    off = np.asarray(seg_offsets, dtype=np.int64)
    E = wq.shape[0]
    T = xq.shape[0]
    N = wq.shape[1]
    Y = np.zeros((T, N))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            Y[lo:hi] = block_gemm(xq[lo:hi], x_scale[lo:hi], wq[e], w_scale[e],
                                  None, block_n, block_k, fmt)
    return Y
