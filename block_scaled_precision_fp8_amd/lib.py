"""Thin ctypes binding of libbsfp8.so (declared in include/bsfp8.h).

Argument marshalling only: every function here takes torch device tensors,
passes their data pointers, sizes and torch's current HIP stream to the
C entry point of the same name, and raises ``BsFp8Error`` on a non-OK
status.  Nothing is computed in Python.  The library is loaded from the
package directory; if it is missing, every call raises (there is no
fallback path).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsfp8.so")

OK, EINVAL, ENOTSUP, ENOSPC, EHIP = 0, 1, 2, 3, 4
SCALE_FLOAT, SCALE_UE8M0 = 0, 1
ACT_DYNAMIC, ACT_STATIC = 0, 1
OP_BLOCK_GEMM, OP_LINEAR, OP_GROUPED_GEMM, OP_FP4_QUANT, OP_FP4_GEMM, OP_FP8_FP4_GEMM = \
    0, 1, 2, 3, 4, 5
OP_LINEAR_B32 = 6
GEMM_NONE, GEMM_TILE_128x256, GEMM_TILE_256x256, GEMM_DECODE = 0, 2, 3, 4

EXPORTS = ("bsfp8_version", "bsfp8_status_string", "bsfp8_workspace_size", "bsfp8_gemm_kernel",
           "fp8_quant_act", "fp8_quant_weight", "fp8_block_gemm", "fp8_linear",
           "fp8_grouped_gemm", "fp4_quant", "fp4_group_gemm", "fp8_dequant_weight",
           "fp8_scale_to_ue8m0", "mxfp4_quant_weight", "fp8_fp4_gemm",
           "fp8_grouped_gemm_silu_mul_quant", "fp8_linear_noalloc", "fp8_fp4_grouped_gemm")
NOALLOC_SCRATCH_BYTES = 32 << 20     # BSFP8_NOALLOC_SCRATCH_BYTES


class BsFp8Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGS = {
    "bsfp8_version": (_I32, []),
    "bsfp8_status_string": (ctypes.c_char_p, [_I32]),
    "bsfp8_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _I32]),
    "bsfp8_gemm_kernel": (_I32, [_I64, _I64, _I64, _P]),
    "fp8_dequant_weight": (_I32, [_P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "fp8_scale_to_ue8m0": (_I32, [_P, _I64, _P, _P]),
    "mxfp4_quant_weight": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "fp8_fp4_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P]),
    "fp8_grouped_gemm_silu_mul_quant": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I64,
                                               _I64, _I32, _P]),
    "fp8_quant_act": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "fp8_quant_weight": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "fp8_block_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32,
                              _P, _SZ, _P]),
    "fp8_linear": (_I32, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                          _P, _P, _SZ, _P]),
    "fp8_linear_noalloc": (_I32, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32,
                                  _I32, _P, _P]),
    "fp8_fp4_grouped_gemm": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _I64, _I64, _I64, _I32, _P]),
    "fp8_grouped_gemm": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _I64, _I64, _I64, _I32, _I32,
                                _I32, _P, _SZ, _P]),
    "fp4_quant": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P, _P, _SZ, _P]),
    "fp4_group_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
}


def load(path=None):
    """Load (once) and return the ctypes handle; raises if the library is
    missing or lacks a declared symbol."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise BsFp8Error("load", -1, f"{p} not built; run "
                         "`python -m block_scaled_precision_fp8_amd.build`")
    # torch first: it brings its own HIP runtime under the same soname the
    # library links (libamdhip64.so.7), so the library then binds to that one
    # and kernels run on the runtime that owns torch's streams and memory.
    # Opened before torch, the library would load the system runtime and
    # torch a second one beside it.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(s):
    return load().bsfp8_status_string(s).decode()


def _check(fn, s):
    if s != OK:
        raise BsFp8Error(fn, s, status_string(s))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_size(op, M, N, K, E=0):
    return int(load().bsfp8_workspace_size(op, M, N, K, E))


def gemm_kernel(M, N, K):
    """(GEMM_* kind, K splits) that fp8_block_gemm / fp8_linear use for M x N x K."""
    sp = ctypes.c_int32(0)
    kind = int(load().bsfp8_gemm_kernel(M, N, K, ctypes.byref(sp)))
    return kind, int(sp.value)


def _workspace(op, M, N, K, E, ws, device):
    need = workspace_size(op, M, N, K, E)
    if ws is None and need:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (ws.numel() * ws.element_size() if ws is not None else 0)


def fp8_quant_act(x, xq, x_scale, group_k=128, act_scheme=ACT_DYNAMIC, scale_fmt=SCALE_FLOAT,
                  stream=None):
    """x: bf16 (M, >=K) with row stride ldx; xq: uint8 (M, K); x_scale: (M, G)."""
    M, K = xq.shape
    ldx = x.stride(0) if x.dim() == 2 else K
    _check("fp8_quant_act", load().fp8_quant_act(_ptr(x), M, K, ldx, group_k, act_scheme,
                                                 scale_fmt, _ptr(xq), _ptr(x_scale),
                                                 _stream(stream)))


def fp8_dequant_weight(wq, w_scale_inv, w, block_n=128, block_k=128, scale_fmt=SCALE_FLOAT,
                       stream=None):
    """wq: uint8 (N, K) E4M3; w_scale_inv: (NB, KB); w: bf16 (N, K) out."""
    N, K = wq.shape
    _check("fp8_dequant_weight", load().fp8_dequant_weight(_ptr(wq), N, K, block_n, block_k,
                                                           scale_fmt, _ptr(w_scale_inv),
                                                           _ptr(w), _stream(stream)))


def fp8_scale_to_ue8m0(scale, out, stream=None):
    """scale: fp32 tensor; out: uint8 tensor of the same number of elements."""
    _check("fp8_scale_to_ue8m0", load().fp8_scale_to_ue8m0(_ptr(scale), scale.numel(),
                                                           _ptr(out), _stream(stream)))


def mxfp4_quant_weight(w, wq4, w_scale, stream=None):
    """w: bf16 (N, >=K); wq4: uint8 (N, K/2); w_scale: uint8 (N, K/32)."""
    N, K = wq4.shape[0], wq4.shape[1] * 2
    ldw = w.stride(0) if w.dim() == 2 else K
    _check("mxfp4_quant_weight", load().mxfp4_quant_weight(_ptr(w), N, K, ldw, _ptr(wq4),
                                                           _ptr(w_scale), _stream(stream)))


def fp8_fp4_gemm(xq, x_scale, wq4, w_scale, y, bias=None, scale_fmt=SCALE_FLOAT,
                 workspace=None, stream=None):
    """xq: uint8 (M, K) E4M3; x_scale (M, K/128); wq4 (N, K/2); w_scale (N, K/32)."""
    M, K = xq.shape
    N = wq4.shape[0]
    ws, wsb = _workspace(OP_FP8_FP4_GEMM, M, N, K, 0, workspace, xq.device)
    _check("fp8_fp4_gemm", load().fp8_fp4_gemm(_ptr(xq), _ptr(x_scale), _ptr(wq4), _ptr(w_scale),
                                               _ptr(bias), _ptr(y), M, N, K, scale_fmt, _ptr(ws), wsb,
                                               _stream(stream)))


def fp8_grouped_gemm_silu_mul_quant(xq, x_scale, wq, w_scale_inv, seg_offsets, hq, h_scale,
                                    h_bf16=None, scale_fmt=SCALE_FLOAT, stream=None):
    """xq (T, K); wq (E, 2I, K) gate rows then up rows; hq (T, I) uint8;
    h_scale (T, I/128); h_bf16 optional bf16 (T, I)."""
    T, K = xq.shape
    E, N2 = wq.shape[0], wq.shape[1]
    _check("fp8_grouped_gemm_silu_mul_quant", load().fp8_grouped_gemm_silu_mul_quant(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale_inv), _ptr(seg_offsets), E, _ptr(hq),
        _ptr(h_scale), _ptr(h_bf16), T, N2 // 2, K, scale_fmt, _stream(stream)))


def fp8_quant_weight(w, wq, w_scale_inv, block_n=128, block_k=128, scale_fmt=SCALE_FLOAT,
                     stream=None):
    N, K = wq.shape
    ldw = w.stride(0) if w.dim() == 2 else K
    _check("fp8_quant_weight", load().fp8_quant_weight(_ptr(w), N, K, ldw, block_n, block_k,
                                                       scale_fmt, _ptr(wq), _ptr(w_scale_inv),
                                                       _stream(stream)))


def fp8_block_gemm(xq, x_scale, wq, w_scale_inv, y, bias=None, block_n=128, block_k=128,
                   scale_fmt=SCALE_FLOAT, workspace=None, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    ws, wsb = (None, 0) if block_n == 32 else _workspace(OP_BLOCK_GEMM, M, N, K, 0, workspace,
                                                          xq.device)
    _check("fp8_block_gemm", load().fp8_block_gemm(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale_inv), _ptr(bias), _ptr(y), M, N, K,
        block_n, block_k, scale_fmt, _ptr(ws), wsb, _stream(stream)))


def fp8_linear(x, wq, w_scale_inv, y, bias=None, block_n=128, block_k=128,
               act_scheme=ACT_DYNAMIC, scale_fmt=SCALE_FLOAT, act_scale=None, workspace=None,
               stream=None):
    """act_scale: device tensor holding the static scheme's calibrated scale
    (fp32, or one E8M0 byte); None for the dynamic scheme."""
    M = x.shape[0]
    N, K = wq.shape
    ws, wsb = _workspace(OP_LINEAR_B32 if block_k == 32 else OP_LINEAR, M, N, K, 0, workspace,
                         x.device)
    _check("fp8_linear", load().fp8_linear(
        _ptr(x), x.stride(0), _ptr(wq), _ptr(w_scale_inv), _ptr(bias), _ptr(y), M, N, K,
        block_n, block_k, act_scheme, scale_fmt, _ptr(act_scale), _ptr(ws), wsb,
        _stream(stream)))


def fp8_grouped_gemm(xq, x_scale, wq, w_scale_inv, seg_offsets, y, block_n=128, block_k=128,
                     scale_fmt=SCALE_FLOAT, workspace=None, stream=None):
    T, K = xq.shape
    E, N, _ = wq.shape
    ws, wsb = _workspace(OP_GROUPED_GEMM, T, N, K, E, workspace, xq.device)
    _check("fp8_grouped_gemm", load().fp8_grouped_gemm(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale_inv), _ptr(seg_offsets), E, _ptr(y),
        T, N, K, block_n, block_k, scale_fmt, _ptr(ws), wsb, _stream(stream)))


def fp8_fp4_grouped_gemm(xq, x_scale, wq4, w_scale, seg_offsets, y, scale_fmt=SCALE_FLOAT,
                         stream=None):
    """xq (T, K) E4M3; x_scale (T, K/128); wq4 uint8 (E, N, K/2); w_scale
    uint8 (E, N, K/32); seg_offsets int32 (E+1,) on the device; y bf16 (T, N)."""
    T, K = xq.shape
    E, N = wq4.shape[0], wq4.shape[1]
    _check("fp8_fp4_grouped_gemm", load().fp8_fp4_grouped_gemm(
        _ptr(xq), _ptr(x_scale), _ptr(wq4), _ptr(w_scale), _ptr(seg_offsets), E, _ptr(y), T, N, K,
        scale_fmt, _stream(stream)))


def fp4_quant(x, q4, gscale, tscale, dynamic_tscale=1, workspace=None, stream=None):
    R, K = x.shape
    ws, wsb = _workspace(OP_FP4_QUANT, R, 0, K, 0, workspace, x.device)
    _check("fp4_quant", load().fp4_quant(_ptr(x), R, K, dynamic_tscale, _ptr(q4), _ptr(gscale),
                                         _ptr(tscale), _ptr(ws), wsb, _stream(stream)))


def fp4_group_gemm(xq4, x_gscale, x_tscale, wq4, w_gscale, w_tscale, y, workspace=None,
                   stream=None):
    M = xq4.shape[0]
    N = wq4.shape[0]
    K = xq4.shape[1] * 2
    ws, wsb = _workspace(OP_FP4_GEMM, M, N, K, 0, workspace, xq4.device)
    _check("fp4_group_gemm", load().fp4_group_gemm(
        _ptr(xq4), _ptr(x_gscale), _ptr(x_tscale), _ptr(wq4), _ptr(w_gscale), _ptr(w_tscale),
        _ptr(y), M, N, K, _ptr(ws), wsb, _stream(stream)))
