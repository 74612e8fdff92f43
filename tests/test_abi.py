"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

from block_scaled_precision_fp8_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsfp8.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libbsfp8.so not built")

FAKE = 0x100000       # 16-byte aligned, never dereferenced by the checks
MIS = 0x100008        # misaligned


def declared():
    src = open(HEADER).read()
    return re.findall(r"BSFP8_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declarations_match_binding():
    names = declared()
    assert sorted(names) == sorted(L.EXPORTS)


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define\s+BSFP8_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES


def test_noalloc_argument_checks():
    """fp8_linear_noalloc shares fp8_linear's checks; a problem whose
    workspace exceeds the library's array is refused before any HIP call."""
    f = L.load().fp8_linear_noalloc
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 128, 128, 1, 0, None,
             None) == L.EINVAL
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 64, 64, 0, 0, None,
             None) == L.ENOTSUP
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 0, 256, 256, 128, 128, 0, 0, None,
             None) == L.OK
    M, N, K = 8192, 4096, 14336
    assert L.workspace_size(L.OP_LINEAR, M, N, K) > L.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, K, FAKE, FAKE, None, FAKE, M, N, K, 128, 128, 0, 0, None,
             None) == L.ENOSPC


def test_every_declared_symbol_exported():
    L.load()                      # the binding's load order (torch's HIP runtime first)
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def test_one_hip_runtime_in_process():
    """torch ships its own HIP runtime under the soname the library links;
    after load() the process must map exactly one libamdhip64 (two would
    run the kernels on a runtime that does not own torch's streams)."""
    L.load()
    import torch  # noqa: F401
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_version_and_status_strings():
    lib = L.load()
    assert lib.bsfp8_version() >= 100
    for s in range(5):
        assert L.status_string(s)
    assert L.status_string(99) == "unknown status"


def _qa(**kw):
    a = dict(x=FAKE, M=16, K=256, ldx=256, gk=128, sch=0, fmt=0, xq=FAKE, xs=FAKE, st=None)
    a.update(kw)
    return L.load().fp8_quant_act(a["x"], a["M"], a["K"], a["ldx"], a["gk"], a["sch"], a["fmt"],
                                  a["xq"], a["xs"], a["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), L.EINVAL), (dict(K=-16), L.EINVAL), (dict(K=200), L.EINVAL),
    (dict(ldx=128), L.EINVAL), (dict(ldx=260), L.EINVAL), (dict(fmt=2), L.EINVAL),
    (dict(sch=5), L.EINVAL), (dict(gk=0), L.EINVAL), (dict(gk=64), L.ENOTSUP),
    (dict(sch=1, M=0), L.OK), (dict(sch=1, xs=None), L.EINVAL),
    (dict(x=None), L.EINVAL), (dict(xq=None), L.EINVAL),
    (dict(xs=None), L.EINVAL), (dict(x=MIS), L.EINVAL), (dict(M=0), L.OK),
    (dict(M=0, x=None), L.OK),
])
def test_quant_act_argument_checks(kw, code):
    assert _qa(**kw) == code


def _qw(**kw):
    a = dict(w=FAKE, N=256, K=256, ldw=256, bn=128, bk=128, fmt=0, wq=FAKE, ws=FAKE)
    a.update(kw)
    return L.load().fp8_quant_weight(a["w"], a["N"], a["K"], a["ldw"], a["bn"], a["bk"],
                                     a["fmt"], a["wq"], a["ws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), L.EINVAL), (dict(K=8), L.EINVAL), (dict(bn=0), L.EINVAL),
    (dict(bk=-128), L.EINVAL), (dict(bn=64, bk=64), L.ENOTSUP), (dict(bn=32, bk=128), L.ENOTSUP), (dict(fmt=-1), L.EINVAL),
    (dict(wq=None), L.EINVAL), (dict(ws=MIS), L.EINVAL), (dict(N=0), L.OK),
])
def test_quant_weight_argument_checks(kw, code):
    assert _qw(**kw) == code


def _gemm(**kw):
    a = dict(xq=FAKE, xs=FAKE, wq=FAKE, ws=FAKE, b=None, y=FAKE, M=16, N=256, K=256, bn=128,
             bk=128, fmt=0, w=None, wb=0)
    a.update(kw)
    return L.load().fp8_block_gemm(a["xq"], a["xs"], a["wq"], a["ws"], a["b"], a["y"], a["M"],
                                   a["N"], a["K"], a["bn"], a["bk"], a["fmt"], a["w"], a["wb"],
                                   None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), L.EINVAL), (dict(N=12), L.EINVAL), (dict(K=100), L.EINVAL),
    (dict(fmt=3), L.EINVAL), (dict(bn=64), L.ENOTSUP), (dict(bk=0), L.EINVAL),
    (dict(y=None), L.EINVAL), (dict(wq=None), L.EINVAL), (dict(b=MIS), L.EINVAL),
    (dict(M=0), L.OK), (dict(N=0), L.EINVAL), (dict(M=2**31), L.EINVAL),
    (dict(K=2**22 + 16), L.ENOTSUP),
])
def test_block_gemm_argument_checks(kw, code):
    assert _gemm(**kw) == code


def test_block_gemm_workspace_too_small():
    need = L.workspace_size(L.OP_BLOCK_GEMM, 64, 4096, 4096)
    assert need > 0
    assert _gemm(M=64, N=4096, K=4096, w=FAKE, wb=need - 1) == L.ENOSPC
    assert _gemm(M=64, N=4096, K=4096, w=None, wb=need) == L.EINVAL


def test_decode_needs_no_workspace():
    """M <= 16 runs in one launch with no workspace; fp8_linear fuses the
    activation quantization there up to N K = 2^24 with K <= 6144, and with
    M K <= 40960 also on the persistent decode kernel's shapes (at least 384
    16-row tiles or 48 K blocks; below 4 rows two blocks per wave): X
    quantized once per workgroup.  Elsewhere it stages it (every workgroup
    of the per-block form would re-quantize all of X).  For M > 16 it fuses
    it into the large-M GEMM on 128 x 256 tiles."""
    for M in (1, 2, 3, 16):
        assert L.workspace_size(L.OP_BLOCK_GEMM, M, 28672, 4096) == 0
        assert L.workspace_size(L.OP_LINEAR, M, 4096, 4096) == 0
        assert L.workspace_size(L.OP_LINEAR, M, 2728, 6144) == 0
        assert L.workspace_size(L.OP_LINEAR, M, 4104, 4096) > 0   # 257 tiles of 32 blocks
        for (N, K) in ((1536, 7168), (8192, 4096), (4096, 14336), (7168, 18432)):
            fused = M * K <= 40960
            assert (L.workspace_size(L.OP_LINEAR, M, N, K) == 0) == fused, (M, N, K)
        # one block per wave and tile (K <= 2048): staged below 4 rows
        assert (L.workspace_size(L.OP_LINEAR, M, 24576, 1536) == 0) == (M >= 4)
    # M > 16 on the 128 x 256 tile with M K ceil(N / 256) <= 2^21: the GEMM
    # quantizes in its K loop, so the workspace is the K splits' partial
    # sums only (none here); otherwise the codes and scales are staged
    assert L.workspace_size(L.OP_LINEAR, 17, 256, 256) == 0
    for (M, N, K) in ((40, 1024, 1536), (32, 4096, 4096), (32, 1536, 7168)):
        assert L.gemm_kernel(M, N, K)[0] == L.GEMM_TILE_128x256
        assert L.workspace_size(L.OP_LINEAR, M, N, K) == L.workspace_size(L.OP_BLOCK_GEMM, M, N, K)
    for (M, N, K) in ((64, 4096, 4096), (128, 4096, 4096), (2048, 4096, 4096), (2048, 6144, 4096)):
        assert L.workspace_size(L.OP_LINEAR, M, N, K) >= M * K + L.workspace_size(
            L.OP_BLOCK_GEMM, M, N, K)


def test_linear_argument_checks():
    lib = L.load()
    f = lib.fp8_linear
    # static scheme: a calibrated scale is required (device pointer; fp32
    # scales 4-byte aligned), and it takes 128 x 128 blocks only
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 128, 128, 1, 0, None, FAKE,
             1 << 20, None) == L.EINVAL
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 128, 128, 1, 0, FAKE + 2, FAKE,
             1 << 20, None) == L.EINVAL
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 32, 32, 1, 0, FAKE, FAKE,
             1 << 20, None) == L.ENOTSUP
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 16, 256, 256, 128, 128, 2, 0, FAKE, FAKE,
             1 << 20, None) == L.EINVAL
    assert f(FAKE, 256, FAKE, FAKE, None, FAKE, 0, 256, 256, 128, 128, 1, 0, None, FAKE,
             1 << 20, None) == L.OK
    assert f(FAKE, 128, FAKE, FAKE, None, FAKE, 16, 256, 256, 128, 128, 0, 0, None, FAKE,
             1 << 20, None) == L.EINVAL
    need = L.workspace_size(L.OP_LINEAR, 2048, 6144, 4096)
    assert need > 0
    assert f(FAKE, 4096, FAKE, FAKE, None, FAKE, 2048, 6144, 4096, 128, 128, 0, 0, None, FAKE,
             need - 1, None) == L.ENOSPC
    assert f(FAKE, 4096, FAKE, FAKE, None, FAKE, 2048, 6144, 4096, 128, 128, 1, 1, FAKE + 1,
             FAKE, need - 1, None) == L.ENOSPC


def test_grouped_argument_checks():
    f = L.load().fp8_grouped_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 64, 256, 256, 128, 128, 0, None, 0, None]
    bad = list(args); bad[5] = 0
    assert f(*bad) == L.EINVAL
    bad = list(args); bad[5] = 1025
    assert f(*bad) == L.EINVAL
    bad = list(args); bad[4] = None
    assert f(*bad) == L.EINVAL
    bad = list(args); bad[12] = 7
    assert f(*bad) == L.EINVAL
    bad = list(args); bad[7] = 0
    assert f(*bad) == L.OK


def test_fp8_fp4_grouped_argument_checks():
    f = L.load().fp8_fp4_grouped_gemm
    #       xq    xs    wq4   ws    seg   E  y     T   N    K    fmt stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 64, 256, 256, 0, None]
    for i, v, code in [(5, 0, L.EINVAL), (5, 1025, L.EINVAL), (4, None, L.EINVAL),
                       (4, 0x100002, L.EINVAL), (9, 48, L.EINVAL), (9, 100, L.EINVAL),
                       (8, 12, L.EINVAL), (10, 2, L.EINVAL), (6, None, L.EINVAL),
                       (2, MIS, L.EINVAL), (9, 2**22 + 32, L.ENOTSUP), (7, 0, L.OK)]:
        a = list(args); a[i] = v
        assert f(*a) == code, (i, v)


def test_fp4_argument_checks():
    lib = L.load()
    assert lib.fp4_quant(FAKE, 4, 48, 1, FAKE, FAKE, FAKE, None, 0, None) == L.EINVAL
    assert lib.fp4_quant(FAKE, 4, 64, 2, FAKE, FAKE, FAKE, None, 0, None) == L.EINVAL
    assert lib.fp4_quant(FAKE, 0, 64, 1, FAKE, FAKE, FAKE, None, 0, None) == L.OK
    assert lib.fp4_group_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 48, None, 0,
                              None) == L.EINVAL
    assert lib.fp4_group_gemm(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, None, 0,
                              None) == L.EINVAL
    # K beyond 2^22: its 32-bit tile offsets would wrap (as the FP8 GEMMs)
    assert lib.fp4_group_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 2**22 + 32, None,
                              0, None) == L.ENOTSUP


def test_workspace_size_unknown_op():
    assert L.workspace_size(99, 1, 1, 16) == 2**64 - 1
    assert L.load().bsfp8_workspace_size(0, -1, 1, 16, 0) == 2**64 - 1


def test_gemm_kernel_choice():
    """Host-side kernel choice: the one-launch decode kernel up to M = 16,
    then the LDS MFMA kernel with the tile and K split picked by the cost
    model (rounds of workgroups over 256 CUs x per-K-block tile time, plus
    the partial sums of a split)."""
    k = L.gemm_kernel
    assert k(0, 256, 256)[0] == L.GEMM_NONE and k(5, 0, 256)[0] == L.GEMM_NONE
    assert L.load().bsfp8_gemm_kernel(-1, 8, 128, None) == -1
    for M in (1, 16):
        assert k(M, 28672, 4096) == (L.GEMM_DECODE, 1)
    # few output tiles: K is split so the grid covers the CUs
    kind, s = k(128, 4096, 4096)
    assert kind == L.GEMM_TILE_128x256 and s == 8
    kind, s = k(128, 28672, 4096)
    assert kind == L.GEMM_TILE_128x256 and s == 2
    # large problems: no split; 256 x 256 tiles once they fill the CUs
    assert k(2048, 4096, 4096) == (L.GEMM_TILE_128x256, 1)
    assert k(2048, 6144, 4096) == (L.GEMM_TILE_256x256, 1)
    for N in (4096, 6144, 28672):
        assert k(8192, N, 4096) == (L.GEMM_TILE_256x256, 1)
    assert k(4100, 4104, 384)[0] == L.GEMM_TILE_256x256     # the ragged big-tile parity case
    # the workspace is the partial sums of a split
    assert L.workspace_size(L.OP_BLOCK_GEMM, 128, 4096, 4096) == 8 * 128 * 4096 * 4
    assert L.workspace_size(L.OP_BLOCK_GEMM, 8192, 4096, 4096) == 0


def test_dequant_and_ue8m0_argument_checks():
    lib = L.load()
    d = lib.fp8_dequant_weight
    assert d(FAKE, -1, 256, 128, 128, 0, FAKE, FAKE, None) == L.EINVAL
    assert d(FAKE, 256, 200, 128, 128, 0, FAKE, FAKE, None) == L.EINVAL
    assert d(FAKE, 256, 256, 64, 128, 0, FAKE, FAKE, None) == L.ENOTSUP
    assert d(FAKE, 256, 256, 128, 128, 3, FAKE, FAKE, None) == L.EINVAL
    assert d(None, 256, 256, 128, 128, 0, FAKE, FAKE, None) == L.EINVAL
    assert d(FAKE, 256, 256, 128, 128, 0, FAKE, MIS, None) == L.EINVAL
    assert d(FAKE, 0, 256, 128, 128, 0, None, None, None) == L.OK
    c = lib.fp8_scale_to_ue8m0
    assert c(FAKE, -1, FAKE, None) == L.EINVAL
    assert c(None, 4, FAKE, None) == L.EINVAL
    assert c(FAKE, 0, None, None) == L.OK


def test_mxfp4_argument_checks():
    lib = L.load()
    q = lib.mxfp4_quant_weight
    assert q(FAKE, 4, 48, 48, FAKE, FAKE, None) == L.EINVAL          # K % 32
    assert q(FAKE, 4, 64, 60, FAKE, FAKE, None) == L.EINVAL          # ldw < K
    assert q(FAKE, 4, 64, 68, FAKE, FAKE, None) == L.EINVAL          # ldw % 8
    assert q(None, 4, 64, 64, FAKE, FAKE, None) == L.EINVAL
    assert q(MIS, 4, 64, 64, FAKE, FAKE, None) == L.EINVAL
    assert q(FAKE, -1, 64, 64, FAKE, FAKE, None) == L.EINVAL
    assert q(None, 0, 64, 64, None, None, None) == L.OK
    g = lib.fp8_fp4_gemm
    args = [FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 256, 256, 0, None, 0, None]
    for i, v, code in [(8, 48, L.EINVAL), (8, 2**22 + 32, L.ENOTSUP), (7, 12, L.EINVAL),
                       (9, 2, L.EINVAL), (2, None, L.EINVAL), (3, MIS, L.EINVAL),
                       (6, 0, L.OK), (6, -3, L.EINVAL)]:
        a = list(args); a[i] = v
        assert g(*a) == code, (i, v)
    # M > 16 may split K: the workspace is checked like the FP8 GEMM's
    need = L.workspace_size(L.OP_FP8_FP4_GEMM, 128, 4096, 4096)
    assert need > 0
    assert L.workspace_size(L.OP_FP8_FP4_GEMM, 16, 28672, 4096) == 0
    a = list(args); a[6:9] = [128, 4096, 4096]; a[10] = FAKE; a[11] = need - 1
    assert g(*a) == L.ENOSPC


def test_silu_mul_quant_argument_checks():
    f = L.load().fp8_grouped_gemm_silu_mul_quant
    #       xq    xs    wq    ws    seg   E  hq    hs    hb    T   I    K    fmt stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, None, 64, 256, 256, 0, None]
    for i, v, code in [(10, 0, L.EINVAL), (10, 192, L.EINVAL), (10, -128, L.EINVAL),
                       (5, 0, L.EINVAL), (5, 1025, L.EINVAL), (7, None, L.EINVAL),
                       (7, 0x100002, L.EINVAL), (8, MIS, L.EINVAL), (4, None, L.EINVAL),
                       (6, None, L.EINVAL), (6, MIS, L.EINVAL), (11, 200, L.EINVAL),
                       (12, 2, L.EINVAL), (11, 2**22 + 16, L.ENOTSUP), (9, 0, L.OK)]:
        a = list(args); a[i] = v
        assert f(*a) == code, (i, v)
    # one expert's gate/up weight (2 I K bytes) must stay below 2^31 bytes:
    # its rows are addressed with 32-bit offsets from one base
    a = list(args); a[10] = 2**17; a[11] = 2**13
    assert f(*a) == L.ENOTSUP
    a[11] = 2**13 - 16
    assert f(*a) != L.ENOTSUP


def test_block32_argument_checks():
    lib = L.load()
    # (32, 32) is accepted by the quantizers and the GEMM; mixed sizes are not
    assert _qw(bn=32, bk=128) == L.ENOTSUP and _qw(bn=64, bk=64) == L.ENOTSUP
    assert _qa(gk=32, sch=1) == L.ENOTSUP          # static scheme: 128 only
    assert _gemm(bn=32, bk=32, M=0) == L.OK and _gemm(bn=32, bk=64) == L.ENOTSUP
    g = lib.fp8_grouped_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 64, 256, 256, 32, 32, 0, None, 0, None]
    assert g(*args) == L.EHIP                      # (32, 32) experts: past the checks
    bad = list(args); bad[10] = 64; bad[11] = 64
    assert g(*bad) == L.ENOTSUP                    # other sizes
    bad = list(args); bad[10] = 32; bad[11] = 128
    assert g(*bad) == L.ENOTSUP                    # mixed sizes
    assert L.workspace_size(L.OP_LINEAR_B32, 64, 256, 256) >= 64 * 256 + 64 * 8 * 4
