"""Host-side checks of libw4a8.so: it loads, exports every function include/w4a8.h
declares, and rejects invalid arguments before launching anything.

No GPU work happens here: every call below fails validation (or is an empty
no-op) before the library touches the HIP runtime's launch path; fake pointers
are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")
LIB = os.path.join(ROOT, "w4a8_quantized_gemm_quantize_amd", "libw4a8.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP, ERR_NONFINITE = range(7)

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libw4a8.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.quantize_act_blockwise.argtypes = [P, I64, I64, I32, P, P, P]
    L.dequantize_act_blockwise.argtypes = [P, P, I64, I64, I32, P, ctypes.c_int, P]
    L.pack_w4_grouped.argtypes = [P, I64, I64, I32, P, P, P, P]
    L.unpack_w4_grouped.argtypes = [P, P, I64, I64, I32, P, P, P]
    L.w4a8_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I32, P, ctypes.c_int, P]
    L.w4a8_gemm_bf16act.argtypes = [P, P, P, P, I64, I64, I64, I32, P, ctypes.c_int, P,
                                    ctypes.c_size_t, P]
    L.w4a8_gemm_bf16act_workspace_bytes.argtypes = [I64, I64]
    L.w4a8_gemm_bf16act_workspace_bytes.restype = ctypes.c_size_t
    L.w4a8_status_string.restype = ctypes.c_char_p
    return L


A = ctypes.c_void_p(0x10000)       # aligned fake device pointers: never dereferenced
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
D = ctypes.c_void_p(0x40000)
E = ctypes.c_void_p(0x50000)
MIS = ctypes.c_void_p(0x10008)     # 8-byte aligned only
NUL = None


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["quantize_act_blockwise", "dequantize_act_blockwise", "pack_w4_grouped",
                 "unpack_w4_grouped", "w4a8_gemm", "w4a8_gemm_bf16act",
                 "w4a8_gemm_bf16act_workspace_bytes", "w4a8_gemm_workspace_bytes",
                 "w4a8_gemm_ws", "w4a8_abi_version",
                 "w4a8_pack_layout_version", "w4a8_status_string"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_versions_and_status_strings(lib):
    assert lib.w4a8_abi_version() == 1
    assert lib.w4a8_pack_layout_version() == 1
    seen = set()
    for s in range(7):
        txt = lib.w4a8_status_string(s).decode()
        assert txt and txt not in seen
        seen.add(txt)
    assert lib.w4a8_status_string(99)


def test_quantize_validation(lib):
    q = lib.quantize_act_blockwise
    assert q(A, -1, 64, 32, B, C, NUL) == ERR_SHAPE
    assert q(A, 4, 64, 12, B, C, NUL) == ERR_SHAPE        # block not a multiple of 8
    assert q(A, 4, 64, 0, B, C, NUL) == ERR_SHAPE
    assert q(A, 4, 96, 64, B, C, NUL) == ERR_SHAPE        # cols not a multiple of block
    assert q(NUL, 4, 64, 32, B, C, NUL) == ERR_NULL
    assert q(A, 4, 64, 32, NUL, C, NUL) == ERR_NULL
    assert q(A, 4, 64, 32, B, NUL, NUL) == ERR_NULL
    assert q(MIS, 4, 64, 32, B, C, NUL) == ERR_MISALIGNED
    assert q(A, 4, 64, 32, B, MIS, NUL) == ERR_MISALIGNED
    assert q(NUL, 0, 64, 32, NUL, NUL, NUL) == OK          # empty: nothing to do


def test_dequantize_validation(lib):
    d = lib.dequantize_act_blockwise
    assert d(A, B, 4, 64, 32, C, 2, NUL) == ERR_UNSUPPORTED   # int32 output not defined
    assert d(A, B, 4, 64, 24, C, 0, NUL) == ERR_SHAPE
    assert d(A, NUL, 4, 64, 32, C, 0, NUL) == ERR_NULL
    assert d(A, B, 4, 64, 32, MIS, 1, NUL) == ERR_MISALIGNED
    assert d(NUL, NUL, 0, 64, 32, NUL, 0, NUL) == OK


def test_pack_validation(lib):
    p = lib.pack_w4_grouped
    assert p(A, 32, 256, 128, B, C, D, NUL) == ERR_UNSUPPORTED   # group 128
    assert p(A, 17, 256, 64, B, C, D, NUL) == ERR_SHAPE          # n not a multiple of 16
    assert p(A, 32, 96, 64, B, C, D, NUL) == ERR_SHAPE           # k not a multiple of 64
    assert p(A, 32, 256, 64, NUL, C, D, NUL) == ERR_NULL
    assert p(A, 32, 256, 64, B, C, MIS, NUL) == ERR_MISALIGNED
    assert p(NUL, 0, 256, 64, NUL, NUL, NUL, NUL) == OK
    u = lib.unpack_w4_grouped
    assert u(A, B, 32, 256, 32, C, D, NUL) == ERR_UNSUPPORTED
    assert u(A, B, 32, 256, 64, NUL, D, NUL) == ERR_NULL


def test_gemm_validation(lib):
    g = lib.w4a8_gemm
    assert g(A, B, C, D, E, 8, 64, 256, 128, A, 0, NUL) == ERR_UNSUPPORTED  # group
    assert g(A, B, C, D, E, 8, 60, 256, 64, A, 0, NUL) == ERR_SHAPE        # n % 16
    assert g(A, B, C, D, E, 8, 64, 200, 64, A, 0, NUL) == ERR_SHAPE        # k % 64
    assert g(A, B, C, D, E, -1, 64, 256, 64, A, 0, NUL) == ERR_SHAPE
    assert g(A, B, C, D, E, 8, 64, 150976 + 64, 64, A, 0, NUL) == ERR_UNSUPPORTED  # K_MAX
    assert g(A, B, C, D, E, 8, 64, 256, 64, A, 7, NUL) == ERR_UNSUPPORTED  # out dtype
    assert g(NUL, B, C, D, E, 8, 64, 256, 64, A, 0, NUL) == ERR_NULL
    assert g(A, NUL, C, D, E, 8, 64, 256, 64, A, 0, NUL) == ERR_NULL
    assert g(A, B, C, D, NUL, 8, 64, 256, 64, A, 0, NUL) == ERR_NULL
    assert g(A, B, C, D, E, 8, 64, 256, 64, NUL, 0, NUL) == ERR_NULL
    assert g(A, B, MIS, D, E, 8, 64, 256, 64, A, 0, NUL) == ERR_MISALIGNED
    assert g(NUL, NUL, NUL, NUL, NUL, 0, 64, 256, 64, NUL, 1, NUL) == OK   # m == 0


def test_bf16act_workspace_and_validation(lib):
    ws = lib.w4a8_gemm_bf16act_workspace_bytes
    assert ws(8, 4096) == 8 * 4096 + 256
    assert ws(3, 64) == 256 + 256
    assert ws(0, 64) == 0
    f = lib.w4a8_gemm_bf16act
    need = ws(8, 4096)
    assert f(A, B, C, D, 8, 64, 4096, 64, E, 1, A, need - 1, NUL) == ERR_SHAPE
    assert f(A, B, C, D, 8, 64, 4096, 64, E, 1, NUL, need, NUL) == ERR_NULL
    assert f(A, B, C, D, 8, 64, 4096, 64, E, 1, MIS, need, NUL) == ERR_MISALIGNED
    assert f(A, B, C, D, 8, 64, 0, 64, E, 1, A, need, NUL) == ERR_SHAPE    # k == 0
    assert f(A, B, C, D, 8, 64, 4096, 32, E, 1, A, need, NUL) == ERR_UNSUPPORTED


def splitk_small_pays(m, n, k, s):
    """The modelled times of the two small-batch paths, restated in exact
    integers (ns scaled by 256 and by 1000): split when
    (7400 + 360 C max(256, G) / 256) < 0.9 (1500 + R k (300 + 28 m) / 1000)
    with C chunks per slice, G = S ceil(n / 128) split workgroups and R rounds
    of 256 one-pass workgroups (one 16-channel tile each, two for m > 32 with
    at least 512 tiles)."""
    chunks = -(-(k // 128) // s)
    wgs = -(-n // 128) * s
    t_split = 7400 * 256 + 360 * chunks * max(wgs, 256)
    tiles = n // 16
    per_wg = 2 if (m > 32 and tiles >= 512) else 1
    rounds = -(-(-(-tiles // per_wg)) // 256)
    t_one = 1500 * 1000 + rounds * k * (300 + 28 * m)
    return t_split * 10000 < t_one * 2304


def splitk_bytes_expected(m, n, k):
    """Split-K scratch size restated from its definition, for at least two whole
    128-wide chunks:
    - 5 <= m <= 64: S = min(ceil(512 / ceil(n / 128)), k // 128, 16); for
      16 < m with 32 S m <= k that S, otherwise S cut to k // (32 m) and split
      only if S >= 2 and the small-batch model favours it;
    - m > 64: S = min(256 // (ceil(m / 128) ceil(n / 256)), cap, (k // 128) // 4,
      16) with cap = k // (8 m), raised to (64 MiB) // (8 m n) where k >= 4096,
      or k >= 2048 with at most 32 tiles; split only if S >= 2;
    one int32 [m, n] slice per slice of K actually used."""
    if m < 5 or k < 256:
        return 0
    nfull = k // 128
    if m > 64:
        tiles = -(-m // 128) * -(-n // 256)
        cap = k // (8 * m)
        if nfull >= 32 or (nfull >= 16 and tiles <= 32):
            cap = max(cap, (64 << 20) // (8 * m * n))
        s = min(256 // tiles, cap, nfull // 4, 16)
        if s < 2:
            return 0
    else:
        s = min(-(-512 // -(-n // 128)), nfull, 16)
        if not (m > 16 and 32 * s * m <= k):
            s = min(s, k // (32 * m))
            if s < 2 or not splitk_small_pays(m, n, k, s):
                return 0
        elif s < 2:
            return 0
    kslice = -(-nfull // s) * 128
    return -(-k // kslice) * m * n * 4


def test_gemm_ws_workspace_and_validation(lib):
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    ws = lib.w4a8_gemm_workspace_bytes
    ws.argtypes = [I64, I64, I64]
    ws.restype = ctypes.c_size_t
    for m, n, k in [(64, 8192, 28672), (37, 8192, 1088), (17, 256, 4096), (64, 48, 512),
                    (16, 8192, 28672), (65, 8192, 4096), (40, 4096, 128), (0, 64, 256),
                    (33, 8208, 640), (20, 16384, 2624), (17, 32768, 1216),
                    (64, 28672, 8192), (24, 14352, 4096), (48, 8192, 8192), (17, 256, 10304)]:
        assert ws(m, n, k) == splitk_bytes_expected(m, n, k), (m, n, k)
    assert ws(64, 8192, 28672) == 8 * 64 * 8192 * 4       # 8 slices of 28 chunks
    assert ws(20, 16384, 2624) == 5 * 20 * 16384 * 4      # 4 x 5 chunks + a half-chunk slice
    assert ws(17, 256, 10304) == 17 * 17 * 256 * 4        # 16 x 5 chunks + a half-chunk slice
    assert ws(48, 8192, 8192) == 5 * 48 * 8192 * 4        # S cut from 8 to 5, modelled faster
    assert ws(24, 4096, 4096) == 0                        # cut to 5 slices: one pass is faster
    assert ws(64, 8192, 4096) == 0
    assert ws(16, 8192, 28672) == 8 * 16 * 8192 * 4       # a decode batch at large K
    assert ws(16, 4096, 14336) == 0                       # one round of one-pass workgroups
    assert ws(16, 1024, 28672) == 16 * 16 * 1024 * 4      # few channels leave CUs idle
    assert ws(4, 8192, 65536) == 0                        # m < 5 never splits
    assert ws(128, 8192, 28672) == 8 * 128 * 8192 * 4     # 32 tiles of 128 x 256: 8 slices
    assert ws(512, 8192, 28672) == 2 * 512 * 8192 * 4
    assert ws(512, 4096, 4096) == 4 * 512 * 4096 * 4      # partials within 64 MiB
    assert ws(512, 4096, 2048) == 0                       # k = 2048 with 64 tiles
    assert ws(256, 2048, 2048) == 4 * 256 * 2048 * 4      # k = 2048 with 16 tiles
    assert ws(1024, 8192, 28672) == 0                     # 256 tiles fill the CUs
    assert ws(4096, 14336, 4096) == 0
    # the rule over seeded random shapes around its edges (m range, half chunks,
    # the 16-slice cap, the 32 S m <= k cut, the modelled choice)
    rng = np.random.default_rng(7)
    for _ in range(2000):
        m = int(rng.integers(0, 80)) if rng.random() < 0.6 else int(rng.integers(64, 1100))
        n = 16 * int(rng.integers(1, 2400))
        k = 64 * int(rng.integers(1, 600))
        assert ws(m, n, k) == splitk_bytes_expected(m, n, k), (m, n, k)
    g = lib.w4a8_gemm_ws
    g.argtypes = [P, P, P, P, P, I64, I64, I64, I32, P, ctypes.c_int, P, ctypes.c_size_t, P]
    need = ws(64, 8192, 28672)
    assert need > 0
    assert g(A, B, C, D, E, 64, 8192, 28672, 64, A, 1, NUL, need, NUL) == ERR_NULL
    assert g(A, B, C, D, E, 64, 8192, 28672, 64, A, 1, MIS, need, NUL) == ERR_MISALIGNED
    assert g(A, B, C, D, E, 64, 8192, 28672, 64, A, 1, A, need - 1, NUL) == ERR_SHAPE
    assert g(A, B, C, D, E, 64, 8192, 28672, 128, A, 1, A, need, NUL) == ERR_UNSUPPORTED
    assert g(NUL, NUL, NUL, NUL, NUL, 0, 64, 256, 64, NUL, 1, NUL, 0, NUL) == OK   # m == 0


@pytest.fixture(scope="module")
def ext(lib):
    P, I64, I32, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.pack_w4_lqq.argtypes = [P, I64, I64, I32, P, P, P, P]
    lib.unpack_w4_lqq.argtypes = [P, P, I64, I64, I32, P, P, P, P]
    lib.w4a8_gemm_lqq.argtypes = [P, P, P, P, P, I64, I64, I64, I32, P, INT, P]
    lib.w4a8_gemm_lqq_bf16act.argtypes = [P, P, P, P, I64, I64, I64, I32, P, INT, P,
                                          ctypes.c_size_t, P]
    lib.pack_w8_channel.argtypes = [P, I64, I64, P, P, P]
    lib.unpack_w8_channel.argtypes = [P, I64, I64, P, P]
    lib.w8a8_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, INT, P]
    lib.w8a8_gemm_bf16act.argtypes = [P, P, P, I64, I64, I64, P, INT, P, ctypes.c_size_t, P]
    lib.w4a8_gemm_blockact.argtypes = [P, P, P, P, P, I64, I64, I64, I32, I32, P, INT, P]
    lib.dequant_add_requant.argtypes = [P, P, P, INT, I64, I64, I32, P, P, P, P]
    return lib


def test_extension_entry_points_declared():
    names = declared_functions()
    for want in ["pack_w4_lqq", "unpack_w4_lqq", "w4a8_gemm_lqq", "w4a8_gemm_lqq_bf16act",
                 "pack_w8_channel", "unpack_w8_channel", "w8a8_gemm", "w8a8_gemm_bf16act",
                 "w4a8_gemm_blockact", "dequant_add_requant"]:
        assert want in names


def test_lqq_validation(ext):
    lqq_kmax = 133120
    assert lqq_kmax == (2**31 - 1) // (127 * 127) // 64 * 64
    p = ext.pack_w4_lqq
    assert p(A, 32, 256, 128, B, C, D, NUL) == ERR_UNSUPPORTED
    assert p(A, 20, 256, 64, B, C, D, NUL) == ERR_SHAPE
    assert p(A, 32, 256, 64, B, NUL, D, NUL) == ERR_NULL
    assert p(A, 32, 256, 64, B, MIS, D, NUL) == ERR_MISALIGNED
    u = ext.unpack_w4_lqq
    assert u(A, B, 32, 256, 64, C, D, NUL, NUL) == ERR_NULL
    g = ext.w4a8_gemm_lqq
    # the W4 bound (150976) is too large for LQQ operands: the LQQ bound applies
    assert g(A, B, C, D, E, 8, 64, lqq_kmax + 64, 64, A, 0, NUL) == ERR_UNSUPPORTED
    assert g(A, B, C, NUL, E, 8, 64, 256, 64, A, 0, NUL) == ERR_NULL
    f = ext.w4a8_gemm_lqq_bf16act
    need = ext.w4a8_gemm_bf16act_workspace_bytes(8, 256)
    assert f(A, B, C, D, 8, 64, 256, 64, E, 1, A, need - 1, NUL) == ERR_SHAPE
    assert f(A, B, C, D, 8, 64, lqq_kmax + 64, 64, E, 1, A, 1 << 30, NUL) == ERR_UNSUPPORTED


def test_w8a8_validation(ext):
    assert ext.pack_w8_channel(A, 24, 256, B, C, NUL) == ERR_SHAPE
    assert ext.pack_w8_channel(A, 32, 256, NUL, C, NUL) == ERR_NULL
    assert ext.unpack_w8_channel(A, 32, 100, B, NUL) == ERR_SHAPE
    g = ext.w8a8_gemm
    assert g(A, B, C, D, 8, 64, 133120 + 64, E, 0, NUL) == ERR_UNSUPPORTED
    assert g(A, B, NUL, D, 8, 64, 256, E, 0, NUL) == ERR_NULL
    assert g(A, B, C, D, 8, 64, 256, MIS, 0, NUL) == ERR_MISALIGNED
    assert g(NUL, NUL, NUL, NUL, 0, 64, 256, NUL, 1, NUL) == OK


def test_blockact_validation(ext):
    g = ext.w4a8_gemm_blockact
    assert g(A, B, C, D, E, 8, 64, 256, 64, 48, A, 0, NUL) == ERR_UNSUPPORTED   # block 48
    assert g(A, B, C, D, E, 8, 64, 256, 64, 256, A, 0, NUL) == ERR_UNSUPPORTED  # block 256
    assert g(A, B, C, D, E, 8, 64, 192, 64, 128, A, 0, NUL) == ERR_SHAPE        # 192 % 128
    assert g(A, B, C, D, E, 8, 64, 256, 64, 64, A, 2, NUL) == ERR_UNSUPPORTED   # int32 out
    assert g(A, NUL, C, D, E, 8, 64, 256, 64, 64, A, 0, NUL) == ERR_NULL


def test_dequant_add_requant_validation(ext):
    f = ext.dequant_add_requant
    assert f(A, B, C, 0, 4, 64, 48, D, E, A, NUL) == ERR_SHAPE       # 64 % 48
    assert f(A, B, C, 2, 4, 64, 32, D, E, A, NUL) == ERR_UNSUPPORTED  # int32 partial sums
    assert f(A, B, NUL, 0, 4, 64, 32, D, E, A, NUL) == ERR_NULL
    assert f(A, B, C, 1, 4, 64, 32, MIS, E, A, NUL) == ERR_MISALIGNED  # sum_out misaligned


def test_mfma_probe_validation(lib):
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = lib.w4a8_probe_mfma_i8
    f.argtypes = [I64, I32, P, P, P]
    assert f(0, 10, A, B, NUL) == ERR_SHAPE
    assert f(65536, 10, A, B, NUL) == ERR_SHAPE
    assert f(256, 0, A, B, NUL) == ERR_SHAPE
    assert f(256, 10, NUL, B, NUL) == ERR_NULL
    assert f(256, 10, A, MIS, NUL) == ERR_MISALIGNED


def test_noalloc_validation(lib):
    # shape and size errors are returned before the device is touched
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = lib.w4a8_gemm_bf16act_noalloc
    f.argtypes = [P, P, P, P, I64, I64, I64, I32, P, ctypes.c_int, P]
    assert f(A, B, C, D, 8, 64, 0, 64, E, 1, NUL) == ERR_SHAPE
    assert f(A, B, C, D, -1, 64, 256, 64, E, 1, NUL) == ERR_SHAPE
    assert f(A, B, C, D, 0, 64, 256, 64, E, 1, NUL) == OK
    assert f(A, B, C, D, 4096, 64, 32768, 64, E, 1, NUL) == ERR_UNSUPPORTED  # 128 MiB of codes
    assert f(A, NUL, C, D, 8, 64, 256, 64, E, 1, NUL) == ERR_NULL
    assert f(A, B, C, D, 8, 64, 256, 64, MIS, 1, NUL) == ERR_MISALIGNED
