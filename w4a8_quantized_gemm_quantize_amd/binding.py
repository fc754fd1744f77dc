"""Thin Python binding of libw4a8.so (C ABI in include/w4a8.h).

Argument marshalling only: torch tensors (device memory) become raw pointers,
the current torch stream becomes the hipStream_t, and a non-OK status raises.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  Importing this module loads the library and raises ImportError if
it has not been built (``python -m w4a8_quantized_gemm_quantize_amd.build_lib``
or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libw4a8.so is not built ({LIB_PATH}); run build_lib.py first")

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP, ERR_NONFINITE = range(7)
F32, BF16, I32 = 0, 1, 2
GROUP = 64
N_TILE = 16
K_MAX = 150976
LQQ_K_MAX = 133120

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGS = {
    "w4a8_abi_version": ([], ctypes.c_int32),
    "w4a8_pack_layout_version": ([], ctypes.c_int32),
    "w4a8_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "quantize_act_blockwise": ([_P, _I64, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "dequantize_act_blockwise": ([_P, _P, _I64, _I64, _I32, _P, ctypes.c_int, _P], ctypes.c_int),
    "pack_w4_grouped": ([_P, _I64, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "unpack_w4_grouped": ([_P, _P, _I64, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "w4a8_gemm": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P],
                  ctypes.c_int),
    "w4a8_gemm_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "w4a8_gemm_ws": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P,
                      ctypes.c_size_t, _P], ctypes.c_int),
    "w4a8_gemm_bf16act_workspace_bytes": ([_I64, _I64], ctypes.c_size_t),
    "w4a8_gemm_bf16act": ([_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P,
                           ctypes.c_size_t, _P], ctypes.c_int),
    "pack_w4_lqq": ([_P, _I64, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "unpack_w4_lqq": ([_P, _P, _I64, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "w4a8_gemm_lqq": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P],
                      ctypes.c_int),
    "w4a8_gemm_lqq_bf16act": ([_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P,
                               ctypes.c_size_t, _P], ctypes.c_int),
    "pack_w8_channel": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "unpack_w8_channel": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "w8a8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P], ctypes.c_int),
    "w8a8_gemm_bf16act": ([_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P, ctypes.c_size_t,
                           _P], ctypes.c_int),
    "w4a8_gemm_blockact": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, ctypes.c_int,
                            _P], ctypes.c_int),
    "dequant_add_requant": ([_P, _P, _P, ctypes.c_int, _I64, _I64, _I32, _P, _P, _P, _P],
                            ctypes.c_int),
    "w4a8_probe_mfma_i8": ([_I64, _I32, _P, _P, _P], ctypes.c_int),
    "w4a8_gemm_bf16act_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, ctypes.c_int, _P],
                                  ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class W4A8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def abi_version() -> int:
    return int(_lib.w4a8_abi_version())


def pack_layout_version() -> int:
    return int(_lib.w4a8_pack_layout_version())


def status_string(status: int) -> str:
    return _lib.w4a8_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _empty(stream, shape, dtype, device):
    """A new tensor for a call enqueued on `stream`.  Allocated under that stream,
    so torch's caching allocator does not hand the memory to work on another
    stream while the call's kernels may still use it (a workspace the binding
    creates is released when the call returns, before its kernels finish)."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _check(fn, status):
    if status != OK:
        raise W4A8Error(fn, status)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


class W4A8SizeError(W4A8Error):
    """A tensor argument holds fewer elements than the call's sizes need (raised
    before anything is launched; status W4A8_ERR_SHAPE)."""

    def __init__(self, fn: str, name: str, have: int, need: int):
        self.status = ERR_SHAPE
        RuntimeError.__init__(self, f"{fn}: {name} holds {have} elements, the call needs {need}")


_U8 = (torch.uint8, torch.int8)
_I16 = (torch.int16,)
_F32 = (torch.float32,)


def _sized(fn, t, dtypes, need, name):
    """The library takes raw pointers and cannot see buffer sizes: check that a
    tensor argument is a contiguous CUDA tensor of one of `dtypes` holding at
    least `need` elements.  None passes through (the library rejects a missing
    pointer itself)."""
    if t is None:
        return
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{fn}: {name} must be a contiguous CUDA tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} must be of dtype {' or '.join(map(str, dtypes))}, "
                         f"not {t.dtype}")
    if t.numel() < need:
        raise W4A8SizeError(fn, name, t.numel(), need)


def _per(total: int, block: int) -> int:
    return total // block if block > 0 else 0


def _gemm_args(fn, m, n, k, a_scale, w_packed, w_bytes_per_elem, params, param_dtypes,
               group, ch_scale, out):
    """Sizes of the GEMM operands: a_scale [m], weights n k w_bytes_per_elem bytes,
    group parameters [n, k / group] (if the format has them), ch_scale [n], out [m, n]."""
    _sized(fn, a_scale, _F32, m, "a_scale")
    _sized(fn, w_packed, _U8, (n * k * w_bytes_per_elem) // 2, "w_packed")
    if param_dtypes is not None:
        _sized(fn, params, param_dtypes, n * _per(k, group), "group parameters")
    _sized(fn, ch_scale, _F32, n, "ch_scale")
    _sized(fn, out, tuple(_OUT), m * n, "out")


# ------------------------------------------------------------ activations --

def quantize_act_blockwise(x: torch.Tensor, block: int, q=None, scales=None, stream=None):
    """x bf16 [rows, cols] -> (q int8 [rows, cols], scales f32 [rows, cols // block])."""
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if q is None:
        q = _empty(stream, (rows, cols), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = _empty(stream, (rows, cols // block if block > 0 else 0), dtype=torch.float32,
                             device=x.device)
    _sized("quantize_act_blockwise", q, (torch.int8,), rows * cols, "q")
    _sized("quantize_act_blockwise", scales, _F32, rows * _per(cols, block), "scales")
    _check("quantize_act_blockwise",
           _lib.quantize_act_blockwise(_ptr(x), rows, cols, block, _ptr(q), _ptr(scales),
                                       _stream(stream)))
    return q, scales


def dequantize_act_blockwise(q: torch.Tensor, scales: torch.Tensor, block: int,
                             out_dtype=torch.float32, out=None, stream=None):
    """-> x_hat [rows, cols] as float32 or bfloat16."""
    _dev(q, torch.int8, "q")
    _dev(scales, torch.float32, "scales")
    rows, cols = q.shape
    code = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if out is None:
        out = _empty(stream, (rows, cols), dtype=out_dtype, device=q.device)
    _sized("dequantize_act_blockwise", scales, _F32, rows * _per(cols, block), "scales")
    _sized("dequantize_act_blockwise", out, (out_dtype,), rows * cols, "out")
    _check("dequantize_act_blockwise",
           _lib.dequantize_act_blockwise(_ptr(q), _ptr(scales), rows, cols, block, _ptr(out),
                                         code, _stream(stream)))
    return out


# ---------------------------------------------------------------- weights --

def pack_w4_grouped(w: torch.Tensor, group: int = GROUP, stream=None):
    """w bf16 [n, k] -> (w_packed uint8 [n*k/2], grp_scale uint8 [n*k/group], ch_scale f32 [n])."""
    _dev(w, torch.bfloat16, "w")
    n, k = w.shape
    dev = w.device
    w_packed = _empty(stream, (n * k // 2,), dtype=torch.uint8, device=dev)
    grp_scale = _empty(stream, (n * (k // group) if group > 0 else 0,), dtype=torch.uint8,
                            device=dev)
    ch_scale = _empty(stream, (n,), dtype=torch.float32, device=dev)
    _check("pack_w4_grouped",
           _lib.pack_w4_grouped(_ptr(w), n, k, group, _ptr(w_packed), _ptr(grp_scale),
                                _ptr(ch_scale), _stream(stream)))
    return w_packed, grp_scale, ch_scale


def unpack_w4_grouped(w_packed, grp_scale, n: int, k: int, group: int = GROUP, stream=None):
    """Test hook: packed layout -> (q int8 [n, k], s_g uint8 [n, k/group]) canonical."""
    dev = w_packed.device
    q = _empty(stream, (n, k), dtype=torch.int8, device=dev)
    s_g = _empty(stream, (n, k // group), dtype=torch.uint8, device=dev)
    _sized("unpack_w4_grouped", w_packed, _U8, n * k // 2, "w_packed")
    _sized("unpack_w4_grouped", grp_scale, _U8, n * _per(k, group), "grp_scale")
    _check("unpack_w4_grouped",
           _lib.unpack_w4_grouped(_ptr(w_packed), _ptr(grp_scale), n, k, group, _ptr(q),
                                  _ptr(s_g), _stream(stream)))
    return q, s_g


# ------------------------------------------------------------------- GEMM --

_OUT = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32}


def w4a8_gemm(a_q, a_scale, w_packed, grp_scale, ch_scale, n: int, out_dtype=torch.bfloat16,
              group: int = GROUP, out=None, stream=None):
    """a_q int8 [m, k], a_scale f32 [m] -> out [m, n] (float32, bfloat16 or raw int32 acc)."""
    _dev(a_q, torch.int8, "a_q")
    m, k = a_q.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a_q.device)
    _gemm_args("w4a8_gemm", m, n, k, a_scale, w_packed, 1, grp_scale, _U8, group, ch_scale, out)
    _check("w4a8_gemm",
           _lib.w4a8_gemm(_ptr(a_q), _ptr(a_scale), _ptr(w_packed), _ptr(grp_scale),
                          _ptr(ch_scale), m, n, k, group, _ptr(out), _OUT[out.dtype],
                          _stream(stream)))
    return out


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    """Split-K scratch of w4a8_gemm_ws for an m x n x k product (0: not split)."""
    return int(_lib.w4a8_gemm_workspace_bytes(m, n, k))


def w4a8_gemm_ws(a_q, a_scale, w_packed, grp_scale, ch_scale, n: int,
                 out_dtype=torch.bfloat16, group: int = GROUP, out=None, workspace=None,
                 stream=None):
    """w4a8_gemm with a caller workspace that lets batches whose output tiles would
    not fill the GPU (5 <= m <= 64 where a split pays, or m > 64 with few tiles) split K
    (same result)."""
    _dev(a_q, torch.int8, "a_q")
    m, k = a_q.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a_q.device)
    need = gemm_workspace_bytes(m, n, k)
    if workspace is None and need > 0:
        workspace = _empty(stream, (need,), dtype=torch.uint8, device=a_q.device)
    _gemm_args("w4a8_gemm_ws", m, n, k, a_scale, w_packed, 1, grp_scale, _U8, group, ch_scale,
               out)
    _sized("w4a8_gemm_ws", workspace, _U8, 0, "workspace")
    _check("w4a8_gemm_ws",
           _lib.w4a8_gemm_ws(_ptr(a_q), _ptr(a_scale), _ptr(w_packed), _ptr(grp_scale),
                             _ptr(ch_scale), m, n, k, group, _ptr(out), _OUT[out.dtype],
                             _ptr(workspace), 0 if workspace is None else workspace.numel(),
                             _stream(stream)))
    return out


def workspace_bytes(m: int, k: int, n: int = None) -> int:
    """Workspace of the fused entry points: codes and scales, plus (given n) the
    split-K partials that let batches whose output tiles would not fill the GPU
    split K."""
    base = int(_lib.w4a8_gemm_bf16act_workspace_bytes(m, k))
    return base + (gemm_workspace_bytes(m, n, k) if n is not None else 0)


def w4a8_gemm_bf16act(a, w_packed, grp_scale, ch_scale, n: int, out_dtype=torch.bfloat16,
                      group: int = GROUP, out=None, workspace=None, stream=None):
    """a bf16 [m, k] -> out [m, n]; per-token quantization into `workspace` then the GEMM."""
    _dev(a, torch.bfloat16, "a")
    m, k = a.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a.device)
    need = workspace_bytes(m, k, n)
    if workspace is None:
        workspace = _empty(stream, (max(need, 16),), dtype=torch.uint8, device=a.device)
    _gemm_args("w4a8_gemm_bf16act", m, n, k, None, w_packed, 1, grp_scale, _U8, group, ch_scale,
               out)
    _sized("w4a8_gemm_bf16act", workspace, _U8, 0, "workspace")
    _check("w4a8_gemm_bf16act",
           _lib.w4a8_gemm_bf16act(_ptr(a), _ptr(w_packed), _ptr(grp_scale), _ptr(ch_scale), m,
                                  n, k, group, _ptr(out), _OUT[out.dtype], _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def w4a8_gemm_bf16act_noalloc(a, w_packed, grp_scale, ch_scale, n: int, out,
                              group: int = GROUP, stream=None):
    """w4a8_gemm_bf16act with the library's static device workspace: the caller
    passes `out` ([m, n] float32, bfloat16 or int32) and nothing is allocated.
    Calls that overlap on one GPU share that workspace and race."""
    _dev(a, torch.bfloat16, "a")
    m, k = a.shape
    _gemm_args("w4a8_gemm_bf16act_noalloc", m, n, k, None, w_packed, 1, grp_scale, _U8, group,
               ch_scale, out)
    _check("w4a8_gemm_bf16act_noalloc",
           _lib.w4a8_gemm_bf16act_noalloc(_ptr(a), _ptr(w_packed), _ptr(grp_scale),
                                          _ptr(ch_scale), m, n, k, group, _ptr(out),
                                          _OUT[out.dtype], _stream(stream)))
    return out


def workspace_views(workspace, m: int, k: int):
    """(a_q [m, k] int8, a_scale [m] f32) views of a w4a8_gemm_bf16act workspace."""
    off = (m * k + 255) // 256 * 256
    a_q = workspace[: m * k].view(torch.int8).view(m, k)
    a_s = workspace[off: off + 4 * m].view(torch.float32)
    return a_q, a_s


# ------------------------------------------------------------ LQQ weights --

def pack_w4_lqq(w: torch.Tensor, group: int = GROUP, stream=None):
    """w bf16 [n, k] -> (w_packed uint8 [n*k/2], grp_param int16 [n*k/group] holding
    uint16 s | (128 + min) << 8, ch_scale f32 [n])."""
    _dev(w, torch.bfloat16, "w")
    n, k = w.shape
    dev = w.device
    w_packed = _empty(stream, (n * k // 2,), dtype=torch.uint8, device=dev)
    grp_param = _empty(stream, (n * (k // group) if group > 0 else 0,), dtype=torch.int16,
                            device=dev)
    ch_scale = _empty(stream, (n,), dtype=torch.float32, device=dev)
    _check("pack_w4_lqq",
           _lib.pack_w4_lqq(_ptr(w), n, k, group, _ptr(w_packed), _ptr(grp_param),
                            _ptr(ch_scale), _stream(stream)))
    return w_packed, grp_param, ch_scale


def unpack_w4_lqq(w_packed, grp_param, n: int, k: int, group: int = GROUP, stream=None):
    """Test hook -> (q_u4 uint8 [n, k], s_u8 uint8 [n, k/group], w_min int8 [n, k/group])."""
    dev = w_packed.device
    q = _empty(stream, (n, k), dtype=torch.uint8, device=dev)
    s_u8 = _empty(stream, (n, k // group), dtype=torch.uint8, device=dev)
    w_min = _empty(stream, (n, k // group), dtype=torch.int8, device=dev)
    _sized("unpack_w4_lqq", w_packed, _U8, n * k // 2, "w_packed")
    _sized("unpack_w4_lqq", grp_param, _I16, n * _per(k, group), "grp_param")
    _check("unpack_w4_lqq",
           _lib.unpack_w4_lqq(_ptr(w_packed), _ptr(grp_param), n, k, group, _ptr(q),
                              _ptr(s_u8), _ptr(w_min), _stream(stream)))
    return q, s_u8, w_min


def w4a8_gemm_lqq(a_q, a_scale, w_packed, grp_param, ch_scale, n: int,
                  out_dtype=torch.bfloat16, group: int = GROUP, out=None, stream=None):
    _dev(a_q, torch.int8, "a_q")
    m, k = a_q.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a_q.device)
    _gemm_args("w4a8_gemm_lqq", m, n, k, a_scale, w_packed, 1, grp_param, _I16, group,
               ch_scale, out)
    _check("w4a8_gemm_lqq",
           _lib.w4a8_gemm_lqq(_ptr(a_q), _ptr(a_scale), _ptr(w_packed), _ptr(grp_param),
                              _ptr(ch_scale), m, n, k, group, _ptr(out), _OUT[out.dtype],
                              _stream(stream)))
    return out


def w4a8_gemm_lqq_bf16act(a, w_packed, grp_param, ch_scale, n: int, out_dtype=torch.bfloat16,
                          group: int = GROUP, out=None, workspace=None, stream=None):
    _dev(a, torch.bfloat16, "a")
    m, k = a.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a.device)
    if workspace is None:
        workspace = _empty(stream, (max(workspace_bytes(m, k, n), 16),), dtype=torch.uint8,
                                device=a.device)
    _gemm_args("w4a8_gemm_lqq_bf16act", m, n, k, None, w_packed, 1, grp_param, _I16, group,
               ch_scale, out)
    _sized("w4a8_gemm_lqq_bf16act", workspace, _U8, 0, "workspace")
    _check("w4a8_gemm_lqq_bf16act",
           _lib.w4a8_gemm_lqq_bf16act(_ptr(a), _ptr(w_packed), _ptr(grp_param), _ptr(ch_scale),
                                      m, n, k, group, _ptr(out), _OUT[out.dtype],
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


# ------------------------------------------------------------------ W8A8 --

def pack_w8_channel(w: torch.Tensor, stream=None):
    """w bf16 [n, k] -> (w_packed int8 [n*k] tiled layout, ch_scale f32 [n])."""
    _dev(w, torch.bfloat16, "w")
    n, k = w.shape
    w_packed = _empty(stream, (n * k,), dtype=torch.int8, device=w.device)
    ch_scale = _empty(stream, (n,), dtype=torch.float32, device=w.device)
    _check("pack_w8_channel",
           _lib.pack_w8_channel(_ptr(w), n, k, _ptr(w_packed), _ptr(ch_scale), _stream(stream)))
    return w_packed, ch_scale


def unpack_w8_channel(w_packed, n: int, k: int, stream=None):
    q8 = _empty(stream, (n, k), dtype=torch.int8, device=w_packed.device)
    _sized("unpack_w8_channel", w_packed, _U8, n * k, "w_packed")
    _check("unpack_w8_channel",
           _lib.unpack_w8_channel(_ptr(w_packed), n, k, _ptr(q8), _stream(stream)))
    return q8


def w8a8_gemm(a_q, a_scale, w_packed, ch_scale, n: int, out_dtype=torch.bfloat16, out=None,
              stream=None):
    _dev(a_q, torch.int8, "a_q")
    m, k = a_q.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a_q.device)
    _gemm_args("w8a8_gemm", m, n, k, a_scale, w_packed, 2, None, None, GROUP, ch_scale, out)
    _check("w8a8_gemm",
           _lib.w8a8_gemm(_ptr(a_q), _ptr(a_scale), _ptr(w_packed), _ptr(ch_scale), m, n, k,
                          _ptr(out), _OUT[out.dtype], _stream(stream)))
    return out


def w8a8_gemm_bf16act(a, w_packed, ch_scale, n: int, out_dtype=torch.bfloat16, out=None,
                      workspace=None, stream=None):
    _dev(a, torch.bfloat16, "a")
    m, k = a.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a.device)
    if workspace is None:
        workspace = _empty(stream, (max(workspace_bytes(m, k, n), 16),), dtype=torch.uint8,
                                device=a.device)
    _gemm_args("w8a8_gemm_bf16act", m, n, k, None, w_packed, 2, None, None, GROUP, ch_scale, out)
    _sized("w8a8_gemm_bf16act", workspace, _U8, 0, "workspace")
    _check("w8a8_gemm_bf16act",
           _lib.w8a8_gemm_bf16act(_ptr(a), _ptr(w_packed), _ptr(ch_scale), m, n, k, _ptr(out),
                                  _OUT[out.dtype], _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
    return out


# ------------------------------------------ per-block activation scales GEMM --

def w4a8_gemm_blockact(a_q, a_scale, w_packed, grp_scale, ch_scale, n: int, block: int,
                       out_dtype=torch.bfloat16, group: int = GROUP, out=None, stream=None):
    """a_q int8 [m, k], a_scale f32 [m, k / block] -> out [m, n] (float32 or bfloat16)."""
    _dev(a_q, torch.int8, "a_q")
    _dev(a_scale, torch.float32, "a_scale")
    m, k = a_q.shape
    if out is None:
        out = _empty(stream, (m, n), dtype=out_dtype, device=a_q.device)
    _gemm_args("w4a8_gemm_blockact", 0, n, k, None, w_packed, 1, grp_scale, _U8, group,
               ch_scale, out)
    _sized("w4a8_gemm_blockact", a_scale, _F32, m * _per(k, block), "a_scale")
    _sized("w4a8_gemm_blockact", out, tuple(_OUT), m * n, "out")
    _check("w4a8_gemm_blockact",
           _lib.w4a8_gemm_blockact(_ptr(a_q), _ptr(a_scale), _ptr(w_packed), _ptr(grp_scale),
                                   _ptr(ch_scale), m, n, k, group, block, _ptr(out),
                                   _OUT[out.dtype], _stream(stream)))
    return out


# ---------------------------------------------------- EQuARX receive step --

def dequant_add_requant(q_in, s_in, x, block: int, want_sum: bool = False, q_out=None,
                        s_out=None, sum_out=None, stream=None):
    """(q_in int8 [r, c], s_in f32 [r, c/block]) + x (float32 or bfloat16 [r, c])
    -> (q_out int8, s_out f32, sum f32 or None): requantized per block."""
    _dev(q_in, torch.int8, "q_in")
    _dev(s_in, torch.float32, "s_in")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    _dev(x, x.dtype, "x")
    rows, cols = q_in.shape
    dev = q_in.device
    if q_out is None:
        q_out = _empty(stream, (rows, cols), dtype=torch.int8, device=dev)
    if s_out is None:
        s_out = _empty(stream, (rows, cols // block if block > 0 else 0), dtype=torch.float32,
                            device=dev)
    if want_sum and sum_out is None:
        sum_out = _empty(stream, (rows, cols), dtype=torch.float32, device=dev)
    fn = "dequant_add_requant"
    _sized(fn, s_in, _F32, rows * _per(cols, block), "s_in")
    _sized(fn, x, (x.dtype,), rows * cols, "x")
    _sized(fn, q_out, (torch.int8,), rows * cols, "q_out")
    _sized(fn, s_out, _F32, rows * _per(cols, block), "s_out")
    _sized(fn, sum_out, _F32, rows * cols, "sum_out")
    _check("dequant_add_requant",
           _lib.dequant_add_requant(_ptr(q_in), _ptr(s_in), _ptr(x),
                                    BF16 if x.dtype == torch.bfloat16 else F32, rows, cols,
                                    block, _ptr(sum_out), _ptr(q_out), _ptr(s_out),
                                    _stream(stream)))
    return q_out, s_out, sum_out


# -------------------------------------------------------- measurement aid --

def probe_mfma_i8(workgroups: int, iters: int, device=None, stream=None):
    """Int8 matrix-core reference loop: returns (ops, sink, clocks) where ops is
    the int8 operation count of the launch and clocks (after the stream is
    synchronized) holds [shader clock ticks, 100 MHz real-time ticks]."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    sink = _empty(stream, (workgroups * 512,), dtype=torch.int32, device=dev)
    clocks = _empty(stream, (2,), dtype=torch.int64, device=dev)
    _check("w4a8_probe_mfma_i8",
           _lib.w4a8_probe_mfma_i8(workgroups, iters, _ptr(sink), _ptr(clocks), _stream(stream)))
    return workgroups * iters * 4194304, sink, clocks
