"""ctypes binding of libqgemv.so (C ABI in include/qgemv.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Functions keep the C names; buffer arguments accept
torch tensors (device pointers taken with ``data_ptr()``) or raw integer
device addresses.  A negative status raises :class:`QgemvError`.

If the library has not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

PATH_AUTO = 0
PATH_DOT = 1
PATH_MFMA = 2
_PATHS = {"auto": PATH_AUTO, "dot": PATH_DOT, "mfma": PATH_MFMA}

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EALIGN = -3
EHIP = -4

FMT_MXFP4 = 1
FMT_NVFP4 = 2
FMT_MXFP8 = 3
_FMTS = {"mxfp4": FMT_MXFP4, "nvfp4": FMT_NVFP4, "mxfp8": FMT_MXFP8}

MAX_M = 16
MAX_K = 131072
MAX_N = 4194304
MAX_EXPERTS = 4096
MAX_PAIRS = 256

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemv.so")

_lib = None


class QgemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {qgemv_strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libqgemv.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m few_row_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        gemv = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.qgemv_small.argtypes = gemv
        L.qgemv_run_path.argtypes = [i] + gemv
        gemv_add = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.qgemv_small_add.argtypes = gemv_add
        L.qgemv_run_path_add.argtypes = [i] + gemv_add
        L.qgemv_select.argtypes = [i, i, i, i, i]
        L.qgemv_gather.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        gemv_fp = [vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.qgemv_small_fp.argtypes = gemv_fp
        L.qgemv_run_path_fp.argtypes = [i] + gemv_fp
        L.qgemv_select_fp.argtypes = [i, i, i, i]
        L.qgemv_path_supported_fp.argtypes = [i, i, i, i, i]
        L.qgemv_unpack_probe_fp.argtypes = [i, vp, vp, i, i, i, vp]
        L.qgemv_path_supported.argtypes = [i, i, i, i, i, i]
        L.qgemv_unpack_probe.argtypes = [i, vp, vp, i, i, i, i, vp]
        L.qgemv_stream_probe.argtypes = [vp, u64, vp, i, i, vp]
        L.qgemv_stream_probe_blocks.argtypes = [u64]
        L.qgemv_strerror.argtypes = [i]
        L.qgemv_strerror.restype = ctypes.c_char_p
        L.qgemv_version.argtypes = []
        for name in ("qgemv_small", "qgemv_run_path", "qgemv_small_add", "qgemv_run_path_add",
                     "qgemv_small_fp", "qgemv_run_path_fp", "qgemv_select_fp", "qgemv_gather",
                     "qgemv_path_supported_fp", "qgemv_unpack_probe_fp",
                     "qgemv_select", "qgemv_path_supported",
                     "qgemv_unpack_probe", "qgemv_stream_probe", "qgemv_stream_probe_blocks",
                     "qgemv_version"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)  # torch.cuda.Stream


def _check(status: int, where: str) -> int:
    if status < 0:
        raise QgemvError(status, where)
    return status


def _path(path: Union[int, str]) -> int:
    return _PATHS[path] if isinstance(path, str) else int(path)


# ---------------------------------------------------------------- C entry points

def qgemv_small(codes, scales, biases, x, y, M: int, N: int, K: int, bits: int, group_size: int,
                stream=None) -> int:
    return _check(lib().qgemv_small(_ptr(codes), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y),
                                    M, N, K, bits, group_size, _stream(stream)), "qgemv_small")


def qgemv_run_path(path, codes, scales, biases, x, y, M: int, N: int, K: int, bits: int,
                   group_size: int, stream=None) -> int:
    return _check(lib().qgemv_run_path(_path(path), _ptr(codes), _ptr(scales), _ptr(biases),
                                       _ptr(x), _ptr(y), M, N, K, bits, group_size,
                                       _stream(stream)), "qgemv_run_path")


def qgemv_small_add(codes, scales, biases, x, residual, y, M: int, N: int, K: int, bits: int,
                    group_size: int, stream=None) -> int:
    return _check(lib().qgemv_small_add(_ptr(codes), _ptr(scales), _ptr(biases), _ptr(x),
                                        _ptr(residual), _ptr(y), M, N, K, bits, group_size,
                                        _stream(stream)), "qgemv_small_add")


def qgemv_run_path_add(path, codes, scales, biases, x, residual, y, M: int, N: int, K: int,
                       bits: int, group_size: int, stream=None) -> int:
    return _check(lib().qgemv_run_path_add(_path(path), _ptr(codes), _ptr(scales), _ptr(biases),
                                           _ptr(x), _ptr(residual), _ptr(y), M, N, K, bits,
                                           group_size, _stream(stream)), "qgemv_run_path_add")


def _fmt(fmt) -> int:
    return _FMTS[fmt] if isinstance(fmt, str) else int(fmt)


def qgemv_small_fp(codes, scales, x, residual, y, M: int, N: int, K: int, fmt, stream=None) -> int:
    return _check(lib().qgemv_small_fp(_ptr(codes), _ptr(scales), _ptr(x), _ptr(residual), _ptr(y),
                                       M, N, K, _fmt(fmt), _stream(stream)), "qgemv_small_fp")


def qgemv_run_path_fp(path, codes, scales, x, residual, y, M: int, N: int, K: int, fmt,
                      stream=None) -> int:
    return _check(lib().qgemv_run_path_fp(_path(path), _ptr(codes), _ptr(scales), _ptr(x),
                                          _ptr(residual), _ptr(y), M, N, K, _fmt(fmt),
                                          _stream(stream)), "qgemv_run_path_fp")


def qgemv_select_fp(M: int, N: int, K: int, fmt) -> int:
    return _check(lib().qgemv_select_fp(M, N, K, _fmt(fmt)), "qgemv_select_fp")


def qgemv_path_supported_fp(path, M: int, N: int, K: int, fmt) -> bool:
    return bool(_check(lib().qgemv_path_supported_fp(_path(path), M, N, K, _fmt(fmt)),
                       "qgemv_path_supported_fp"))


def qgemv_unpack_probe_fp(path, codes, out, N: int, K: int, fmt, stream=None) -> int:
    return _check(lib().qgemv_unpack_probe_fp(_path(path), _ptr(codes), _ptr(out), N, K, _fmt(fmt),
                                              _stream(stream)), "qgemv_unpack_probe_fp")


def qgemv_gather(codes, scales, biases, x, x_idx, e_idx, y, P: int, X: int, E: int, N: int, K: int,
                 bits: int, group_size: int, stream=None) -> int:
    return _check(lib().qgemv_gather(_ptr(codes), _ptr(scales), _ptr(biases), _ptr(x), _ptr(x_idx),
                                     _ptr(e_idx), _ptr(y), P, X, E, N, K, bits, group_size,
                                     _stream(stream)), "qgemv_gather")


def qgemv_select(M: int, N: int, K: int, bits: int, group_size: int) -> int:
    return _check(lib().qgemv_select(M, N, K, bits, group_size), "qgemv_select")


def qgemv_path_supported(path, M: int, N: int, K: int, bits: int, group_size: int) -> bool:
    return bool(_check(lib().qgemv_path_supported(_path(path), M, N, K, bits, group_size),
                       "qgemv_path_supported"))


def qgemv_unpack_probe(path, codes, q_out, N: int, K: int, bits: int, group_size: int,
                       stream=None) -> int:
    return _check(lib().qgemv_unpack_probe(_path(path), _ptr(codes), _ptr(q_out), N, K, bits,
                                           group_size, _stream(stream)), "qgemv_unpack_probe")


def qgemv_stream_probe(buf, nbytes: int, out, loads_per_thread: int = 4, layout: int = 0,
                       stream=None) -> int:
    return _check(lib().qgemv_stream_probe(_ptr(buf), nbytes, _ptr(out), loads_per_thread, layout,
                                           _stream(stream)), "qgemv_stream_probe")


def qgemv_stream_probe_blocks(nbytes: int) -> int:
    return lib().qgemv_stream_probe_blocks(nbytes)


def qgemv_strerror(status: int) -> str:
    return lib().qgemv_strerror(status).decode()


def qgemv_version() -> int:
    return lib().qgemv_version()


# ---------------------------------------------------------------- torch convenience

def small(codes, scales, biases, x, bits: int, group_size: int, out=None, path="auto",
          stream=None, residual=None):
    """y = x . dequant(W)^T (+ residual) on torch device tensors.

    codes uint8 [N, K*bits/8]; scales/biases float16 (or int16) [N, K/gs];
    x bfloat16 (or int16) [M, K]; returns (or fills) y float32 [M, N].
    residual: optional float32 [M, N] added in the kernels' store (may be `out`).
    """
    import torch

    if codes.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes must be a 2-D uint8 tensor")
    N = codes.shape[0]
    K = codes.shape[1] * 8 // bits
    M = x.shape[0]
    for name, t, dts in (("scales", scales, (torch.float16, torch.int16)),
                         ("biases", biases, (torch.float16, torch.int16)),
                         ("x", x, (torch.bfloat16, torch.int16))):
        if t.dtype not in dts:
            raise ValueError(f"{name} has dtype {t.dtype}")
        if not t.is_contiguous() or t.device != codes.device:
            raise ValueError(f"{name} must be contiguous on {codes.device}")
    if x.shape[1] != K or scales.shape != (N, K // group_size) or biases.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, N] tensor")
    if residual is None:
        qgemv_run_path(path, codes, scales, biases, x, out, M, N, K, bits, group_size, stream)
        return out
    if (residual.dtype != torch.float32 or tuple(residual.shape) != (M, N)
            or not residual.is_contiguous() or residual.device != codes.device):
        raise ValueError("residual must be a contiguous float32 [M, N] tensor on the same device")
    qgemv_run_path_add(path, codes, scales, biases, x, residual, out, M, N, K, bits, group_size,
                       stream)
    return out
