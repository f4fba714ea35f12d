"""ctypes binding of libsata_ceilings.so (include/sata_ceilings.h): the ceiling
kernels that measure the machine's HBM streams and matrix-core rates. Argument
marshalling only."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsata_ceilings.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m constant_cost_taylor_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, sz, i, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
        L.sata_ceil_copy.argtypes = [p, p, sz, p]
        L.sata_ceil_rmw.argtypes = [p, sz, p]
        L.sata_ceil_read_partials.argtypes = [sz]
        L.sata_ceil_read_partials.restype = i64
        L.sata_ceil_read.argtypes = [p, sz, p, p]
        L.sata_ceil_mfma.argtypes = [i, i, i, p, p]
        L.sata_ceil_mfma_flops.argtypes = [i, i, i]
        L.sata_ceil_mfma_flops.restype = ctypes.c_double
        for f in (L.sata_ceil_copy, L.sata_ceil_rmw, L.sata_ceil_read, L.sata_ceil_mfma):
            f.restype = i
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def copy(src, dst, stream: int):
    _check(lib().sata_ceil_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), stream),
           "sata_ceil_copy")


def rmw(buf, stream: int):
    _check(lib().sata_ceil_rmw(buf.data_ptr(), buf.numel() * buf.element_size(), stream), "sata_ceil_rmw")


def read_partials(nbytes: int) -> int:
    return int(lib().sata_ceil_read_partials(nbytes))


def read(src, partial, stream: int):
    nbytes = src.numel() * src.element_size()
    if partial.numel() < read_partials(nbytes):
        raise ValueError("partial buffer too small")
    _check(lib().sata_ceil_read(src.data_ptr(), nbytes, partial.data_ptr(), stream), "sata_ceil_read")


def mfma(dtype_code: int, blocks: int, iters: int, out, stream: int):
    if out.numel() < blocks * 512:
        raise ValueError("out buffer too small")
    _check(lib().sata_ceil_mfma(dtype_code, blocks, iters, out.data_ptr(), stream), "sata_ceil_mfma")


def mfma_flops(dtype_code: int, blocks: int, iters: int) -> float:
    return float(lib().sata_ceil_mfma_flops(dtype_code, blocks, iters))
