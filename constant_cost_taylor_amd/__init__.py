"""Python binding of the MI355X SATA library (libsata.so, C ABI in include/sata.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.  If the
library is not built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsata.so")

SATA_OK = 0
SATA_ERR_INVALID_ARG = -1
SATA_ERR_UNSUPPORTED = -2
SATA_ERR_WORKSPACE = -3
SATA_ERR_HIP = -4
SATA_ERR_OOM = -5
SATA_ERR_SCRATCH = -6
SATA_F32 = 0
SATA_BF16 = 1

_lib = None


class SataError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def _declare(lib):
    c_int, c_i64, c_sz, c_dbl, c_vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double, ctypes.c_void_p
    P = ctypes.POINTER
    lib.sata_build_basis.argtypes = [c_int, c_int, c_dbl, P(c_vp)]
    lib.sata_build_basis.restype = c_int
    lib.sata_build_basis_host.argtypes = [c_int, c_int, c_dbl, P(c_vp)]
    lib.sata_build_basis_host.restype = c_int
    lib.sata_free_basis.argtypes = [c_vp]
    lib.sata_free_basis.restype = None
    lib.sata_basis_info.argtypes = [c_vp, P(c_int), P(c_int), P(c_dbl), P(c_i64)]
    lib.sata_basis_info.restype = c_int
    lib.sata_basis_rows.argtypes = [c_vp, c_int, P(c_i64)]
    lib.sata_basis_rows.restype = c_int
    lib.sata_basis_copy_tables.argtypes = [c_vp, c_int, c_vp, c_vp]
    lib.sata_basis_copy_tables.restype = c_int
    lib.sata_basis_download_rows.argtypes = [c_vp, c_vp, c_vp]
    lib.sata_basis_download_rows.restype = c_int
    lib.sata_state_floats.argtypes = [c_vp, c_int]
    lib.sata_state_floats.restype = c_i64
    lib.sata_state_stride.argtypes = [c_vp, c_int]
    lib.sata_state_stride.restype = c_i64
    lib.sata_prefill_workspace.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, P(c_sz)]
    lib.sata_prefill_workspace.restype = c_int
    lib.sata_prefill.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 c_vp, c_sz, c_vp]
    lib.sata_prefill.restype = c_int
    lib.sata_prefill_strided.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_i64, c_vp, c_sz, c_vp]
    lib.sata_prefill_strided.restype = c_int
    lib.sata_prefill_varlen.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_i64, c_vp, c_sz, c_vp]
    lib.sata_prefill_varlen.restype = c_int
    lib.sata_decode_workspace.argtypes = [c_vp, c_int, c_int, c_int, P(c_sz)]
    lib.sata_decode_workspace.restype = c_int
    lib.sata_decode_step.argtypes = [c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_sz, c_vp]
    lib.sata_decode_step.restype = c_int
    lib.sata_decode_step_strided.argtypes = [c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                             c_vp, c_sz, c_vp]
    lib.sata_decode_step_strided.restype = c_int
    lib.sata_decode_step_noalloc.argtypes = [c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                             c_vp]
    lib.sata_decode_step_noalloc.restype = c_int
    lib.sata_decode_noalloc_max_bytes.argtypes = []
    lib.sata_decode_noalloc_max_bytes.restype = c_sz
    lib.sata_mixed_state_bytes.argtypes = [c_vp, c_int]
    lib.sata_mixed_state_bytes.restype = c_i64
    lib.sata_state_to_mixed.argtypes = [c_vp, c_int, c_int, c_vp, c_i64, c_vp, c_vp]
    lib.sata_state_to_mixed.restype = c_int
    lib.sata_state_from_mixed.argtypes = [c_vp, c_int, c_int, c_vp, c_vp, c_i64, c_vp]
    lib.sata_state_from_mixed.restype = c_int
    lib.sata_decode_mixed_workspace.argtypes = [c_vp, c_int, c_int, c_int, P(c_sz)]
    lib.sata_decode_mixed_workspace.restype = c_int
    lib.sata_decode_step_mixed.argtypes = [c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                           c_vp]
    lib.sata_decode_step_mixed.restype = c_int
    lib.sata_softmax_attention.argtypes = [c_int, c_int, c_int, c_int, c_int, c_dbl, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.sata_softmax_attention.restype = c_int
    lib.sata_status_string.argtypes = [c_int]
    lib.sata_status_string.restype = ctypes.c_char_p


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m constant_cost_taylor_amd.build`"
                               " (the SATA path has no fallback)")
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def status_string(status: int) -> str:
    return lib().sata_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != SATA_OK:
        raise SataError(status, what)


class Basis:
    """Handle of the minimal-basis tables for (d_k, P, c) on the current device."""

    def __init__(self, d_k: int, P: int, c: float = 1.0, host_only: bool = False):
        h = ctypes.c_void_p()
        fn = lib().sata_build_basis_host if host_only else lib().sata_build_basis
        _check(fn(int(d_k), int(P), float(c), ctypes.byref(h)), "sata_build_basis")
        self._h = h
        self.d_k = int(d_k)
        self.P = int(P)
        self.c = float(c)
        D = ctypes.c_int64()
        _check(lib().sata_basis_info(h, None, None, None, ctypes.byref(D)), "sata_basis_info")
        self.total_rows = int(D.value)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.sata_free_basis(h)
            self._h = None

    def rows(self, p: int) -> int:
        r = ctypes.c_int64()
        _check(lib().sata_basis_rows(self._h, int(p), ctypes.byref(r)), "sata_basis_rows")
        return int(r.value)

    def tables(self, p: int) -> Tuple[np.ndarray, np.ndarray]:
        n = self.rows(p)
        idx = np.zeros((n, p), dtype=np.int32)
        mult = np.zeros(n, dtype=np.uint32)
        _check(lib().sata_basis_copy_tables(self._h, int(p), idx.ctypes.data if p > 0 else None,
                                            mult.ctypes.data), "sata_basis_copy_tables")
        return idx, mult

    def device_rows(self) -> Tuple[np.ndarray, np.ndarray]:
        packed = np.zeros(self.total_rows, dtype=np.uint32)
        weight = np.zeros(self.total_rows, dtype=np.float32)
        _check(lib().sata_basis_download_rows(self._h, packed.ctypes.data, weight.ctypes.data),
               "sata_basis_download_rows")
        return packed, weight

    def state_floats(self, d_v: Optional[int] = None) -> int:
        return int(lib().sata_state_floats(self._h, int(self.d_k if d_v is None else d_v)))

    def state_stride(self, d_v: Optional[int] = None) -> int:
        return int(lib().sata_state_stride(self._h, int(self.d_k if d_v is None else d_v)))


def build_basis(d_k: int, P: int, c: float = 1.0, host_only: bool = False) -> Basis:
    return Basis(d_k, P, c, host_only)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SATA_F32
    if t.dtype == torch.bfloat16:
        return SATA_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _stream_ptr(device) -> int:
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def new_state(basis: Basis, count: int, device="cuda", packed: bool = False):
    """Zero states (empty prefix) for `count` heads: [count, state_stride] float32
    (rows 256-byte aligned, the layout the decode step streams fastest), or
    [count, state_floats] with packed=True (heads back to back)."""
    import torch
    width = basis.state_floats() if packed else basis.state_stride()
    return torch.zeros((count, width), dtype=torch.float32, device=device)


def _state_stride(basis: Basis, state, count: int, d_v: int, device) -> int:
    """Head stride of a [count, stride] state tensor (stride >= state_floats)."""
    import torch
    if state.dtype != torch.float32 or not state.is_contiguous() or state.device != device:
        raise ValueError(f"state must be a contiguous float32 tensor on {device}")
    if state.dim() != 2 or state.shape[0] != count:
        raise ValueError(f"state must be [{count}, stride] (one row per head), got {tuple(state.shape)}")
    if state.shape[1] < basis.state_floats(d_v):
        raise ValueError(f"state rows hold {state.shape[1]} floats, a head needs {basis.state_floats(d_v)}")
    return int(state.shape[1])


def prefill_workspace_bytes(basis: Basis, B: int, H: int, n: int, d_v: int, dtype_code: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().sata_prefill_workspace(basis.handle, B, H, n, d_v, dtype_code, ctypes.byref(b)),
           "sata_prefill_workspace")
    return int(b.value)


def decode_workspace_bytes(basis: Basis, S: int, d_v: int, dtype_code: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().sata_decode_workspace(basis.handle, S, d_v, dtype_code, ctypes.byref(b)),
           "sata_decode_workspace")
    return int(b.value)


def workspace(nbytes: int, device="cuda"):
    """A 256-byte aligned device buffer of nbytes (torch's allocator aligns to 512)."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _check_inputs(basis: Basis, q, k, v):
    """q, k, v: one dtype, contiguous, on one GPU, q's last dim = the basis d_k
    (the C calls take d_v only and read d_k coordinates per row)."""
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if q.shape[-1] != basis.d_k:
        raise ValueError(f"q, k have last dimension {q.shape[-1]}, the basis was built for d_k = {basis.d_k}")
    if q.device.type != "cuda" or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU")


def _check_buffer(name: str, t, dtype, numel: int, device):
    """A caller-provided output buffer: dtype, contiguous, on the inputs' GPU and
    at least numel elements (the C calls see only its address)."""
    if t.dtype != dtype or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on {device}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call writes {numel}")


def prefill(basis: Basis, q, k, v, state=None, out=None, ws=None, lengths=None):
    """Causal prefill. q, k: [B, H, n, d_k], v: [B, H, n, d_v] (float32 or bfloat16,
    contiguous, on the GPU). state: [B*H, stride] float32 with stride >= state_floats
    (new_state; zeros = empty prefix), read and written. lengths: optional int32
    tensor of B*H per-head token counts on the GPU (head h takes its first
    lengths[h] tokens; its output rows past that are zeros). ws: optional
    workspace, by default prefill_workspace_bytes; a larger one selects the
    least-time plan, a smaller one (down to prefill_workspace_bytes(basis, 1,
    1, min(n, 512), ...)) runs the heads in more groups or the tokens in more
    windows. Returns
    (out [B, H, n, d_v] float32, state)."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B, H, n, d_k] and v [B, H, n, d_v]")
    _check_inputs(basis, q, k, v)
    B, H, n, _ = q.shape
    d_v = v.shape[3]
    code = _dtype_code(q)
    if state is None:
        state = new_state(basis, B * H, q.device)
    stride = _state_stride(basis, state, B * H, d_v, q.device)
    if out is None:
        out = torch.empty((B, H, n, d_v), dtype=torch.float32, device=q.device)
    _check_buffer("out", out, torch.float32, B * H * n * d_v, q.device)
    need = prefill_workspace_bytes(basis, B, H, n, d_v, code)
    if ws is None:
        ws = workspace(need, q.device)
    if ws.device != q.device:
        raise ValueError(f"ws must be on {q.device}")
    if lengths is not None:
        if lengths.dtype != torch.int32 or not lengths.is_contiguous() or lengths.device != q.device \
                or lengths.numel() != B * H:
            raise ValueError(f"lengths must be a contiguous int32 tensor of {B * H} elements on {q.device}")
        st = lib().sata_prefill_varlen(basis.handle, B, H, n, d_v, code, q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), lengths.data_ptr(), out.data_ptr(), state.data_ptr(), stride,
                                       ws.data_ptr(), ws.numel() * ws.element_size(), _stream_ptr(q.device))
        _check(st, "sata_prefill_varlen")
        return out, state
    st = lib().sata_prefill_strided(basis.handle, B, H, n, d_v, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    out.data_ptr(), state.data_ptr(), stride, ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream_ptr(q.device))
    _check(st, "sata_prefill_strided")
    return out, state


def decode_step(basis: Basis, q, k, v, state, out=None, ws=None):
    """One decode step for S states: q, k [S, d_k], v [S, d_v]; state [S, stride] in/out.
    Returns out [S, d_v] float32."""
    import torch
    if q.dim() != 2 or k.shape != q.shape or v.dim() != 2 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [S, d_k] and v [S, d_v]")
    _check_inputs(basis, q, k, v)
    S = q.shape[0]
    d_v = v.shape[1]
    code = _dtype_code(q)
    stride = _state_stride(basis, state, S, d_v, q.device)
    if out is None:
        out = torch.empty((S, d_v), dtype=torch.float32, device=q.device)
    _check_buffer("out", out, torch.float32, S * d_v, q.device)
    if ws is None:
        ws = workspace(decode_workspace_bytes(basis, S, d_v, code), q.device)
    if ws.device != q.device:
        raise ValueError(f"ws must be on {q.device}")
    st = lib().sata_decode_step_strided(basis.handle, S, d_v, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        out.data_ptr(), state.data_ptr(), stride, ws.data_ptr(),
                                        ws.numel() * ws.element_size(), _stream_ptr(q.device))
    _check(st, "sata_decode_step_strided")
    return out


def decode_step_noalloc(basis: Basis, q, k, v, state, out):
    """decode_step through sata_decode_step_noalloc: the library allocates
    nothing (its partial records live in a static device array shared by every
    call on the device, so calls must not overlap in time).  out [S, d_v]
    float32 is caller-provided.  Returns out."""
    import torch
    if q.dim() != 2 or k.shape != q.shape or v.dim() != 2 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [S, d_k] and v [S, d_v]")
    _check_inputs(basis, q, k, v)
    S = q.shape[0]
    d_v = v.shape[1]
    stride = _state_stride(basis, state, S, d_v, q.device)
    _check_buffer("out", out, torch.float32, S * d_v, q.device)
    st = lib().sata_decode_step_noalloc(basis.handle, S, d_v, _dtype_code(q), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), out.data_ptr(), state.data_ptr(), stride,
                                        _stream_ptr(q.device))
    _check(st, "sata_decode_step_noalloc")
    return out


# ---- mixed-precision decode state (orders >= 2 of S in float16) ---------------

def mixed_state_bytes(basis: Basis, d_v: Optional[int] = None) -> int:
    return int(lib().sata_mixed_state_bytes(basis.handle, int(basis.d_k if d_v is None else d_v)))


def new_mixed_state(basis: Basis, count: int, device="cuda"):
    """Uninitialised mixed states: [count, mixed_state_bytes] uint8 (fill with to_mixed)."""
    import torch
    return torch.empty((count, mixed_state_bytes(basis)), dtype=torch.uint8, device=device)


def _check_mixed(basis: Basis, mixed, count: int, device):
    import torch
    if mixed.dtype != torch.uint8 or not mixed.is_contiguous() or mixed.device != device:
        raise ValueError(f"mixed state must be a contiguous uint8 tensor on {device}")
    if mixed.dim() != 2 or mixed.shape[0] != count or mixed.shape[1] != mixed_state_bytes(basis):
        raise ValueError(f"mixed state must be [{count}, {mixed_state_bytes(basis)}]")


def to_mixed(basis: Basis, state, mixed=None):
    """float32 states [S, stride] -> mixed states [S, mixed_state_bytes]."""
    S = state.shape[0]
    stride = _state_stride(basis, state, S, basis.d_k, state.device)
    if mixed is None:
        mixed = new_mixed_state(basis, S, state.device)
    _check_mixed(basis, mixed, S, state.device)
    _check(lib().sata_state_to_mixed(basis.handle, S, basis.d_k, state.data_ptr(), stride, mixed.data_ptr(),
                                     _stream_ptr(state.device)), "sata_state_to_mixed")
    return mixed


def from_mixed(basis: Basis, mixed, state=None):
    """mixed states [S, mixed_state_bytes] -> float32 states [S, stride]."""
    S = mixed.shape[0]
    if state is None:
        state = new_state(basis, S, mixed.device)
    stride = _state_stride(basis, state, S, basis.d_k, mixed.device)
    _check_mixed(basis, mixed, S, mixed.device)
    _check(lib().sata_state_from_mixed(basis.handle, S, basis.d_k, mixed.data_ptr(), state.data_ptr(), stride,
                                       _stream_ptr(mixed.device)), "sata_state_from_mixed")
    return state


def decode_mixed_workspace_bytes(basis: Basis, S: int, d_v: int, dtype_code: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().sata_decode_mixed_workspace(basis.handle, S, d_v, dtype_code, ctypes.byref(b)),
           "sata_decode_mixed_workspace")
    return int(b.value)


def decode_step_mixed(basis: Basis, q, k, v, mixed, out=None, ws=None):
    """decode_step on mixed states [S, mixed_state_bytes] (in/out). Returns out [S, d_v]."""
    import torch
    if q.dim() != 2 or k.shape != q.shape or v.dim() != 2 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [S, d_k] and v [S, d_v]")
    _check_inputs(basis, q, k, v)
    S = q.shape[0]
    d_v = v.shape[1]
    code = _dtype_code(q)
    _check_mixed(basis, mixed, S, q.device)
    if out is None:
        out = torch.empty((S, d_v), dtype=torch.float32, device=q.device)
    _check_buffer("out", out, torch.float32, S * d_v, q.device)
    if ws is None:
        ws = workspace(decode_mixed_workspace_bytes(basis, S, d_v, code), q.device)
    st = lib().sata_decode_step_mixed(basis.handle, S, d_v, code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      out.data_ptr(), mixed.data_ptr(), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream_ptr(q.device))
    _check(st, "sata_decode_step_mixed")
    return out


# ---- exact causal softmax attention (the baseline SATA is measured against) ----

def softmax_attention(q, k, v, c: float = 1.0, out=None):
    """Exact causal softmax attention of [B, H, n, d] q, k, v (float32 or
    bfloat16, one GPU): returns out [B, H, n, d] float32."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, n, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if q.device.type != "cuda" or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU")
    B, H, n, d = q.shape
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    _check_buffer("out", out, torch.float32, B * H * n * d, q.device)
    _check(lib().sata_softmax_attention(B, H, n, d, _dtype_code(q), float(c), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), out.data_ptr(), _stream_ptr(q.device)),
           "sata_softmax_attention")
    return out
