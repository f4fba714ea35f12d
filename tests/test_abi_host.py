"""CPU checks of the C ABI: the library loads, exports every declared symbol,
builds basis tables on the host that equal the oracle's enumeration bit for
bit, and rejects invalid arguments before touching a GPU."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import constant_cost_taylor_amd as SA
from oracle import sata_oracle as O

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "sata.h")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sata_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = SA.lib()
    names = _declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name


def test_ceilings_library_exports_every_declared_symbol():
    from constant_cost_taylor_amd import ceilings as CL
    lib = CL.lib()
    names = _declared_functions(os.path.join(INCLUDE, "sata_ceilings.h"))
    assert len(names) == 6
    for name in names:
        assert hasattr(lib, name), name
    # host-side checks: argument errors launch nothing; the FLOP count formula
    assert lib.sata_ceil_copy(None, None, 1024, None) == -1
    assert lib.sata_ceil_rmw(16, 24, None) == -1          # not a multiple of 16 bytes
    assert lib.sata_ceil_mfma(2, 1, 1, 16, None) == -1    # no such dtype
    assert CL.read_partials(1 << 20) == (1 << 20) // (16 * 1024)
    assert CL.mfma_flops(1, 3, 5) == 2 * 16 * 16 * 32 * 8 * 8 * 3 * 5
    assert CL.mfma_flops(0, 2, 7) == 2 * 16 * 16 * 4 * 8 * 8 * 2 * 7


@pytest.mark.parametrize("d,P", [(8, 1), (8, 3), (16, 4), (32, 4), (64, 4), (64, 2), (16, 5), (64, 5)])
def test_host_tables_bit_exact(d, P):
    b = SA.build_basis(d, P, 1.0, host_only=True)
    ref = O.enumerate_basis(d, P)
    assert b.total_rows == sum(r[0].shape[0] for r in ref) == math.comb(d + P - 1, P - 1)
    for p, (idx, mult, _) in enumerate(ref):
        hi, hm = b.tables(p)
        assert hi.dtype == np.int32 and hm.dtype == np.uint32
        np.testing.assert_array_equal(hi, idx)
        np.testing.assert_array_equal(hm, mult)


@pytest.mark.parametrize("d,P", [(8, 3), (16, 4), (64, 4), (32, 4), (8, 5), (64, 5)])
def test_state_size_matches_closed_form(d, P):
    b = SA.build_basis(d, P, 1.0, host_only=True)
    assert b.state_floats() == O.cost_model(d, d, P)[0]
    assert b.state_stride() % 64 == 0 and 0 <= b.state_stride() - b.state_floats() < 64


def test_invalid_builds():
    h = ctypes.c_void_p()
    L = SA.lib()
    assert L.sata_build_basis_host(7, 3, 1.0, ctypes.byref(h)) == SA.SATA_ERR_UNSUPPORTED
    assert L.sata_build_basis_host(16, 6, 1.0, ctypes.byref(h)) == SA.SATA_ERR_UNSUPPORTED
    assert L.sata_build_basis_host(16, 0, 1.0, ctypes.byref(h)) == SA.SATA_ERR_UNSUPPORTED
    assert L.sata_build_basis_host(16, 3, 0.0, ctypes.byref(h)) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_build_basis_host(16, 3, float("nan"), ctypes.byref(h)) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_build_basis_host(16, 3, 1.0, None) == SA.SATA_ERR_INVALID_ARG


def test_host_only_handle_rejects_compute():
    """Validation runs before any HIP call: a host-only handle, a null
    pointer or a wrong size is refused on a machine without a GPU."""
    b = SA.build_basis(16, 4, 1.0, host_only=True)
    L = SA.lib()
    buf = (ctypes.c_float * 8192)()
    p = ctypes.c_void_p((ctypes.addressof(buf) + 255) // 256 * 256)   # 256-byte aligned
    # n = 0 and S = 0 are valid no-ops
    assert L.sata_prefill(b.handle, 1, 1, 0, 16, SA.SATA_F32, None, None, None, None, None, None, 0, None) == SA.SATA_OK
    assert L.sata_decode_step(b.handle, 0, 16, SA.SATA_F32, None, None, None, None, None, None, 0, None) == SA.SATA_OK
    assert L.sata_prefill(b.handle, 1, 1, 4, 16, SA.SATA_F32, None, p, p, p, p, p, 1 << 20, None) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_prefill(b.handle, 1, 1, 4, 8, SA.SATA_F32, p, p, p, p, p, p, 1 << 20, None) == SA.SATA_ERR_UNSUPPORTED
    assert L.sata_prefill(b.handle, 1, 1, 4, 16, 7, p, p, p, p, p, p, 1 << 20, None) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_prefill(b.handle, 1, 1, -1, 16, SA.SATA_F32, p, p, p, p, p, p, 1 << 20, None) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_prefill(b.handle, 1, 1, 4, 16, SA.SATA_F32, p, p, p, p, p, p, 8, None) == SA.SATA_ERR_WORKSPACE
    assert L.sata_decode_step(b.handle, 2, 16, SA.SATA_F32, p, p, p, p, p, p, 0, None) == SA.SATA_ERR_WORKSPACE
    # the strided calls refuse a head stride below the state size
    F = b.state_floats()
    assert L.sata_prefill_strided(b.handle, 1, 1, 4, 16, SA.SATA_F32, p, p, p, p, p, F - 1, p, 1 << 20,
                                  None) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_decode_step_strided(b.handle, 2, 16, SA.SATA_F32, p, p, p, p, p, F - 1, p, 1 << 20,
                                      None) == SA.SATA_ERR_INVALID_ARG
    # a host-only handle is refused once everything else checks out
    assert L.sata_decode_step(b.handle, 2, 16, SA.SATA_F32, p, p, p, p, p, p, 1 << 20, None) == SA.SATA_ERR_INVALID_ARG
    assert SA.status_string(SA.SATA_ERR_HIP).startswith("SATA_ERR_HIP")


def test_prefill_workspace_plans(monkeypatch):
    """The fastest plan's workspace is the largest; a cap down to the
    one-head, one-readout-window minimum still yields a plan, below it none."""
    b = SA.build_basis(64, 4, 1.0, host_only=True)
    least = SA.prefill_workspace_bytes(b, 1, 1, 512, 64, SA.SATA_BF16)
    full = SA.prefill_workspace_bytes(b, 8, 32, 4096, 64, SA.SATA_BF16)
    assert least < SA.prefill_workspace_bytes(b, 1, 2, 512, 64, SA.SATA_BF16) < full
    monkeypatch.setenv("SATA_PREFILL_WS_CAP", str(least))
    assert SA.prefill_workspace_bytes(b, 8, 32, 4096, 64, SA.SATA_BF16) == least
    monkeypatch.setenv("SATA_PREFILL_WS_CAP", str(least - 1))
    with pytest.raises(SA.SataError) as e:
        SA.prefill_workspace_bytes(b, 8, 32, 4096, 64, SA.SATA_BF16)
    assert e.value.status == SA.SATA_ERR_WORKSPACE


def test_prefill_segment_workspace(monkeypatch):
    """One bf16 head of 2^20 tokens at d = 32 runs as sequence segments: its
    workspace holds the segment states on top of the segment prefill's; four
    heads fill the chip at d = 64 and 256 heads at d = 32 take no segments,
    nor does float32; SATA_PREFILL_SEGMENTS=0 turns them off."""
    def sizes(d, H, n, code):
        b = SA.build_basis(d, 4, 1.0, host_only=True)
        monkeypatch.delenv("SATA_PREFILL_SEGMENTS", raising=False)
        seg = SA.prefill_workspace_bytes(b, 1, H, n, d, code)
        monkeypatch.setenv("SATA_PREFILL_SEGMENTS", "0")
        plain = SA.prefill_workspace_bytes(b, 1, H, n, d, code)
        monkeypatch.delenv("SATA_PREFILL_SEGMENTS")
        return b, seg, plain
    b, seg, plain = sizes(32, 1, 1 << 20, SA.SATA_BF16)
    assert seg > plain
    assert seg - plain >= 2 * b.state_stride(32) * 4     # at least two segment states
    for d, H, n, code in ((64, 4, 16384, SA.SATA_BF16), (32, 256, 4096, SA.SATA_BF16), (32, 1, 1 << 20, SA.SATA_F32),
                          (32, 1, 1000, SA.SATA_BF16)):
        _, seg, plain = sizes(d, H, n, code)
        assert seg == plain, (d, H, n, code)


def test_workspace_sizes():
    b = SA.build_basis(64, 4, 1.0, host_only=True)
    assert SA.prefill_workspace_bytes(b, 1, 4, 0, 64, SA.SATA_BF16) == 0
    small = SA.prefill_workspace_bytes(b, 1, 4, 100, 64, SA.SATA_BF16)
    big = SA.prefill_workspace_bytes(b, 1, 4, 16384, 64, SA.SATA_BF16)
    assert 0 < small < big
    # decode: per tile of 16 rows (two rows of 64 floats per thread of a
    # 128-thread block) and state, d_v value partials and one den partial.
    # fp32 inputs: fp32 records in two 256-byte aligned regions.  bf16
    # inputs: f16 value records, one scale a record, fp32 value records for
    # the 5 tiles holding rows 0..64 (orders 0 and 1), fp32 den records.
    tiles = math.ceil(47905 / 16)
    lo_t = math.ceil(65 / 16)
    up = lambda x: (x + 255) // 256 * 256
    assert SA.decode_workspace_bytes(b, 256, 64, SA.SATA_F32) == up(256 * tiles * 64 * 4) + up(256 * tiles * 4)
    assert SA.decode_workspace_bytes(b, 256, 64, SA.SATA_BF16) == (up(256 * tiles * 64 * 2) + up(256 * tiles * 4) +
                                                                   up(256 * lo_t * 64 * 4) + up(256 * tiles * 4))
    # three states: the tile records are reduced in 11 groups (256 records or
    # more each), whose fp32 sums take two more regions
    groups = min(-(-256 // 3), tiles // 256)
    assert groups == 11
    assert SA.decode_workspace_bytes(b, 3, 64, SA.SATA_F32) == (up(3 * tiles * 64 * 4) + up(3 * tiles * 4) +
                                                                up(3 * groups * 64 * 4) + up(3 * groups * 4))
    assert SA.decode_workspace_bytes(b, 3, 64, SA.SATA_BF16) == (up(3 * tiles * 64 * 2) + up(3 * tiles * 4) +
                                                                 up(3 * lo_t * 64 * 4) + up(3 * tiles * 4) +
                                                                 up(3 * groups * 64 * 4) + up(3 * groups * 4))


def test_binding_checks_inputs_before_any_call():
    """Input checks of the Python binding run on the host: mismatched shapes,
    dtypes, d_k and device are refused before the C library is called."""
    import torch
    b = SA.build_basis(16, 3, 1.0, host_only=True)
    q = torch.zeros((1, 1, 4, 16))
    with pytest.raises(ValueError):
        SA.prefill(b, q, q, q[:, :, :3])                       # v length differs
    with pytest.raises(TypeError):
        SA.prefill(b, q, q.to(torch.bfloat16), q)              # dtypes differ
    with pytest.raises(ValueError, match="d_k"):
        SA.prefill(b, q[..., :8].contiguous(), q[..., :8].contiguous(), q[..., :8].contiguous())
    with pytest.raises(ValueError, match="GPU"):
        SA.prefill(b, q, q, q)                                 # host tensors
    with pytest.raises(ValueError, match="GPU"):
        SA.decode_step(b, q[0, 0], q[0, 0], q[0, 0], torch.zeros((4, b.state_stride())))


def test_noalloc_decode_size_limit_on_host():
    """The allocation-free decode refuses a call whose partial records exceed
    its static scratch before touching a GPU (a host-only handle answers the
    size check first); within the limit the host-only handle is refused."""
    b = SA.build_basis(64, 4, 1.0, host_only=True)
    L = SA.lib()
    cap = L.sata_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    buf = (ctypes.c_float * 64)()
    p = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    F = b.state_floats()
    S = 1
    while SA.decode_workspace_bytes(b, S, 64, SA.SATA_BF16) <= cap:
        S += 1
    assert S == 82
    assert L.sata_decode_step_noalloc(b.handle, S, 64, SA.SATA_BF16, p, p, p, p, p, F, None) == SA.SATA_ERR_SCRATCH
    assert L.sata_decode_step_noalloc(b.handle, S - 1, 64, SA.SATA_BF16, p, p, p, p, p, F,
                                      None) == SA.SATA_ERR_INVALID_ARG
    assert L.sata_decode_step_noalloc(b.handle, 0, 64, SA.SATA_BF16, None, None, None, None, None, F,
                                      None) == SA.SATA_OK
    assert SA.status_string(SA.SATA_ERR_SCRATCH).startswith("SATA_ERR_SCRATCH")
