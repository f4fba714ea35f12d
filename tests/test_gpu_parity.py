"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Gate (row-normwise, max over rows of ||o_i - r_i||_inf / ||r_i||_inf):
1e-5 for float32 inputs, 3e-3 for bfloat16 inputs with float32 state.
Basis tables: bit-exact.  Every input comes from the seeded generators in
workloads.py; every expected value from oracle/.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import sata_oracle as O

torch = pytest.importorskip("torch")
import constant_cost_taylor_amd as SA  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {W.F32: 1e-5, W.BF16: 3e-3}


def note(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    SA.lib()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == W.BF16 else t
    return t.to("cuda")


def f64(x):
    return np.asarray(x, dtype=np.float64)


def oracle_rows(q, k, v, P, c, rows=None):
    return O.direct_taylor(f64(q), f64(k), f64(v), P, c, rows=rows)


def run_prefill(basis, q, k, v, dtype, state=None):
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out, st = SA.prefill(basis, qd, kd, vd, state=state)
    torch.cuda.synchronize()
    return out, st


# ----------------------------------------------------------------------------
# Tables
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,P,c", [(8, 3, 1.0), (16, 4, 1.0), (32, 4, 0.5), (64, 4, 1.0), (64, 1, 2.0),
                                   (16, 5, 1.0), (64, 5, 0.5)])
def test_device_tables_bit_exact(d, P, c):
    note(f"device tables d={d} P={P} c={c}")
    b = SA.build_basis(d, P, c)
    packed, weight = b.device_rows()
    ref = O.enumerate_basis(d, P, c)
    exp_packed = []
    exp_weight = []
    for p, (idx, mult, scale) in enumerate(ref):
        for r in range(idx.shape[0]):
            key = p << 24   # six bits per index
            for j in range(p):
                key |= int(idx[r, j]) << (6 * j)
            exp_packed.append(key)
        exp_weight.append((mult.astype(np.float64) * scale).astype(np.float32))
    np.testing.assert_array_equal(packed, np.array(exp_packed, dtype=np.uint32))
    np.testing.assert_array_equal(weight, np.concatenate(exp_weight))


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,P,dtype,steps", [(8, 3, W.F32, 80), (16, 4, W.BF16, 40), (32, 4, W.BF16, 24),
                                             (32, 3, W.F32, 24), (64, 4, W.BF16, 12), (64, 4, W.F32, 8),
                                             (8, 5, W.F32, 40), (32, 5, W.BF16, 16), (64, 5, W.F32, 6)])
def test_decode_steps_from_empty_state(d, P, dtype, steps):
    """Token-by-token decode from a zero state reproduces causal attention."""
    note(f"decode from empty d={d} P={P} {dtype} steps={steps}")
    S = 3
    q, k, v = W.make_qkv(1, S, steps, d, d, dtype, 7000 + d)
    b = SA.build_basis(d, P, 1.0)
    state = SA.new_state(b, S)
    got = np.zeros((S, steps, d))
    qd, kd, vd = to_dev(q[0], dtype), to_dev(k[0], dtype), to_dev(v[0], dtype)
    for t in range(steps):
        out = SA.decode_step(b, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), state)
        got[:, t] = out.cpu().numpy()
    for s in range(S):
        ref = oracle_rows(q[0, s], k[0, s], v[0, s], P, 1.0)
        err = O.row_normwise_error(got[s], ref)
        assert err <= TOL[dtype], (s, err)


# ----------------------------------------------------------------------------
# Prefill: small and ragged shapes (several chunks and tiles, ragged tail)
# ----------------------------------------------------------------------------

CASES = [
    # name, B, H, n, d, P, c, dtype
    ("tiny_full", 1, 1, 256, 8, 3, 1.0, W.F32),
    ("d8_P1", 1, 2, 100, 8, 1, 1.0, W.F32),
    ("d8_P2_c2", 2, 1, 77, 8, 2, 2.0, W.F32),
    ("d16_ragged", 1, 3, 1000, 16, 4, 1.0, W.F32),
    ("d16_n1", 1, 2, 1, 16, 4, 1.0, W.F32),
    ("d32_f32", 1, 1, 300, 32, 3, 1.0, W.F32),
    ("d64_f32", 1, 1, 130, 64, 4, 1.0, W.F32),
    ("d16_bf16", 2, 2, 513, 16, 4, 1.0, W.BF16),
    ("d32_bf16", 1, 2, 777, 32, 4, 1.0, W.BF16),
    ("d64_bf16", 1, 2, 333, 64, 4, 1.0, W.BF16),
    # 17 chunks in one call: two readout windows, an unpaired last chunk
    ("d64_bf16_odd_chunks", 1, 1, 1050, 64, 4, 1.0, W.BF16),
    ("d64_bf16_P3", 1, 1, 200, 64, 3, 0.75, W.BF16),
    ("d8_bf16", 1, 1, 97, 8, 4, 1.0, W.BF16),
    # several readout windows at small head dims: the scan's readout carries
    # a large share of each output, which averages many values
    ("d8_bf16_long", 1, 2, 2000, 8, 4, 1.0, W.BF16),
    ("d16_bf16_long", 1, 2, 2000, 16, 5, 1.0, W.BF16),
    # chunk (64) and readout-window (512) boundaries of the bf16 path
    ("d64_bf16_n1", 1, 2, 1, 64, 4, 1.0, W.BF16),
    ("d64_bf16_n63", 1, 1, 63, 64, 4, 1.0, W.BF16),
    ("d64_bf16_n64", 1, 1, 64, 64, 4, 1.0, W.BF16),
    ("d64_bf16_n65", 1, 1, 65, 64, 4, 1.0, W.BF16),
    ("d32_bf16_n511", 1, 1, 511, 32, 4, 1.0, W.BF16),
    ("d32_bf16_n512", 1, 1, 512, 32, 4, 1.0, W.BF16),
    ("d32_bf16_n513", 1, 1, 513, 32, 4, 1.0, W.BF16),
    # orders 0..4
    ("d8_P5", 1, 2, 300, 8, 5, 1.0, W.F32),
    ("d8_P5_bf16", 1, 1, 200, 8, 5, 1.0, W.BF16),
    ("d16_P5_bf16", 1, 2, 600, 16, 5, 1.0, W.BF16),
    ("d32_P5_f32", 1, 1, 200, 32, 5, 1.0, W.F32),
    ("d32_P5_bf16", 1, 1, 530, 32, 5, 0.75, W.BF16),
    ("d64_P5_f32", 1, 1, 100, 64, 5, 1.0, W.F32),
    ("d64_P5_bf16", 1, 2, 300, 64, 5, 1.0, W.BF16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_small(case):
    name, B, H, n, d, P, c, dtype = case
    note(f"prefill {name} B={B} H={H} n={n} d={d} P={P} c={c} {dtype}")
    q, k, v = W.make_qkv(B, H, n, d, d, dtype, 9000 + 17 * d + n)
    b = SA.build_basis(d, P, c)
    out, _ = run_prefill(b, q, k, v, dtype)
    got = out.cpu().numpy()
    for bb in range(B):
        for h in range(H):
            ref = oracle_rows(q[bb, h], k[bb, h], v[bb, h], P, c)
            err = O.row_normwise_error(got[bb, h], ref)
            assert err <= TOL[dtype], (bb, h, err)


def test_prefill_empty_is_noop():
    note("prefill n=0")
    b = SA.build_basis(16, 4, 1.0)
    q = torch.zeros((1, 1, 0, 16), device="cuda")
    out, st = SA.prefill(b, q, q, q)
    assert out.shape == (1, 1, 0, 16) and float(st.abs().sum()) == 0.0


@pytest.mark.parametrize("d,P,dtype,n", [(16, 4, W.F32, 300), (8, 3, W.F32, 70), (64, 4, W.BF16, 96),
                                         (32, 4, W.BF16, 150), (16, 5, W.F32, 200), (32, 5, W.BF16, 120)])
def test_prefill_state_matches_direct_state(d, P, dtype, n):
    """The state written back equals sum_j phi(k_j) v_j and sum_j phi(k_j)
    (unweighted monomials, canonical row order)."""
    note(f"prefill state d={d} P={P} {dtype} n={n}")
    q, k, v = W.make_qkv(1, 2, n, d, d, dtype, 11000 + d)
    b = SA.build_basis(d, P, 1.0)
    _, st = run_prefill(b, q, k, v, dtype)
    st = st.cpu().numpy()
    basis = O.enumerate_basis(d, P)
    D = b.total_rows
    for h in range(2):
        S, z = O.direct_state(f64(k[0, h]), f64(v[0, h]), basis)
        gS = st[h, :D * d].reshape(D, d)
        gz = st[h, D * d:D * (d + 1)]
        tol = TOL[dtype]
        # normwise per row block: max |err| / max |ref| over each order
        off = 0
        for p in range(P):
            rows = math.comb(d + p - 1, p)
            sl = slice(off, off + rows)
            assert np.max(np.abs(gS[sl] - S[sl])) <= tol * np.max(np.abs(S[sl])) + 1e-30, (h, p)
            assert np.max(np.abs(gz[sl] - z[sl])) <= tol * np.max(np.abs(z[sl])) + 1e-30, (h, p)
            off += rows


@pytest.mark.parametrize("d,P,dtype,n1,n2", [(16, 4, W.F32, 200, 333), (64, 4, W.BF16, 100, 161),
                                             (8, 3, W.F32, 33, 64), (64, 5, W.BF16, 100, 161),
                                             (32, 4, W.BF16, 512, 600), (32, 4, W.BF16, 64, 1)])
def test_prefill_continuation(d, P, dtype, n1, n2):
    """prefill(a) then prefill(b | state) gives the rows of prefill(a + b)."""
    note(f"continuation d={d} P={P} {dtype} {n1}+{n2}")
    q, k, v = W.make_qkv(1, 2, n1 + n2, d, d, dtype, 12000 + d)
    b = SA.build_basis(d, P, 1.0)
    out1, st = run_prefill(b, q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], dtype)
    out2, st = run_prefill(b, q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], dtype, state=st)
    got = np.concatenate([out1.cpu().numpy(), out2.cpu().numpy()], axis=2)
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[dtype]


@pytest.mark.parametrize("d,P,dtype", [(16, 4, W.F32), (32, 4, W.BF16), (64, 4, W.BF16), (32, 5, W.BF16),
                                       (64, 5, W.F32)])
def test_prefill_then_decode(d, P, dtype):
    note(f"prefill then decode d={d} P={P} {dtype}")
    n, steps, H = 257, 9, 3
    q, k, v = W.make_qkv(1, H, n + steps, d, d, dtype, 13000 + d)
    b = SA.build_basis(d, P, 1.0)
    _, st = run_prefill(b, q[:, :, :n], k[:, :, :n], v[:, :, :n], dtype)
    qd, kd, vd = to_dev(q[0], dtype), to_dev(k[0], dtype), to_dev(v[0], dtype)
    got = np.zeros((H, steps, d))
    for s in range(steps):
        t = n + s
        got[:, s] = SA.decode_step(b, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                                   st).cpu().numpy()
    for h in range(H):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0, rows=np.arange(n, n + steps))
        assert O.row_normwise_error(got[h], ref) <= TOL[dtype]


@pytest.mark.parametrize("d,P", [(64, 4), (16, 4), (32, 5), (8, 3)])
def test_decode_16bit_records_extreme_value_scales(d, P):
    """bf16 decode writes its per-tile readout records as f16 with a
    power-of-two scale per tile (fp32 for the tiles of the order-0/1 rows):
    values scaled by 2^-90 and 2^60 (exact in bf16) keep the relative error
    of unit-scale values, and a state whose values are all zero (every
    record zero) reads out exact zeros."""
    note(f"decode 16-bit records, value scales 2^-90 / 2^60 / 0, d={d} P={P}")
    n, steps, H = 300, 6, 4
    q, k, v = W.make_qkv(1, H, n + steps, d, d, W.BF16, 31000 + d + P)
    scale = np.array([2.0 ** -90, 2.0 ** 60, 0.0, 1.0])
    v = (v.astype(np.float64) * scale[None, :, None, None]).astype(np.float32)
    b = SA.build_basis(d, P, 1.0)
    _, st = run_prefill(b, q[:, :, :n], k[:, :, :n], v[:, :, :n], W.BF16)
    qd, kd, vd = to_dev(q[0], W.BF16), to_dev(k[0], W.BF16), to_dev(v[0], W.BF16)
    got = np.zeros((H, steps, d))
    for s in range(steps):
        t = n + s
        got[:, s] = SA.decode_step(b, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                                   st).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(got[2] == 0.0)
    for h in (0, 1, 3):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0, rows=np.arange(n, n + steps))
        assert O.row_normwise_error(got[h], ref) <= TOL[W.BF16], h


@pytest.mark.parametrize("d,P,dtype", [(64, 4, W.BF16), (16, 4, W.F32), (32, 5, W.BF16)])
def test_ragged_batched_decode(d, P, dtype):
    """States at different positions (prefilled to 0, 1, 63, 200 and 517
    tokens by separate calls) decode together in one batched call per step:
    the state carries no position, so each row must equal causal attention
    over its own sequence."""
    lens = [0, 1, 63, 200, 517]
    steps = 5
    note(f"ragged batched decode d={d} P={P} {dtype} lens={lens}")
    S = len(lens)
    b = SA.build_basis(d, P, 1.0)
    st = SA.new_state(b, S)
    seqs = [W.make_qkv(1, 1, n + steps, d, d, dtype, 18000 + 7 * d + i) for i, n in enumerate(lens)]
    for i, n in enumerate(lens):
        if n:
            q, k, v = (x[:, :, :n] for x in seqs[i])
            run_prefill(b, q, k, v, dtype, state=st[i:i + 1])
    got = np.zeros((S, steps, d))
    for t in range(steps):
        qt, kt, vt = (np.stack([seqs[i][j][0, 0, lens[i] + t] for i in range(S)]) for j in range(3))
        got[:, t] = SA.decode_step(b, to_dev(qt, dtype), to_dev(kt, dtype), to_dev(vt, dtype), st).cpu().numpy()
    for i, n in enumerate(lens):
        q, k, v = (x[0, 0] for x in seqs[i])
        ref = oracle_rows(q, k, v, P, 1.0, rows=np.arange(n, n + steps))
        assert O.row_normwise_error(got[i], ref) <= TOL[dtype], (i, n)


@pytest.mark.parametrize("d,P,dtype,n", [(64, 4, W.BF16, 700), (16, 4, W.F32, 530), (32, 5, W.BF16, 700)])
def test_prefill_many_windows(d, P, dtype, n, monkeypatch):
    """A small workspace cap splits the sequence into many windows (the state
    is written back and reloaded between them); results are unchanged."""
    b = SA.build_basis(d, P, 1.0)
    q, k, v = W.make_qkv(1, 2, n, d, d, dtype, 15000 + d)
    code = SA.SATA_BF16 if dtype == W.BF16 else SA.SATA_F32
    full = SA.prefill_workspace_bytes(b, 1, 2, n, d, code)
    least = SA.prefill_workspace_bytes(b, 1, 1, min(n, 512), d, code)
    monkeypatch.setenv("SATA_PREFILL_WS_CAP", str(max(least, full // 6)))
    small = SA.prefill_workspace_bytes(b, 1, 2, n, d, code)
    note(f"many windows d={d} {dtype} n={n} ws {full} -> {small}")
    assert small < full
    out, _ = run_prefill(b, q, k, v, dtype)
    got = out.cpu().numpy()
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[dtype], h


@pytest.mark.parametrize("d,P,dtype", [(16, 4, W.BF16), (64, 4, W.BF16), (32, 5, W.BF16), (16, 4, W.F32)])
def test_prefill_head_groups_bitwise(d, P, dtype):
    """A workspace with room for two heads runs five heads (with and without
    per-head lengths) as groups of 2, 2 and 1: outputs and states are
    bit-identical to the one-group call, and the outputs match the oracle."""
    # one readout window (bf16: 512 tokens, fp32: 64-token records), so that
    # only head groups can shrink the workspace
    B, H, n = (1, 5, 480) if dtype == W.BF16 else (1, 5, 64)
    lens = [480, 1, 300, 0, 417] if dtype == W.BF16 else [64, 1, 37, 0, 63]
    note(f"head groups d={d} P={P} {dtype} H={H} n={n}")
    q, k, v = W.make_qkv(B, H, n, d, d, dtype, 28000 + d + P)
    b = SA.build_basis(d, P, 1.0)
    code = SA.SATA_BF16 if dtype == W.BF16 else SA.SATA_F32
    full = SA.prefill_workspace_bytes(b, B, H, n, d, code)
    two = SA.prefill_workspace_bytes(b, 1, 2, n, d, code)
    assert two < full
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    res = []
    for nbytes in (full, two):
        for lengths in (None, lt):
            out, st = SA.prefill(b, qd, kd, vd, ws=SA.workspace(nbytes), lengths=lengths)
            torch.cuda.synchronize()
            res.append((out.clone(), st.clone()))
    for i in range(2):
        assert torch.equal(res[i][0], res[2 + i][0]) and torch.equal(res[i][1], res[2 + i][1]), i
    got = res[2][0].cpu().numpy()
    for h in (0, 4):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[dtype], h
    gl = res[3][0].cpu().numpy()
    for h, L in enumerate(lens):
        assert np.all(gl[0, h, L:] == 0.0), h
        if L:
            ref = oracle_rows(q[0, h, :L], k[0, h, :L], v[0, h, :L], P, 1.0)
            assert O.row_normwise_error(gl[0, h, :L], ref) <= TOL[dtype], (h, L)


@pytest.mark.parametrize("d,P,dtype", [(32, 4, W.BF16), (16, 4, W.F32)])
def test_prefill_workspace_down_to_minimum(d, P, dtype):
    """Workspaces from the fastest plan's down to the one-head, one-window
    minimum (head groups, windows or both): every output matches the oracle,
    every state the fastest plan's; one byte less than the minimum is refused
    with nothing written."""
    B, H, n = 1, 5, 1300
    note(f"workspace plans d={d} P={P} {dtype} H={H} n={n}")
    q, k, v = W.make_qkv(B, H, n, d, d, dtype, 29000 + d)
    b = SA.build_basis(d, P, 1.0)
    code = SA.SATA_BF16 if dtype == W.BF16 else SA.SATA_F32
    sizes = [SA.prefill_workspace_bytes(b, B, H, n, d, code), SA.prefill_workspace_bytes(b, 1, 3, n, d, code),
             SA.prefill_workspace_bytes(b, 1, 2, 700, d, code), SA.prefill_workspace_bytes(b, 1, 1, 512, d, code)]
    assert sizes == sorted(sizes, reverse=True) and sizes[-1] < sizes[0]
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    refs = {h: oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0) for h in (0, 2, 4)}
    st0 = None
    for nbytes in sizes:
        out, st = SA.prefill(b, qd, kd, vd, ws=SA.workspace(nbytes))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for h, ref in refs.items():
            assert O.row_normwise_error(got[0, h], ref) <= TOL[dtype], (nbytes, h)
        if st0 is None:
            st0 = st.clone()
        else:
            assert torch.allclose(st, st0, rtol=1e-5, atol=1e-6 * float(st0.abs().max())), nbytes
    # below the minimum (the fp32 minimum is one 64-token record window)
    least = SA.prefill_workspace_bytes(b, 1, 1, 64, d, code) if dtype == W.F32 else sizes[-1]
    out = torch.full((B, H, n, d), 7.0, device="cuda")
    st = SA.new_state(b, B * H)
    with pytest.raises(SA.SataError) as e:
        SA.prefill(b, qd, kd, vd, state=st, out=out, ws=SA.workspace(least - 256))
    assert e.value.status == SA.SATA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.min()) == 7.0 and float(st.abs().sum()) == 0.0


def test_prefill_f32_both_tilings():
    """float32 inputs at d = 16 use 64-row tiles when the batch has few heads
    (32 here) and 128-row tiles otherwise (64 heads): both match the oracle,
    and the shared heads agree between the two calls to fp32 rounding."""
    d, P, n = 16, 4, 700
    note(f"fp32 tilings d={d} P={P} n={n} heads 32 / 64")
    q, k, v = W.make_qkv(1, 64, n, d, d, W.F32, 30000)
    b = SA.build_basis(d, P, 1.0)
    small, _ = run_prefill(b, q[:, :32], k[:, :32], v[:, :32], W.F32)
    full, _ = run_prefill(b, q, k, v, W.F32)
    gs, gf = small.cpu().numpy(), full.cpu().numpy()
    for h in (0, 31):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(gs[0, h], ref) <= TOL[W.F32], h
        assert O.row_normwise_error(gf[0, h], ref) <= TOL[W.F32], h
    ref = oracle_rows(q[0, 63], k[0, 63], v[0, 63], P, 1.0)
    assert O.row_normwise_error(gf[0, 63], ref) <= TOL[W.F32]
    assert np.max(np.abs(gs - gf[:, :32])) <= 1e-5 * np.max(np.abs(gf[:, :32]))


@pytest.mark.parametrize("d,P,n,cont", [(32, 4, 5000, False), (64, 4, 36864, False), (16, 5, 3584, False), (16, 4, 8192, True),
                                        (32, 4, 4608, True), (8, 4, 6000, False)])
def test_prefill_sequence_segments(d, P, n, cont, monkeypatch):
    """One head of a long sequence runs as parallel sequence segments (state
    passes, prefix, full passes, tail): outputs match the oracle, the state
    matches the direct state, and both agree with the call that has segments
    turned off; `cont`: from a state that already holds 700 tokens."""
    n0 = 700 if cont else 0
    note(f"sequence segments d={d} P={P} n={n} from {n0} tokens")
    q, k, v = W.make_qkv(1, 1, n0 + n, d, d, W.BF16, 32000 + d + P + n)
    b = SA.build_basis(d, P, 1.0)
    seg_ws = SA.prefill_workspace_bytes(b, 1, 1, n, d, SA.SATA_BF16)
    monkeypatch.setenv("SATA_PREFILL_SEGMENTS", "0")
    plain_ws = SA.prefill_workspace_bytes(b, 1, 1, n, d, SA.SATA_BF16)
    monkeypatch.delenv("SATA_PREFILL_SEGMENTS")
    assert seg_ws != plain_ws, "this shape should take segments"
    res = {}
    for mode in ("seg", "plain"):
        if mode == "plain":
            monkeypatch.setenv("SATA_PREFILL_SEGMENTS", "0")
        st = SA.new_state(b, 1)
        if n0:
            run_prefill(b, q[:, :, :n0], k[:, :, :n0], v[:, :, :n0], W.BF16, state=st)
        out, st = run_prefill(b, q[:, :, n0:], k[:, :, n0:], v[:, :, n0:], W.BF16, state=st)
        res[mode] = (out.cpu().numpy()[0, 0], st.cpu().numpy()[0])
        monkeypatch.delenv("SATA_PREFILL_SEGMENTS", raising=False)
    rows = np.unique(np.concatenate([np.arange(0, n, 97), np.arange(n - 40, n)]))
    ref = oracle_rows(q[0, 0], k[0, 0], v[0, 0], P, 1.0, rows=n0 + rows)
    for mode in ("seg", "plain"):
        assert O.row_normwise_error(res[mode][0][rows], ref) <= TOL[W.BF16], mode
    assert O.row_normwise_error(res["seg"][0], res["plain"][0]) <= TOL[W.BF16]
    basis = O.enumerate_basis(d, P)
    S_ref, z_ref = O.direct_state(f64(k[0, 0]), f64(v[0, 0]), basis)
    D = b.total_rows
    gS = res["seg"][1][:D * d].reshape(D, d)
    gz = res["seg"][1][D * d:D * (d + 1)]
    off = 0
    for p in range(P):
        r = slice(off, off + math.comb(d + p - 1, p))
        assert np.max(np.abs(gS[r] - S_ref[r])) <= TOL[W.BF16] * np.max(np.abs(S_ref[r])), p
        assert np.max(np.abs(gz[r] - z_ref[r])) <= TOL[W.BF16] * np.max(np.abs(z_ref[r])), p
        off = r.stop


def test_prefill_seeded_shapes_and_workspaces():
    """Seeded shapes (head dim, orders, dtype, heads, length, per-head lengths
    or not) each run with a workspace drawn between the minimum and the
    default size (so head groups, windows and segments mix): sampled rows match
    the oracle."""
    rng = np.random.default_rng(33000)
    for case in range(8):
        d = int(rng.choice([8, 16, 32, 64]))
        P = int(rng.integers(1, 6)) if d < 64 else int(rng.integers(1, 5))
        dtype = W.BF16 if rng.random() < 0.7 else W.F32
        H = int(rng.integers(1, 6))
        n = int(rng.integers(1, 3000))
        varlen = bool(rng.random() < 0.3)
        note(f"seeded case {case}: d={d} P={P} {dtype} H={H} n={n} varlen={varlen}")
        q, k, v = W.make_qkv(1, H, n, d, d, dtype, 33100 + case)
        b = SA.build_basis(d, P, 1.0)
        code = SA.SATA_BF16 if dtype == W.BF16 else SA.SATA_F32
        full = SA.prefill_workspace_bytes(b, 1, H, n, d, code)
        least = SA.prefill_workspace_bytes(b, 1, 1, min(n, 512), d, code)
        nbytes = int(least + rng.random() * max(0, full - least)) // 256 * 256
        lens = [int(rng.integers(0, n + 1)) for _ in range(H)] if varlen else [n] * H
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda") if varlen else None
        out, _ = SA.prefill(b, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), ws=SA.workspace(max(nbytes, least)),
                            lengths=lt)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[0]
        for h in range(H):
            L = lens[h]
            if L == 0:
                assert np.all(got[h] == 0.0)
                continue
            rows = np.unique(np.concatenate([np.arange(0, L, max(1, L // 40)), [L - 1]]))
            ref = oracle_rows(q[0, h, :L], k[0, h, :L], v[0, h, :L], P, 1.0, rows=rows)
            assert O.row_normwise_error(got[h, rows], ref) <= TOL[dtype], (case, h)
            assert np.all(got[h, L:] == 0.0), (case, h)


def test_misaligned_and_host_only_rejected():
    note("misaligned pointers / host-only handle on the GPU")
    b = SA.build_basis(16, 4, 1.0)
    x = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(1024, dtype=torch.float32, device="cuda")
    st = SA.new_state(b, 1)
    ws = SA.workspace(1 << 20)
    L = SA.lib()
    p = x.data_ptr()
    # q not 16-byte aligned
    assert L.sata_prefill(b.handle, 1, 1, 8, 16, SA.SATA_BF16, p + 2, p, p, out.data_ptr(), st.data_ptr(),
                          ws.data_ptr(), ws.numel(), None) == SA.SATA_ERR_INVALID_ARG
    # decode: out not 16-byte aligned
    assert L.sata_decode_step(b.handle, 1, 16, SA.SATA_BF16, p, p, p, out.data_ptr() + 4, st.data_ptr(),
                              ws.data_ptr(), ws.numel(), None) == SA.SATA_ERR_INVALID_ARG
    hb = SA.build_basis(16, 4, 1.0, host_only=True)
    assert L.sata_decode_step(hb.handle, 1, 16, SA.SATA_BF16, p, p, p, out.data_ptr(), st.data_ptr(),
                              ws.data_ptr(), ws.numel(), None) == SA.SATA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert float(st.abs().sum()) == 0.0 and float(out.abs().sum()) == 0.0


def test_binding_rejects_bad_buffers():
    """The binding checks what the C calls cannot see: d_k of the inputs and
    the size, dtype and device of caller-provided state / out buffers."""
    note("binding argument checks")
    b = SA.build_basis(16, 3, 1.0)
    q = torch.zeros((1, 2, 8, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="d_k"):
        SA.prefill(b, q[..., :8].contiguous(), q[..., :8].contiguous(), q[..., :8].contiguous())
    with pytest.raises(ValueError, match="state"):
        SA.prefill(b, q, q, q, state=SA.new_state(b, 1))
    with pytest.raises(ValueError, match="state"):
        SA.prefill(b, q, q, q, state=SA.new_state(b, 2).to(torch.float64))
    with pytest.raises(ValueError, match="out"):
        SA.prefill(b, q, q, q, out=torch.zeros((1, 2, 7, 16), device="cuda"))
    with pytest.raises(TypeError):
        SA.prefill(b, q, q.float(), q)
    q1 = torch.zeros((3, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="state"):
        SA.decode_step(b, q1, q1, q1, SA.new_state(b, 2))
    with pytest.raises(ValueError, match="out"):
        SA.decode_step(b, q1, q1, q1, SA.new_state(b, 3), out=torch.zeros((2, 16), device="cuda"))
    with pytest.raises(ValueError, match="contiguous"):
        SA.decode_step(b, torch.zeros((16, 3), device="cuda").t(), q1, q1, SA.new_state(b, 3))
    torch.cuda.synchronize()


def _rows_bf16(x):
    return W.round_bf16(np.asarray(x, dtype=np.float64)).astype(np.float32)


@pytest.mark.parametrize("d,P", [(32, 4), (64, 4), (16, 5), (32, 5)])
def test_prefill_bf16_scaled_inputs(d, P):
    """bf16 inputs far from unit scale (v x 3000, k x 1/64, q x 64: the logits
    are unchanged) exercise the per-head power-of-two operand scaling (the
    state of an order-p row carries 2^-(p ek + ev))."""
    note(f"scaled bf16 inputs d={d} P={P}")
    n = 600
    q, k, v = W.make_qkv(1, 2, n, d, d, W.F32, 16000 + d)
    q, k, v = _rows_bf16(q * 64.0), _rows_bf16(k / 64.0), _rows_bf16(v * 3000.0)
    b = SA.build_basis(d, P, 1.0)
    out, st = run_prefill(b, q, k, v, W.BF16)
    got = out.cpu().numpy()
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[W.BF16], h
    # the state written back is the canonical one, order by order
    basis = O.enumerate_basis(d, P)
    D = b.total_rows
    S, z = O.direct_state(f64(k[0, 1]), f64(v[0, 1]), basis)
    gS = st.cpu().numpy()[1, :D * d].reshape(D, d)
    off = 0
    for p in range(P):
        rows = slice(off, off + math.comb(d + p - 1, p))
        assert np.max(np.abs(gS[rows] - S[rows])) <= TOL[W.BF16] * np.max(np.abs(S[rows])), p
        off = rows.stop


@pytest.mark.parametrize("d,P,q0,kf", [(32, 4, 12.0, 1e-2), (64, 4, 12.0, 1e-2), (32, 5, 12.0, 1e-2),
                                       (32, 4, 40.0, 1e-2), (64, 4, 40.0, 1e-2), (16, 4, 40.0, 1e-2),
                                       (32, 4, 1000.0, 1e-4), (64, 5, 1000.0, 1e-4)])
def test_prefill_bf16_large_query_coordinates(d, P, q0, kf):
    """A query coordinate far larger than the keys' scale (first coordinate of
    q = q0, first coordinate of k ~ 1e-3) with moderate logits: the per-head
    power of two moves magnitude from q to k (q' = q 2^ek, k' = k 2^-ek) so
    that both sides' features fit the f16 operand path, whose readout operand
    is then scaled down to keep the wave partials in range.  q0 = 1000 (key
    coordinate x 1e-4) leaves query features beyond 2^12 even after the
    split, so those heads run the bf16 operand path."""
    note(f"large query coordinates d={d} P={P} q0={q0}")
    n = 1100   # three readout windows: the scan's readout carries the first 512 keys
    q, k, v = W.make_qkv(1, 2, n, d, d, W.F32, 17000 + d)
    q = q.copy()
    k = k.copy()
    q[..., 0] = q0
    k[..., 0] *= kf
    q, k, v = _rows_bf16(q), _rows_bf16(k), _rows_bf16(v)
    b = SA.build_basis(d, P, 1.0)
    out, _ = run_prefill(b, q, k, v, W.BF16)
    got = out.cpu().numpy()
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[W.BF16], h


def _bf16_operand_path(q, k, P):
    """Whether a head takes the bf16 operand path: the exact power-of-two split
    of the magnitude between q and k (the same rule as the kernels': |q| < 2^eq,
    |k| < 2^ekk, ek = (ekk - eq) / 2 truncated) leaves query or key features,
    products of up to P-1 coordinates, at or beyond 2^13."""
    eq = math.frexp(float(np.max(np.abs(q))))[1]
    ekk = math.frexp(float(np.max(np.abs(k))))[1]
    ek = int((ekk - eq) / 2)
    return (P - 1) * max(eq + ek, 0) > 12 or (P - 1) * max(ekk - ek, 0) > 12


@pytest.mark.parametrize("d,P,n", [(8, 4, 2000), (8, 4, 4096), (8, 5, 2000), (8, 5, 4096),
                                   (16, 4, 2000), (16, 4, 4096), (16, 5, 2000), (16, 5, 4096),
                                   (32, 4, 4096), (32, 5, 2000), (64, 4, 4096)])
def test_prefill_bf16_operand_path_small_heads(d, P, n):
    """Heads forced onto the bf16 operand path (a query coordinate of 1000,
    the matching key coordinate x 1e-4) over several readout windows; at
    d <= 32 the path carries its readout operand and wave partials as bf16
    value + residual pairs (few rows per output at small d)."""
    note(f"bf16 operand path d={d} P={P} n={n}")
    q, k, v = W.make_qkv(1, 2, n, d, d, W.F32, 19000 + d + P)
    q = q.copy()
    k = k.copy()
    q[..., 0] = 1000.0
    k[..., 0] *= 1e-4
    q, k, v = _rows_bf16(q), _rows_bf16(k), _rows_bf16(v)
    for h in range(2):
        assert _bf16_operand_path(q[0, h], k[0, h], P), h
    b = SA.build_basis(d, P, 1.0)
    out, _ = run_prefill(b, q, k, v, W.BF16)
    got = out.cpu().numpy()
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref) <= TOL[W.BF16], h


@pytest.mark.parametrize("d,P,dtype", [(8, 3, W.F32), (16, 4, W.BF16), (64, 4, W.BF16)])
def test_packed_state_layout_c_abi(d, P, dtype):
    """sata_prefill and sata_decode_step with heads packed state_floats apart
    (an odd count at these sizes, so every other head starts 4 bytes past a
    16-byte boundary) and the buffer itself 4 bytes off: outputs match the
    oracle, the state equals the padded layout's bit for bit, and guard words
    before and after the buffer are untouched."""
    note(f"packed state layout d={d} P={P} {dtype}")
    H, n, steps = 3, 200, 4
    q, k, v = W.make_qkv(1, H, n + steps, d, d, dtype, 21000 + d)
    b = SA.build_basis(d, P, 1.0)
    F = b.state_floats()
    assert F % 2 == 1
    G = 64
    code = SA.SATA_BF16 if dtype == W.BF16 else SA.SATA_F32
    buf = torch.full((H * F + 2 * G + 1,), 1234.5, dtype=torch.float32, device="cuda")
    st_ptr = buf.data_ptr() + 4 * (G + 1)            # 4-byte aligned, not 16
    L = SA.lib()
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    qp, kp, vp = (x[:, :, :n].contiguous() for x in (qd, kd, vd))
    out = torch.empty((1, H, n, d), dtype=torch.float32, device="cuda")
    ws = SA.workspace(SA.prefill_workspace_bytes(b, 1, H, n, d, code))
    # the state region starts zeroed (empty prefix)
    buf[G + 1:G + 1 + H * F] = 0.0
    st = L.sata_prefill(b.handle, 1, H, n, d, code, qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), out.data_ptr(),
                        st_ptr, ws.data_ptr(), ws.numel(), SA._stream_ptr(torch.device("cuda")))
    assert st == SA.SATA_OK, SA.status_string(st)
    dws = SA.workspace(SA.decode_workspace_bytes(b, H, d, code))
    dout = torch.empty((steps, H, d), dtype=torch.float32, device="cuda")
    for t in range(steps):
        qt, kt, vt = (x[0, :, n + t].contiguous() for x in (qd, kd, vd))
        st = L.sata_decode_step(b.handle, H, d, code, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                dout[t].data_ptr(), st_ptr, dws.data_ptr(), dws.numel(),
                                SA._stream_ptr(torch.device("cuda")))
        assert st == SA.SATA_OK, SA.status_string(st)
    torch.cuda.synchronize()
    # guard words
    assert torch.all(buf[:G + 1] == 1234.5) and torch.all(buf[G + 1 + H * F:] == 1234.5)
    # the same calls on the padded layout give the same bits
    out2, st2 = SA.prefill(b, qp, kp, vp)
    dout2 = torch.stack([SA.decode_step(b, *(x[0, :, n + t].contiguous() for x in (qd, kd, vd)), st2)
                         for t in range(steps)])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(dout, dout2)
    packed = buf[G + 1:G + 1 + H * F].view(H, F)
    assert torch.equal(packed, st2[:, :F])
    tol = TOL[dtype]
    got = out.cpu().numpy()
    gd = dout.cpu().numpy()
    for h in range(H):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, 1.0)
        assert O.row_normwise_error(got[0, h], ref[:n]) <= tol, h
        assert O.row_normwise_error(gd[:, h], ref[n:]) <= tol, h


@pytest.mark.parametrize("d,P,s", [(32, 4, 1024.0), (64, 4, 1024.0), (16, 5, 64.0), (64, 4, 1.0 / 64.0),
                                   (32, 5, 3.0 * 256.0)])
def test_prefill_bf16_logit_scale(d, P, s):
    """q scaled by s with c = s (the logits of unit rows): the power of two of
    c is folded into the staged queries and the row weights, so such heads
    keep the f16 operand path; parity against the oracle at that c."""
    note(f"logit scale d={d} P={P} c={s}")
    n = 1100
    q, k, v = W.make_qkv(1, 2, n, d, d, W.F32, 29000 + d + P)
    q = _rows_bf16(q * s)
    k, v = _rows_bf16(k), _rows_bf16(v)
    b = SA.build_basis(d, P, s)
    out, _ = run_prefill(b, q, k, v, W.BF16)
    got = out.cpu().numpy()
    for h in range(2):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], P, s)
        err = O.row_normwise_error(got[0, h], ref)
        note(f"  head {h}: {err:.3e}")
        assert err <= TOL[W.BF16], h


def test_two_streams_share_a_basis():
    """Prefill and decode of two state batches on two streams at once, with
    one basis, give bit for bit what they give one after the other."""
    note("two streams, one basis")
    d, P, dtype, n, steps = 32, 4, W.BF16, 300, 6
    b = SA.build_basis(d, P, 1.0)
    ins = [W.make_qkv(1, 3, n + steps, d, d, dtype, 15000 + i) for i in range(2)]
    dev = [tuple(to_dev(x[0], dtype) for x in qkv) for qkv in ins]

    def run(i):
        q, k, v = dev[i]
        out, st = SA.prefill(b, q[None, :, :n].contiguous(), k[None, :, :n].contiguous(),
                             v[None, :, :n].contiguous())
        dec = [SA.decode_step(b, q[:, n + t].contiguous(), k[:, n + t].contiguous(),
                              v[:, n + t].contiguous(), st) for t in range(steps)]
        return out, st, torch.stack(dec)

    ref = [run(0), run(1)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for i in range(2):
        with torch.cuda.stream(streams[i]):
            got[i] = run(i)
    torch.cuda.synchronize()
    for i in range(2):
        for a, r in zip(got[i], ref[i]):
            assert torch.equal(a, r), i


def test_prefill_deterministic():
    note("prefill run-twice bitwise")
    d, P, dtype = 32, 4, W.BF16
    q, k, v = W.make_qkv(1, 2, 400, d, d, dtype, 14000)
    b = SA.build_basis(d, P, 1.0)
    o1, s1 = run_prefill(b, q, k, v, dtype)
    o2, s2 = run_prefill(b, q, k, v, dtype)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_workspace_too_small_changes_nothing():
    note("workspace too small")
    d = 16
    b = SA.build_basis(d, 4, 1.0)
    q = torch.randn(1, 1, 64, d, device="cuda")
    out = torch.full((1, 1, 64, d), 7.0, device="cuda")
    st = SA.new_state(b, 1)
    with pytest.raises(SA.SataError) as e:
        SA.prefill(b, q, q, q, state=st, out=out, ws=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == SA.SATA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.min()) == 7.0 and float(st.abs().sum()) == 0.0


# ----------------------------------------------------------------------------
# The study's workloads at full size (sampled rows where the oracle is O(n) per row)
# ----------------------------------------------------------------------------

def test_workload_d16_n4096_full():
    w = W.WORKLOADS["d16_n4096"]
    note(f"workload {w.name} B={w.B} H={w.H} n={w.n}")
    q, k, v = W.workload_inputs(w)
    b = SA.build_basis(w.d_k, w.P, w.c)
    out, _ = run_prefill(b, q, k, v, w.dtype)
    got = out.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(0, w.n, 97), np.arange(w.n - 64, w.n)]))
    for bb in range(w.B):
        for h in range(w.H):
            full = (bb, h) in ((0, 0), (w.B - 1, w.H - 1))
            rr = None if full else rows
            ref = oracle_rows(q[bb, h], k[bb, h], v[bb, h], w.P, w.c, rows=rr)
            g = got[bb, h] if full else got[bb, h][rows]
            assert O.row_normwise_error(g, ref) <= TOL[w.dtype], (bb, h)


def test_workload_d64_n16384_sampled():
    w = W.WORKLOADS["d64_n16384"]
    note(f"workload {w.name} B={w.B} H={w.H} n={w.n}")
    q, k, v = W.workload_inputs(w)
    b = SA.build_basis(w.d_k, w.P, w.c)
    out, _ = run_prefill(b, q, k, v, w.dtype)
    got = out.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(0, w.n, 61), np.arange(w.n - 40, w.n)]))
    for h in range(w.H):
        ref = oracle_rows(q[0, h], k[0, h], v[0, h], w.P, w.c, rows=rows)
        assert O.row_normwise_error(got[0, h][rows], ref) <= TOL[w.dtype], h


def test_workload_decode_256x4096_d64():
    """256 resident states: 4096-token prefill, then decode steps; every
    decode output and sampled prefill rows of 8 states are checked."""
    w = W.WORKLOADS["decode_256x4096_d64"]
    steps = 16
    note(f"workload {w.name} states={w.B * w.H} n={w.n} steps={steps}")
    q, k, v = W.workload_inputs(w)
    qs, ks, vs = W.decode_inputs(w, steps)
    b = SA.build_basis(w.d_k, w.P, w.c)
    out, st = run_prefill(b, q, k, v, w.dtype)
    got_p = out.cpu().numpy().reshape(w.B * w.H, w.n, w.d_v)
    del out
    S = w.B * w.H
    qd, kd, vd = to_dev(qs, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype)
    got_d = np.zeros((steps, S, w.d_v))
    for s in range(steps):
        got_d[s] = SA.decode_step(b, qd[s], kd[s], vd[s], st).cpu().numpy()
    qf = q.reshape(S, w.n, w.d_k)
    kf = k.reshape(S, w.n, w.d_k)
    vf = v.reshape(S, w.n, w.d_v)
    g = np.random.Generator(np.random.PCG64(4321))
    for s in g.choice(S, size=8, replace=False):
        rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(0, w.n, 127), [w.n - 1]]))
        ref = oracle_rows(qf[s], kf[s], vf[s], w.P, w.c, rows=rows)
        assert O.row_normwise_error(got_p[s][rows], ref) <= TOL[w.dtype], ("prefill", s)
    for s in range(S):
        qq = np.concatenate([qf[s], qs[:, s]])
        kk = np.concatenate([kf[s], ks[:, s]])
        vv = np.concatenate([vf[s], vs[:, s]])
        ref = oracle_rows(qq, kk, vv, w.P, w.c, rows=np.arange(w.n, w.n + steps))
        assert O.row_normwise_error(got_d[:, s], ref) <= TOL[w.dtype], ("decode", s)


def test_workload_order5_32x4096_d64():
    """Orders 0..4 at d = 64, 32 states: 4096-token prefill (sampled rows of
    four states), then decode steps (every output checked)."""
    w = W.WORKLOADS["order5_32x4096_d64"]
    steps = 8
    note(f"workload {w.name} states={w.B * w.H} n={w.n} steps={steps}")
    q, k, v = W.workload_inputs(w)
    qs, ks, vs = W.decode_inputs(w, steps)
    b = SA.build_basis(w.d_k, w.P, w.c)
    out, st = run_prefill(b, q, k, v, w.dtype)
    S = w.B * w.H
    got_p = out.cpu().numpy().reshape(S, w.n, w.d_v)
    del out
    qd, kd, vd = to_dev(qs, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype)
    got_d = np.zeros((steps, S, w.d_v))
    for s in range(steps):
        got_d[s] = SA.decode_step(b, qd[s], kd[s], vd[s], st).cpu().numpy()
    qf, kf, vf = (x.reshape(S, w.n, -1) for x in (q, k, v))
    g = np.random.Generator(np.random.PCG64(4322))
    for s in g.choice(S, size=4, replace=False):
        rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(0, w.n, 127), [w.n - 1]]))
        ref = oracle_rows(qf[s], kf[s], vf[s], w.P, w.c, rows=rows)
        assert O.row_normwise_error(got_p[s][rows], ref) <= TOL[w.dtype], ("prefill", s)
    for s in range(S):
        qq, kk, vv = (np.concatenate([a[s], b_[:, s]]) for a, b_ in ((qf, qs), (kf, ks), (vf, vs)))
        ref = oracle_rows(qq, kk, vv, w.P, w.c, rows=np.arange(w.n, w.n + steps))
        assert O.row_normwise_error(got_d[:, s], ref) <= TOL[w.dtype], ("decode", s)


def test_workload_long_d32_n1m_sampled():
    w = W.WORKLOADS["long_d32_n1m"]
    note(f"workload {w.name} H={w.H} n={w.n}")
    rows = W.sampled_rows(w.n)
    b = SA.build_basis(w.d_k, w.P, w.c)
    Q = torch.empty((1, w.H, w.n, w.d_k), dtype=torch.bfloat16, device="cuda")
    K = torch.empty_like(Q)
    V = torch.empty((1, w.H, w.n, w.d_v), dtype=torch.bfloat16, device="cuda")
    host = []
    for h in range(w.H):
        q, k, v = W.head_inputs(w, h)
        Q[0, h] = to_dev(q, w.dtype)
        K[0, h] = to_dev(k, w.dtype)
        V[0, h] = to_dev(v, w.dtype)
        host.append((q, k, v))
    out, _ = SA.prefill(b, Q, K, V)
    torch.cuda.synchronize()
    got = out[0][:, torch.from_numpy(rows).to("cuda")].cpu().numpy()
    del out, Q, K, V
    for h in range(w.H):
        q, k, v = host[h]
        ref = O.direct_taylor(f64(q), f64(k), f64(v), w.P, w.c, rows=rows, block=8)
        assert O.row_normwise_error(got[h], ref) <= TOL[w.dtype], h


# ----------------------------------------------------------------------------
# Mixed-precision decode state (orders >= 2 of S in float16)
# ----------------------------------------------------------------------------

def test_mixed_state_decode_workload_1024_steps():
    """Eight states of the decode workload (d = 64, P = 4, bf16): 4096-token
    prefill on the float32 state, hand-off to the mixed state, 1024 decode
    steps; every decode output checked against the oracle."""
    w = W.WORKLOADS["decode_256x4096_d64"]
    S, steps = 8, 1024
    note(f"mixed state: {S} states, n={w.n}, {steps} decode steps")
    q, k, v = W.make_qkv(1, S, w.n, w.d_k, w.d_v, w.dtype, 1000 * w.seed)
    qs, ks, vs = W.make_qkv(1, steps, S, w.d_k, w.d_v, w.dtype, 1000 * w.seed + 100)
    qs, ks, vs = qs[0], ks[0], vs[0]
    b = SA.build_basis(w.d_k, w.P, w.c)
    _, st = run_prefill(b, q, k, v, w.dtype)
    mixed = SA.to_mixed(b, st)
    qd, kd, vd = to_dev(qs, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype)
    dout = torch.empty((steps, S, w.d_v), dtype=torch.float32, device="cuda")
    ws = SA.workspace(SA.decode_mixed_workspace_bytes(b, S, w.d_v, SA.SATA_BF16))
    for t in range(steps):
        SA.decode_step_mixed(b, qd[t], kd[t], vd[t], mixed, out=dout[t], ws=ws)
    torch.cuda.synchronize()
    got = dout.cpu().numpy()
    for s in range(S):
        qq = np.concatenate([q[0, s], qs[:, s]])
        kk = np.concatenate([k[0, s], ks[:, s]])
        vv = np.concatenate([v[0, s], vs[:, s]])
        ref = oracle_rows(qq, kk, vv, w.P, w.c, rows=np.arange(w.n, w.n + steps))
        assert O.row_normwise_error(got[:, s], ref) <= TOL[w.dtype], s


@pytest.mark.parametrize("d,P,dtype,steps", [(8, 3, W.F32, 60), (8, 3, W.BF16, 40), (16, 4, W.BF16, 40), (32, 4, W.BF16, 30),
                                             (32, 5, W.BF16, 20), (64, 4, W.F32, 12), (64, 5, W.BF16, 6)])
def test_mixed_state_decode_from_empty(d, P, dtype, steps):
    """Mixed decode from an empty state: every tile's scale is re-chosen as
    the state grows from zero."""
    note(f"mixed decode from empty d={d} P={P} {dtype} steps={steps}")
    S = 3
    q, k, v = W.make_qkv(1, S, steps, d, d, dtype, 24000 + d + P)
    b = SA.build_basis(d, P, 1.0)
    mixed = SA.to_mixed(b, SA.new_state(b, S))
    qd, kd, vd = to_dev(q[0], dtype), to_dev(k[0], dtype), to_dev(v[0], dtype)
    got = np.zeros((S, steps, d))
    for t in range(steps):
        got[:, t] = SA.decode_step_mixed(b, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                                         mixed).cpu().numpy()
    for s in range(S):
        ref = oracle_rows(q[0, s], k[0, s], v[0, s], P, 1.0)
        assert O.row_normwise_error(got[s], ref) <= 3e-3, s


@pytest.mark.parametrize("d,P", [(16, 4), (64, 4)])
def test_mixed_state_round_trip(d, P):
    """fp32 -> mixed -> fp32: rows of orders 0 and 1 and z come back bit for
    bit; rows of higher order within half an f16 ulp of their tile's scale
    (relative 2^-11 of each value, absolute 2^-25 of the tile's largest)."""
    note(f"mixed round trip d={d} P={P}")
    n, S = 300, 3
    q, k, v = W.make_qkv(1, S, n, d, d, W.BF16, 25000 + d)
    v = v * 50.0   # values well away from 1
    b = SA.build_basis(d, P, 1.0)
    _, st = run_prefill(b, q, k, _rows_bf16(v), W.BF16)
    back = SA.from_mixed(b, SA.to_mixed(b, st))
    torch.cuda.synchronize()
    a = st.cpu().numpy().astype(np.float64)
    r = back.cpu().numpy().astype(np.float64)
    D = b.total_rows
    lo = 1 + d
    F = b.state_floats()
    np.testing.assert_array_equal(r[:, :lo * d], a[:, :lo * d])
    np.testing.assert_array_equal(r[:, D * d:F], a[:, D * d:F])
    hi_a = a[:, lo * d:D * d]
    hi_r = r[:, lo * d:D * d]
    tile_max = np.max(np.abs(hi_a))
    assert np.all(np.abs(hi_r - hi_a) <= np.abs(hi_a) * 2.0 ** -11 + tile_max * 2.0 ** -25)


# ----------------------------------------------------------------------------
# Per-head lengths (one call for sequences of different lengths)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,P,dtype", [(64, 4, W.BF16), (16, 4, W.F32), (32, 5, W.BF16), (8, 3, W.F32)])
def test_prefill_varlen(d, P, dtype):
    """Six heads of lengths 0, 1, 63, 64, 513 and 700 in one [2, 3, 700]
    call, NaN in every slot past a head's length: each head's rows equal its
    own causal attention, rows past its length are zero, and its state holds
    exactly its own tokens."""
    lens = [0, 1, 63, 64, 513, 700]
    B, H, n = 2, 3, 700
    note(f"varlen prefill d={d} P={P} {dtype} lens={lens}")
    q, k, v = W.make_qkv(B, H, n, d, d, dtype, 26000 + d + P)
    qn, kn, vn = (x.copy().reshape(B * H, n, -1) for x in (q, k, v))
    for h, L in enumerate(lens):
        for x in (qn, kn, vn):
            x[h, L:] = np.nan
    qn, kn, vn = (x.reshape(B, H, n, -1) for x in (qn, kn, vn))
    b = SA.build_basis(d, P, 1.0)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, st = SA.prefill(b, to_dev(qn, dtype), to_dev(kn, dtype), to_dev(vn, dtype), lengths=lt)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B * H, n, d)
    sts = st.cpu().numpy()
    basis = O.enumerate_basis(d, P)
    D = b.total_rows
    qf, kf, vf = (x.reshape(B * H, n, -1) for x in (q, k, v))
    for h, L in enumerate(lens):
        assert np.all(got[h, L:] == 0.0), h
        if L:
            ref = oracle_rows(qf[h, :L], kf[h, :L], vf[h, :L], P, 1.0)
            assert O.row_normwise_error(got[h, :L], ref) <= TOL[dtype], (h, L)
        S_ref, z_ref = O.direct_state(f64(kf[h, :L]), f64(vf[h, :L]), basis)
        gS = sts[h, :D * d].reshape(D, d)
        gz = sts[h, D * d:D * (d + 1)]
        assert np.all(np.isfinite(gS)) and np.all(np.isfinite(gz)), h
        if L == 0:
            assert np.all(gS == 0) and np.all(gz == 0), h
            continue
        off = 0
        for p in range(P):
            rows = slice(off, off + math.comb(d + p - 1, p))
            assert np.max(np.abs(gS[rows] - S_ref[rows])) <= TOL[dtype] * np.max(np.abs(S_ref[rows])) + 1e-30, (h, p)
            assert np.max(np.abs(gz[rows] - z_ref[rows])) <= TOL[dtype] * np.max(np.abs(z_ref[rows])) + 1e-30, (h, p)
            off = rows.stop


@pytest.mark.parametrize("d,P,dtype", [(64, 4, W.BF16), (16, 4, W.F32)])
def test_prefill_varlen_mixes_decode_steps_and_chunks(d, P, dtype):
    """States prefilled to 0, 5, 200 and 600 tokens continue in one varlen
    call with lengths 1, 1, 64 and 1 (three decode steps and a 64-token chunk
    in one batch), then take one sata_decode_step each: every row matches the
    oracle on the concatenated sequence."""
    before = [0, 5, 200, 600]
    now = [1, 1, 64, 1]
    S = len(before)
    note(f"varlen continuation d={d} P={P} {dtype} {before} + {now}")
    total = [a + c + 1 for a, c in zip(before, now)]
    seqs = [W.make_qkv(1, 1, t, d, d, dtype, 27000 + 7 * d + i) for i, t in enumerate(total)]
    b = SA.build_basis(d, P, 1.0)
    st = SA.new_state(b, S)
    for i, L in enumerate(before):
        if L:
            run_prefill(b, *(x[:, :, :L] for x in seqs[i]), dtype, state=st[i:i + 1])
    nmax = max(now)
    qb = np.zeros((1, S, nmax, d), dtype=np.float32)
    kb, vb = qb.copy(), qb.copy()
    for i in range(S):
        for x, dst in zip(seqs[i], (qb, kb, vb)):
            dst[0, i, :now[i]] = x[0, 0, before[i]:before[i] + now[i]]
    lt = torch.tensor(now, dtype=torch.int32, device="cuda")
    out, _ = SA.prefill(b, to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), state=st, lengths=lt)
    last = [np.stack([seqs[i][j][0, 0, total[i] - 1] for i in range(S)]) for j in range(3)]
    dec = SA.decode_step(b, *(to_dev(x, dtype) for x in last), st)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    gd = dec.cpu().numpy()
    for i in range(S):
        q, k, v = (x[0, 0] for x in seqs[i])
        ref = oracle_rows(q, k, v, P, 1.0, rows=np.arange(before[i], total[i]))
        assert O.row_normwise_error(got[i, :now[i]], ref[:now[i]]) <= TOL[dtype], i
        assert np.all(got[i, now[i]:] == 0.0), i
        assert O.row_normwise_error(gd[i:i + 1], ref[now[i]:]) <= TOL[dtype], i


# ----------------------------------------------------------------------------
# Exact causal softmax attention (the baseline)
# ----------------------------------------------------------------------------

SOFTMAX_CASES = [
    # B, H, n, d, c, query scale, dtype
    (1, 1, 1, 64, 1.0, 1.0, W.F32), (1, 2, 300, 8, 1.0, 1.0, W.F32), (2, 1, 257, 16, 0.5, 1.0, W.F32),
    (1, 1, 700, 32, 1.0, 1.0, W.F32), (1, 1, 513, 64, 1.0, 100.0, W.F32),
    (1, 1, 1, 64, 1.0, 1.0, W.BF16), (1, 2, 63, 8, 1.0, 1.0, W.BF16), (1, 1, 64, 16, 1.0, 1.0, W.BF16),
    (2, 1, 65, 32, 0.5, 1.0, W.BF16), (1, 2, 1100, 64, 1.0, 1.0, W.BF16), (1, 1, 777, 64, 1.0, 100.0, W.BF16),
    (1, 1, 2048, 32, 1.0, 8.0, W.BF16),
]


@pytest.mark.parametrize("case", SOFTMAX_CASES, ids=[f"{c[6]}-n{c[2]}-d{c[3]}-x{c[5]:g}" for c in SOFTMAX_CASES])
def test_softmax_attention(case):
    """Stable causal softmax against the oracle's exact_softmax; logits up to
    about 100 (query scale 100) would overflow float32 without the running
    maximum."""
    B, H, n, d, c, qs, dtype = case
    note(f"softmax B={B} H={H} n={n} d={d} c={c} q x {qs} {dtype}")
    q, k, v = W.make_qkv(B, H, n, d, d, W.F32, 28000 + n + d)
    q = q * qs
    if dtype == W.BF16:
        q, k, v = _rows_bf16(q), _rows_bf16(k), _rows_bf16(v)
    out = SA.softmax_attention(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), c)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for bb in range(B):
        for h in range(H):
            ref = O.exact_softmax(f64(q[bb, h]), f64(k[bb, h]), f64(v[bb, h]), c)
            assert O.row_normwise_error(got[bb, h], ref) <= TOL[dtype], (bb, h)
