"""The allocation-free decode entry point (sata_decode_step_noalloc) against
sata_decode_step_strided, through the C ABI: two calls in a row on one state
batch, the second with fewer states, each bit-identical to the workspace
entry point on a copy of the same states, and within the bf16 gate of the
float64 oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import sata_oracle as O

torch = pytest.importorskip("torch")
import constant_cost_taylor_amd as SA  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to("cuda")


@pytest.mark.parametrize("d,P,S1,S2", [(64, 4, 40, 7), (16, 4, 200, 3)])
def test_decode_noalloc_matches_workspace_call(d, P, S1, S2):
    print(f"[gpu case] decode noalloc d={d} P={P} S={S1} then {S2}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n = 130
    q, k, v = W.make_qkv(1, S1, n + 2, d, d, W.BF16, 23000 + d)
    b = SA.build_basis(d, P, 1.0)
    L = SA.lib()
    stream = SA._stream_ptr(torch.device("cuda"))
    need = SA.decode_workspace_bytes(b, S1, d, SA.SATA_BF16)
    assert need <= L.sata_decode_noalloc_max_bytes()
    # both layouts reach the same state through one prefill
    _, st_a = SA.prefill(b, _dev(q[:, :, :n]), _dev(k[:, :, :n]), _dev(v[:, :, :n]))
    st_b = st_a.clone()
    qd, kd, vd = _dev(q[0]), _dev(k[0]), _dev(v[0])
    for step, S in enumerate((S1, S2)):
        t = n + step
        qt, kt, vt = (x[:S, t].contiguous() for x in (qd, kd, vd))
        out_a = torch.full((S, d), float("nan"), device="cuda")
        out_b = torch.full((S, d), float("nan"), device="cuda")
        ws = SA.workspace(SA.decode_workspace_bytes(b, S, d, SA.SATA_BF16))
        r = L.sata_decode_step_strided(b.handle, S, d, SA.SATA_BF16, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                       out_a.data_ptr(), st_a.data_ptr(), st_a.shape[1], ws.data_ptr(),
                                       ws.numel(), stream)
        assert r == SA.SATA_OK, SA.status_string(r)
        r = L.sata_decode_step_noalloc(b.handle, S, d, SA.SATA_BF16, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                       out_b.data_ptr(), st_b.data_ptr(), st_b.shape[1], stream)
        assert r == SA.SATA_OK, SA.status_string(r)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), step
        assert torch.equal(st_a[:S], st_b[:S]), step
        got = out_b.cpu().numpy()
        for s in range(S):
            ref = O.direct_taylor(q[0, s, :t + 1].astype(np.float64), k[0, s, :t + 1].astype(np.float64),
                                  v[0, s, :t + 1].astype(np.float64), P, 1.0, rows=[t])
            assert O.row_normwise_error(got[s:s + 1], ref) <= 3e-3, (step, s)
    # the smallest call beyond the static scratch (found with the host-side
    # size query the entry point uses) is refused before any launch; the
    # buffers passed are real and large enough all the same
    cap = L.sata_decode_noalloc_max_bytes()
    big = S1
    while SA.decode_workspace_bytes(b, big, d, SA.SATA_BF16) <= cap:
        big += 1
    if big <= 128:
        qb = torch.zeros((big, d), dtype=torch.bfloat16, device="cuda")
        ob = torch.zeros((big, d), device="cuda")
        sb = SA.new_state(b, big)
        r = L.sata_decode_step_noalloc(b.handle, big, d, SA.SATA_BF16, qb.data_ptr(), qb.data_ptr(), qb.data_ptr(),
                                       ob.data_ptr(), sb.data_ptr(), sb.shape[1], stream)
        assert r == SA.SATA_ERR_SCRATCH
        torch.cuda.synchronize()
        assert float(ob.abs().sum()) == 0.0 and float(sb.abs().sum()) == 0.0
