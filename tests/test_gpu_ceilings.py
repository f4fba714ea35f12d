"""The ceiling kernels (libsata_ceilings.so) compute what they claim, so that
the rates the bench derives from them count real work."""
import pytest

torch = pytest.importorskip("torch")
from constant_cost_taylor_amd import ceilings as CL  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    CL.lib()


def _sp():
    return torch.cuda.current_stream().cuda_stream


def test_copy_rmw_read():
    print("[gpu case] ceiling streams, 1 MiB + 48 bytes", flush=True)
    g = torch.Generator(device="cuda").manual_seed(3)
    n = (1 << 18) + 12          # a ragged last block
    src = torch.randn(n, generator=g, device="cuda")
    dst = torch.zeros_like(src)
    CL.copy(src, dst, _sp())
    buf = src.clone()
    CL.rmw(buf, _sp())
    part = torch.zeros(CL.read_partials(n * 4), device="cuda")
    CL.read(src, part, _sp())
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.equal(buf, src * 0.5 + 1.0)
    assert part.numel() == -(-n // 4096)       # 1024 16-byte vectors a block
    assert abs(float(part.double().sum()) - float(src.double().sum())) <= 1e-3 * float(src.abs().sum())


@pytest.mark.parametrize("code", [1, 0])
def test_mfma_loop_is_linear_in_iterations(code):
    print(f"[gpu case] ceiling mfma loop dtype {code}", flush=True)
    blocks = 3
    o1 = torch.zeros(blocks * 512, device="cuda")
    o2 = torch.zeros(blocks * 512, device="cuda")
    CL.mfma(code, blocks, 1, o1, _sp())
    CL.mfma(code, blocks, 2, o2, _sp())
    torch.cuda.synchronize()
    assert float(o1.abs().sum()) > 0
    assert torch.equal(o2, 2 * o1)
