"""The measurement probes behind bench.py's measured ceilings, through the C
ABI: the copy probe copies every byte (sizes that leave its grid's last
block partly empty) and writes nothing past them, and the MFMA probe reports
the flops it issues and leaves finite sums (its operands are finite bf16
values)."""
import pytest
import torch

from mixture_experts_sparse_gate_amd import _lib, api

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


@pytest.mark.parametrize("n", [16, 4096 + 16, (1 << 20) + 48])
def test_copy_probe_copies_every_byte(n):
    g = torch.Generator(device="cpu").manual_seed(n)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda")
    api.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert not dst[n:].any(), "nothing written past the copy"


def test_mfma_probe_counts_its_flops():
    per_iter = 256 * 8 * 4 * 2 * 32 * 32 * 16  # blocks x waves x MFMAs x flops of one 32x32x16 MFMA
    for iters in (1, 7, 100):
        flops, sink = api.probe_mfma(iters)
        torch.cuda.synchronize()
        assert flops == per_iter * iters
        assert sink.numel() == int(_lib.load().moe_probe_mfma_sink_floats())
        assert torch.isfinite(sink).all()
        assert (sink != 0).any()
