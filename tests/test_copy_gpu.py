"""The library's streaming copy (kda_stream_copy), the benchmark's measured
HBM reference: an exact copy for sizes that do and do not fill whole
workgroup tiles, and nothing written past the end."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


@pytest.mark.parametrize("n16", [1, 255, 1024, 4096 + 3, (64 << 20) // 16 + 17])
def test_stream_copy_exact(kda, n16):
    gen = torch.Generator(device="cpu").manual_seed(3000 + n16 % 1000)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), dtype=torch.int32, generator=gen).to(DEV)
    dst = torch.full((4 * n16 + 64,), 7, dtype=torch.int32, device=DEV)
    kda.stream_copy(src, dst[:4 * n16])
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n16], src)
    assert torch.all(dst[4 * n16:] == 7)
