"""GPU checks of the kernel's building blocks through the C ABI."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_chunks,offset", [(1, 0), (64, 0), (1000, 16), (4096, 80 * 1024), (3 * 1024, 96 * 1024)])
def test_lds_dma_roundtrip(n_chunks, offset):
    """16-byte chunks copied global -> LDS (at any offset of the 160 KB) -> global arrive unchanged."""
    from persistent_megakernel_loop_amd.binding import selftest_lds_dma

    print(f"[case] lds dma n={n_chunks} offset={offset}", flush=True)
    src = torch.randint(-2**31, 2**31 - 1, (n_chunks * 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    selftest_lds_dma(src, dst, offset)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
