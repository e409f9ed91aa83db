"""The streaming copy helper (carve_stream_copy), the bandwidth probe behind the measured
roofline denominator, copies exactly (needs an MI355X): sizes below one tile, a ragged tail
and many grid-stride rounds."""
import pytest
import torch

from chunk_gated_delta_amd import carve

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 1023, 1024 * 5 + 7, (64 << 20) // 16 + 3])
def test_stream_copy_exact(n16):
    print(f"\n[case] stream copy of {n16} 16-byte vectors", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4 + 8,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.full_like(src, 7)
    carve.stream_copy(dst[:n16 * 4], src[:n16 * 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n16 * 4], src[:n16 * 4])
    assert torch.all(dst[n16 * 4:] == 7)          # nothing past the end is written
