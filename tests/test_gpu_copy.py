"""GPU check of the library's streaming copy (rra_stream_copy), the yardstick
the fused kernels' bandwidth is compared with: every byte of the destination
range equals the source, and nothing outside the range is written, for sizes
from one vector to a ragged multi-workgroup tail."""
import pytest
import torch

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


@pytest.mark.parametrize("vpl", [1, 2, 4, 8])
@pytest.mark.parametrize("nbytes", [16, 4096, 4112, (1 << 20) + 48, 64 << 20])
def test_copy_exact_and_bounded(rra, nbytes, vpl):
    say(f"stream_copy nbytes={nbytes} vectors_per_lane={vpl}")
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    pad = 256
    big = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = big[pad:pad + nbytes]
    rra.stream_copy(src, dst, vpl)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((big[:pad] == 0xA5).all()) and bool((big[pad + nbytes:] == 0xA5).all())


def test_copy_rejects_bad_arguments(rra):
    a = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        rra.stream_copy(a, torch.zeros(32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(rra.RRAError):
        rra.stream_copy(a[:24], torch.zeros(24, dtype=torch.uint8, device="cuda"))
    with pytest.raises(rra.RRAError):
        rra.stream_copy(a[:32], a[16:48])  # overlapping ranges
    with pytest.raises(rra.RRAError):
        rra.stream_copy(a[:32], a[32:], 3)  # vectors per lane
