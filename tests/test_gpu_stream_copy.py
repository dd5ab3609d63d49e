"""GPU test of sscnn_stream_copy, the streaming copy whose rate bench.py
reports as the device's practical HBM ceiling: an exact copy for counts with
and without a tail beyond the last whole 16-byte word, leaving the bytes
after the range untouched."""
import pytest
import torch

from spatially_sharded_cnn_amd import sscnn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("count", [1, 3, 4, 1023, 4096 * 257 + 5, (1 << 24) + 2])
def test_stream_copy_is_exact(count):
    print(f"  stream_copy count={count}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(count)
    src = torch.randn(count, device="cuda", generator=g)
    dst = torch.full((count + 8,), 7.0, device="cuda")
    sscnn.stream_copy(src, dst[:count])
    torch.cuda.synchronize()
    assert torch.equal(dst[:count], src)
    assert bool((dst[count:] == 7.0).all())
