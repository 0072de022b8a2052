"""The measurement copy of uhla_copy_probe is bit-exact through each load path (plain,
nontemporal, direct-to-LDS), including a copy of a single 16 KiB block and one that spans
many workgroups with a tail of odd-looking data."""
import numpy as np
import pytest

from global_attention_image_amd import api

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("nbytes", [16384, 16384 * 1237])
def test_copy_probe_bit_exact(mode, nbytes):
    import torch
    say(f"copy probe mode {mode}, {nbytes} bytes")
    rng = np.random.default_rng(mode * 7 + nbytes % 97)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    dst = torch.full((nbytes + 16384,), 0xA5, dtype=torch.uint8, device="cuda")
    api.copy_probe(src, dst[:nbytes], mode)
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    assert np.array_equal(out[:nbytes], host)
    assert np.all(out[nbytes:] == 0xA5)  # nothing written past the end
