"""Window-first permutation on the GPU vs the oracle's index map: bit-exact.

Full-size tensors at all five workloads (bf16), fp32 rows, batch strides into a joint
[hi | guide] tensor, ragged row widths that force the 4- and 2-byte copy paths, and the
round trip unpermute(permute(x)) = x on the device."""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS

from gpu_util import say

pytestmark = pytest.mark.gpu


def random_bits(shape, dtype, seed):
    # arbitrary bit patterns (NaNs included): the copy must not care
    rng = np.random.default_rng(seed)
    info = np.iinfo(dtype)
    return rng.integers(info.min, info.max, size=shape, dtype=dtype, endpoint=True)


def to_dev_raw(x):
    import torch
    return torch.from_numpy(x).cuda()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_permute_bf16_full_size(name):
    import torch
    g = CONFIGS[name]
    say(f"permute bf16 {name} {g.B}x{g.N}x{g.heads}x{g.head_dim}")
    x = random_bits((g.B, g.N, g.heads, g.head_dim), np.int16, 100 + len(name))
    src = to_dev_raw(x).view(torch.bfloat16)
    dst = torch.empty_like(src)
    api.window_permute(src, dst, g.H, g.W, g.w)
    back = torch.empty_like(src)
    api.window_unpermute(dst, back, g.H, g.W, g.w)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy()
    expect = orc.window_permute(x, g.H, g.W, g.w)
    assert np.array_equal(got, expect)
    del got, expect
    assert torch.equal(back.view(torch.int16), src.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "2k", "nonsquare", "4k"])
def test_permute_fp32(name):
    import torch
    g = CONFIGS[name]
    say(f"permute fp32 {name}")
    x = random_bits((g.B, g.N, g.heads, g.head_dim), np.int32, 7)
    src = to_dev_raw(x).view(torch.float32)
    dst = torch.empty_like(src)
    api.window_permute(src, dst, g.H, g.W, g.w)
    got = dst.view(torch.int32).cpu().numpy()
    assert np.array_equal(got, orc.window_permute(x, g.H, g.W, g.w))
    back = torch.empty_like(src)
    api.window_unpermute(dst, back, g.H, g.W, g.w)
    assert torch.equal(back.view(torch.int32), src.view(torch.int32))


@pytest.mark.parametrize("name", ["tiny", "nonsquare"])
def test_permute_hi_segment_of_joint_tensor(name):
    """Permute the hi rows of [B, N + M, ...] into [B, N, ...] and back into a fresh
    joint buffer: the guide rows of the destination are left untouched."""
    import torch
    g = CONFIGS[name]
    say(f"permute joint {name}")
    x = random_bits((g.B, g.L, g.heads, g.head_dim), np.int16, 3)
    src = to_dev_raw(x).view(torch.bfloat16)
    mid = torch.empty((g.B, g.N, g.heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
    api.window_permute(src, mid, g.H, g.W, g.w, src_tokens_per_batch=g.L,
                       dst_tokens_per_batch=g.N)
    assert np.array_equal(mid.view(torch.int16).cpu().numpy(),
                          orc.window_permute(x[:, :g.N], g.H, g.W, g.w))
    sentinel = random_bits((g.B, g.L, g.heads, g.head_dim), np.int16, 4)
    out = to_dev_raw(sentinel).view(torch.bfloat16)
    api.window_unpermute(mid, out, g.H, g.W, g.w, src_tokens_per_batch=g.N,
                         dst_tokens_per_batch=g.L)
    got = out.view(torch.int16).cpu().numpy()
    assert np.array_equal(got[:, :g.N], x[:, :g.N])
    assert np.array_equal(got[:, g.N:], sentinel[:, g.N:])


@pytest.mark.parametrize("B,H,W,w,heads,d,dtype", [
    (2, 12, 20, 4, 3, 5, np.int16),    # row 30 B: 2-byte path
    (1, 6, 9, 3, 1, 6, np.int16),      # row 12 B: 4-byte path
    (3, 16, 8, 8, 1, 3, np.int32),     # row 12 B fp32: 4-byte path
    (1, 7, 5, 1, 2, 8, np.int16),      # w = 1: identity
    (1, 32, 32, 32, 4, 64, np.int16),  # one window: identity
    (1, 1024, 16, 16, 1, 8, np.int16), # tall grid, one window column
])
def test_permute_ragged_shapes(B, H, W, w, heads, d, dtype):
    import torch
    say(f"permute ragged {B},{H},{W},{w},{heads},{d},{dtype.__name__}")
    x = random_bits((B, H * W, heads, d), dtype, 11)
    tdt = torch.bfloat16 if dtype == np.int16 else torch.float32
    src = to_dev_raw(x).view(tdt)
    dst = torch.empty_like(src)
    api.window_permute(src, dst, H, W, w)
    got = dst.view(torch.int16 if dtype == np.int16 else torch.int32).cpu().numpy()
    assert np.array_equal(got, orc.window_permute(x, H, W, w))
    back = torch.empty_like(src)
    api.window_unpermute(dst, back, H, W, w)
    assert torch.equal(back, src) or np.array_equal(
        back.view(torch.int16 if dtype == np.int16 else torch.int32).cpu().numpy(), x)
