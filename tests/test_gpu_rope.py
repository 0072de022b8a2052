"""Standalone RoPE on the GPU vs the fp64 oracle: within 1 bf16 ulp of the correctly
rounded oracle value (the kernel rotates in fp64 and rounds once, so nearly all elements
are bit-identical to the oracle's correctly rounded value); guide rows bit-identical to hi-res rows at (rho*i, rho*j);
window-first order consistent with the permutation; theta <= 0 copies."""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry

from gpu_util import (bf16_f64, config_inputs, f64_to_bf16_rne, from_dev, say, to_dev,
                      ulp_distance)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": CONFIGS["tiny"],
    "nonsquare_small": Geometry(B=2, heads=3, head_dim=128, H=48, W=32, w=16, H_lr=12, W_lr=8),
    "guide_beyond_grid": Geometry(B=1, heads=2, head_dim=64, H=16, W=16, w=8, H_lr=9, W_lr=7),
    "no_guide": Geometry(B=1, heads=2, head_dim=64, H=16, W=24, w=8, H_lr=0, W_lr=0),
}


def oracle_rope_bits(x_bits, g):
    return f64_to_bf16_rne(orc.rope_joint(bf16_f64(x_bits), g))


@pytest.mark.parametrize("name", list(CASES))
def test_rope_vs_oracle(name):
    g = CASES[name]
    say(f"rope {name}")
    x = config_inputs("tiny")[1] if name == "tiny" else \
        np.random.default_rng(5).standard_normal(g.shape()).astype(np.float32).view(np.uint32)
    if name != "tiny":
        x = (x >> 16).astype(np.uint16)
    src = to_dev(x)
    dst = src.clone()
    api.rope_apply(src, dst, g.H, g.W, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    got = from_dev(dst)
    want = oracle_rope_bits(x, g)
    d = ulp_distance(got, want)
    assert d.max() <= 1, d.max()
    # fp64 rotation with one rounding: only near-ties may differ from the oracle's rounding
    assert (d == 0).mean() > 0.9999, (d == 0).mean()


@pytest.mark.parametrize("name", ["2k", "nonsquare", "4k", "8k"])
def test_rope_full_size(name):
    g, q, _, _ = config_inputs(name)
    say(f"rope full {name}")
    src = to_dev(q)
    api.rope_apply(src, src, g.H, g.W, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)  # in place
    got = from_dev(src)
    del src
    # the oracle in head chunks to bound host memory
    same = 0
    for h in range(0, g.heads, 4):
        sub = g.with_(heads=min(4, g.heads - h))
        want = oracle_rope_bits(q[:, :, h:h + 4], sub)
        d = ulp_distance(got[:, :, h:h + 4], want)
        assert d.max() <= 1, (h, d.max())
        same += int((d == 0).sum())
    frac = same / got.size
    say(f"rope full {name}: {got.size} elements within 1 ulp, {frac:.6f} bit-identical")
    assert frac > 0.9999


def test_guide_rows_bit_identical_to_scaled_hi_rows():
    g = Geometry(B=1, heads=2, head_dim=128, H=64, W=48, w=16, H_lr=16, W_lr=12)
    say("rope guide/hi identity")
    x = np.random.default_rng(9).standard_normal(g.shape()).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    hi_idx = [(g.rho * (s // g.W_lr)) * g.W + g.rho * (s % g.W_lr) for s in range(g.M)]
    bits[:, g.N:] = bits[:, hi_idx]
    t = to_dev(bits)
    api.rope_apply(t, t, g.H, g.W, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    got = from_dev(t)
    assert np.array_equal(got[:, g.N:], got[:, hi_idx])


def test_window_first_order_matches_permuted_raster():
    import torch
    g = Geometry(B=2, heads=3, head_dim=64, H=32, W=48, w=16, H_lr=8, W_lr=12)
    say("rope window-first order")
    x = np.random.default_rng(2).standard_normal(g.shape()).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    raster = to_dev(bits)
    api.rope_apply(raster, raster, g.H, g.W, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    wf = to_dev(bits)
    tmp = torch.empty((g.B, g.N, g.heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
    api.window_permute(wf, tmp, g.H, g.W, g.w, src_tokens_per_batch=g.L, dst_tokens_per_batch=g.N)
    wf[:, :g.N] = tmp
    api.rope_apply(wf, wf, g.H, g.W, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta, w=g.w, hi_order=1)
    got_wf = from_dev(wf)
    got_raster = from_dev(raster)
    assert np.array_equal(got_wf[:, :g.N], orc.window_permute(got_raster[:, :g.N], g.H, g.W, g.w))
    assert np.array_equal(got_wf[:, g.N:], got_raster[:, g.N:])


def test_theta_zero_copies():
    g = CONFIGS["tiny"]
    _, q, _, _ = config_inputs("tiny")
    src = to_dev(q)
    dst = to_dev(np.zeros_like(q))
    api.rope_apply(src, dst, g.H, g.W, g.H_lr, g.W_lr, theta=0.0)
    assert np.array_equal(from_dev(dst), q)
