"""uhla_forward_permute_free (no K/V prep pass: tiles copied from the raster K and V, K
rotated at load, V read transposed from LDS) on the GPU vs the fp64 oracle.

Same bar as uhla_forward (max-abs <= 2e-2, mean-abs <= 2e-3 against the oracle from the
bf16 inputs): every row at small sizes over several tiles, with ragged guide tails (the
last guide tile partial), both head dims, windows of 16, 32, 64 and 128 (tiles of 4, 2, 1
window rows and pieces of a row), guide grids past the hi-res extent, no guide tokens, RoPE
off (the default mask only); stratified
sampled rows at 2K and 8K; the Q = K = 4X identity probe (each row returns its own V row:
the raster gather puts every key where the mask expects it); agreement with uhla_forward;
the window sizes it rejects.
"""
import numpy as np
import pytest

from global_attention_image_amd import api
from global_attention_image_amd.inputs import Geometry, make_qkv_bits

from gpu_util import bf16_f64, config_inputs, from_dev, say, to_dev
from test_gpu_forward import check_close, oracle_rows, stratified_rows

pytestmark = pytest.mark.gpu


def run(g, q, k, v, permute_free=True):
    import torch
    o = api.forward(to_dev(q), to_dev(k), to_dev(v), g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                    theta=g.theta, permute_free=permute_free)
    torch.cuda.synchronize()
    return o


CASES = {
    "d128_multi_tile_ragged_guide": Geometry(B=2, heads=3, head_dim=128, H=48, W=32, w=16,
                                             H_lr=13, W_lr=9),
    "d64_w16": Geometry(B=1, heads=2, head_dim=64, H=64, W=48, w=16, H_lr=16, W_lr=12),
    "guide_beyond_grid": Geometry(B=1, heads=2, head_dim=128, H=32, W=32, w=16, H_lr=11,
                                  W_lr=9),
    "w32": Geometry(B=1, heads=1, head_dim=128, H=64, W=96, w=32, H_lr=16, W_lr=24),
    "w64_d64": Geometry(B=1, heads=1, head_dim=64, H=128, W=64, w=64, H_lr=5, W_lr=3),
    "w128": Geometry(B=1, heads=1, head_dim=128, H=128, W=128, w=128, H_lr=9, W_lr=7),
    "no_guide": Geometry(B=1, heads=2, head_dim=128, H=48, W=48, w=16, H_lr=0, W_lr=0),
    "rope_off": Geometry(B=1, heads=2, head_dim=64, H=32, W=48, w=16, H_lr=8, W_lr=12,
                         theta=0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_permute_free_every_row(name):
    g = CASES[name]
    say(f"permute-free every row: {name} {g}")
    q, k, v = make_qkv_bits(g, 4321)
    got = bf16_f64(from_dev(run(g, q, k, v)))
    for b in range(g.B):
        for h in range(g.heads):
            check_close(got[b, :, h], oracle_rows(g, q, k, v, b, h, np.arange(g.L)),
                        f"{name} b{b} h{h}")


@pytest.mark.parametrize("name,heads_checked,n_hi,n_lr", [
    ("2k", (0, 23), 300, 80),
    ("8k", (0, 13, 23), 500, 100),
])
def test_permute_free_sampled_rows_full_size(name, heads_checked, n_hi, n_lr):
    g, q, k, v = config_inputs(name)
    say(f"permute-free sampled rows {name}")
    got = from_dev(run(g, q, k, v))
    rng = np.random.default_rng(9)
    for h in heads_checked:
        rows = stratified_rows(g, rng, n_hi, n_lr)
        check_close(bf16_f64(got[0, rows, h]), oracle_rows(g, q, k, v, 0, h, rows),
                    f"{name} h{h} ({len(rows)} rows)")


def test_permute_free_matches_forward():
    g, q, k, v = config_inputs("2k")
    say("permute-free vs uhla_forward, 2k")
    a = run(g, q, k, v, permute_free=True).float()
    b = run(g, q, k, v, permute_free=False).float()
    d = (a - b).abs()
    say(f"  max {d.max().item():.3e} mean {d.mean().item():.3e}")
    assert d.max().item() <= 1e-2 and d.mean().item() <= 1e-4


def test_permute_free_identity_probe():
    import torch
    g, x, _, v = config_inputs("nonsquare")
    say("permute-free probe Q=K=4X nonsquare")
    xt = to_dev(x) * 4
    vt = to_dev(v)
    o = api.forward(xt, xt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                    permute_free=True)
    torch.cuda.synchronize()
    frac = (o.view(torch.int16) == vt.view(torch.int16)).float().mean().item()
    assert frac == 1.0, frac


@pytest.mark.parametrize("w,H,W", [(8, 16, 16), (48, 96, 96)])
def test_permute_free_rejects_window_sizes(w, H, W):
    g = Geometry(B=1, heads=1, head_dim=64, H=H, W=W, w=w, H_lr=4, W_lr=4)
    q, k, v = make_qkv_bits(g, 1)
    with pytest.raises(api.UhlaError) as e:
        run(g, q, k, v)
    assert e.value.status == api.UHLA_ERR_UNSUPPORTED
