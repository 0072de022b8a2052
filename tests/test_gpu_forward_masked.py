"""uhla_forward_masked (neighbourhood radius, guide-locality modes) on the GPU vs the fp64
oracle, whose mask for these variants is pinned by enumeration in the oracle tests.

Tolerance as for uhla_forward: max-abs <= 2e-2 and mean-abs <= 2e-3 (bf16 inputs, fp64
oracle).
* every row at small sizes: both head dims, window sizes 8 / 16 / 32, ragged guide grids
  whose cell blocks are partly padding, guide grids reaching past the hi-res extent, a rho
  that does not divide the window size, no guide tokens;
* the default options reproduce uhla_forward bit for bit;
* closed-form probe Q = 0 at the 2K workload: every visible key has equal weight, so with
  V = [key is a guide token] each hi row returns its visible-guide fraction, counted here
  from the definition;
* sampled rows at the 8K workload;
* determinism.
"""
import ctypes

import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry, make_qkv_bits

from gpu_util import bf16_f64, config_inputs, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def run_masked(g, q, k, v):
    import torch
    o = api.forward(to_dev(q), to_dev(k), to_dev(v), g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                    theta=g.theta, radius=g.radius, guide_mode=g.guide_mode)
    torch.cuda.synchronize()
    return o


def oracle_rows(g, q, k, v, b, h, rows):
    qs = bf16_f64(q[b:b + 1, :, h:h + 1, :])
    ks = bf16_f64(k[b:b + 1, :, h:h + 1, :])
    vs = bf16_f64(v[b:b + 1, :, h:h + 1, :])
    return orc.attention_rows(qs, ks, vs, g, 0, 0, rows)


def check_close(got, want, what):
    err = np.abs(got - want)
    say(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS, (what, err.max())
    assert err.mean() <= MEAN_ABS, (what, err.mean())


BASE = {
    "d64_w8": Geometry(B=1, heads=2, head_dim=64, H=32, W=32, w=8, H_lr=8, W_lr=8),
    "d128_ragged_blocks": Geometry(B=2, heads=2, head_dim=128, H=48, W=32, w=16, H_lr=13,
                                   W_lr=9),
    "guide_beyond_grid": Geometry(B=1, heads=2, head_dim=64, H=16, W=16, w=8, H_lr=9, W_lr=7),
    "rho3": Geometry(B=1, heads=1, head_dim=128, H=48, W=48, w=16, H_lr=16, W_lr=16, rho=3),
    "w32": Geometry(B=1, heads=1, head_dim=128, H=64, W=96, w=32, H_lr=16, W_lr=24),
    "no_guide": Geometry(B=1, heads=2, head_dim=128, H=80, W=48, w=16, H_lr=0, W_lr=0),
}
CASES = [(n, r, m) for n in ("d64_w8",) for r in (0, 1, 2) for m in (0, 1, 2)] + [
    ("d128_ragged_blocks", 1, 1), ("d128_ragged_blocks", 1, 2), ("d128_ragged_blocks", 0, 2),
    ("guide_beyond_grid", 1, 1), ("guide_beyond_grid", 1, 2),
    ("rho3", 1, 1), ("rho3", 0, 2), ("rho3", 1, 2),
    ("w32", 0, 1), ("w32", 1, 2),
    ("no_guide", 2, 0), ("no_guide", 0, 1),
]


@pytest.mark.parametrize("name,radius,mode", CASES)
def test_masked_every_row(name, radius, mode):
    g = BASE[name].with_(radius=radius, guide_mode=mode)
    say(f"masked every row: {name} radius {radius} mode {mode}")
    q, k, v = make_qkv_bits(g, 4321)
    got = bf16_f64(from_dev(run_masked(g, q, k, v)))
    for b in range(g.B):
        for h in range(g.heads):
            want = oracle_rows(g, q, k, v, b, h, np.arange(g.L))
            check_close(got[b, :, h], want, f"{name} r{radius} m{mode} b{b} h{h}")


def test_default_options_are_uhla_forward():
    import torch
    g = Geometry(B=1, heads=3, head_dim=128, H=64, W=48, w=16, H_lr=16, W_lr=12)
    say("masked(1, 0) == forward")
    q, k, v = (to_dev(x) for x in make_qkv_bits(g, 99))
    a = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr)
    lib = api.load()
    out = torch.empty_like(q)
    ws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim,
                             radius=1, guide_mode=0)
    st = lib.uhla_forward_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), g.B,
                                 g.H, g.W, g.w, g.H_lr, g.W_lr, g.rho, g.heads, g.head_dim,
                                 0.0, g.theta, 1, 0, ws.data_ptr(), ws.numel(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))


def visible_guide_fraction(g):
    """Per hi row: (visible guide keys) / (visible keys), counted from the definition:
    guide cell (i, j) is visible to window (wy, wx) when its scaled position lies in the
    hi-res grid and in a window within reach (0 for mode 1, the radius for mode 2)."""
    nwy, nwx, w, r = g.H // g.w, g.W // g.w, g.w, g.radius
    reach = 0 if g.guide_mode == 1 else r
    s = np.arange(g.M)
    gy, gx = g.rho * (s // g.W_lr), g.rho * (s % g.W_lr)
    inside = (gy < g.H) & (gx < g.W)
    cwy, cwx = gy // w, gx // w
    frac = np.zeros((nwy, nwx))
    for wy in range(nwy):
        for wx in range(nwx):
            ny = min(nwy - 1, wy + r) - max(0, wy - r) + 1
            nx = min(nwx - 1, wx + r) - max(0, wx - r) + 1
            if g.guide_mode == 0:
                ng = g.M
            else:
                ng = int((inside & (np.abs(cwy - wy) <= reach) & (np.abs(cwx - wx) <= reach)).sum())
            frac[wy, wx] = ng / (ny * nx * w * w + ng)
    rr = np.arange(g.N)
    return frac[(rr // g.W) // w, (rr % g.W) // w]


@pytest.mark.parametrize("radius,mode", [(1, 1), (0, 1), (1, 2), (2, 2), (0, 0), (2, 0)])
def test_probe_uniform_weights_masked(radius, mode):
    import torch
    g = CONFIGS["2k"].with_(radius=radius, guide_mode=mode)
    say(f"masked probe Q=0 2k radius {radius} mode {mode}")
    shape = g.shape()
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    k = to_dev(config_inputs("2k")[2])
    v = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v[:, g.N:, :, 0] = 1.0
    o = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                    radius=radius, guide_mode=mode)
    got = o[0, :g.N, :, 0].float().cpu().numpy()
    want = visible_guide_fraction(g)
    err = np.abs(got - want[:, None]).max()
    say(f"  guide fraction max-abs {err:.2e}")
    assert err <= 4e-3  # bf16 output rounding (<= 2^-9 relative) plus fp32 sums


@pytest.mark.parametrize("radius,mode", [(1, 1), (1, 2)])
def test_masked_sampled_rows_8k(radius, mode):
    g0, q, k, v = config_inputs("8k")
    g = g0.with_(radius=radius, guide_mode=mode)
    say(f"masked sampled rows 8k radius {radius} mode {mode}")
    got = from_dev(run_masked(g, q, k, v))
    rng = np.random.default_rng(7)
    w, nwx = g.w, g.W // g.w
    for h in (0, 13, 23):
        corner = [0, g.W - 1, (g.H - 1) * g.W, g.N - 1, (w * 5 + 3) * g.W + w * (nwx // 2)]
        rows = np.unique(np.concatenate([corner, rng.integers(0, g.N, 250),
                                         g.N + rng.integers(0, g.M, 30)]))
        want = oracle_rows(g, q, k, v, 0, h, rows)
        check_close(bf16_f64(got[0, rows, h]), want, f"8k r{radius} m{mode} h{h}")


def test_masked_deterministic():
    g = CONFIGS["nonsquare"].with_(radius=1, guide_mode=2)
    say("masked determinism")
    _, q, k, v = config_inputs("nonsquare")
    a = from_dev(run_masked(g, q, k, v))
    b = from_dev(run_masked(g, q, k, v))
    assert np.array_equal(a, b)
