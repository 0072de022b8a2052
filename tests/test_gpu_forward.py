"""uhla_forward on the GPU vs the fp64 oracle.

Tolerance (from bf16 inputs, fp64 oracle): max-abs <= 2e-2 and mean-abs <= 2e-3.
* every row at small sizes that span several tiles, ragged guide tails, both head dims,
  window sizes 8 / 16 / 32, no guide tokens, one window, guide grids beyond the hi-res
  extent, RoPE off, a custom scale;
* stratified sampled rows at the 2K, 4K, non-square and 8K workloads, in the launch
  configuration the benchmark times;
* closed-form probes at full size, which catch mask / alignment errors that the
  tolerance alone could hide: Q = 0 (uniform weights -> neighbourhood centroid and guide
  fraction), Q = K = 4X (each row returns its own V row, bit-exact), V = 1;
* determinism and the timed entry point.
"""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry, make_qkv_bits

from gpu_util import bf16_f64, config_inputs, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def run_forward(g, q, k, v, scale=0.0):
    import torch
    qt, kt, vt = to_dev(q), to_dev(k), to_dev(v)
    o = api.forward(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, scale=scale,
                    theta=g.theta)
    torch.cuda.synchronize()
    return o


def oracle_rows(g, q, k, v, b, h, rows, scale=None):
    """Oracle output rows of (b, h), from that head's bf16 inputs widened to fp64."""
    qs = bf16_f64(q[b:b + 1, :, h:h + 1, :])
    ks = bf16_f64(k[b:b + 1, :, h:h + 1, :])
    vs = bf16_f64(v[b:b + 1, :, h:h + 1, :])
    gg = g
    if scale is not None:
        qs = qs * (scale / g.scale)  # oracle applies 1/sqrt(d); fold a custom scale into Q
    return orc.attention_rows(qs, ks, vs, gg, 0, 0, rows)


def check_close(got, want, what):
    err = np.abs(got - want)
    say(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS, (what, err.max())
    assert err.mean() <= MEAN_ABS, (what, err.mean())


FULL_ROW_CASES = {
    "tiny": CONFIGS["tiny"],
    "d128_multi_tile_ragged_guide": Geometry(B=2, heads=3, head_dim=128, H=48, W=32, w=16,
                                             H_lr=13, W_lr=9),
    "d64_w16": Geometry(B=1, heads=2, head_dim=64, H=64, W=48, w=16, H_lr=16, W_lr=12),
    "d128_w8_guide_below_one_tile": Geometry(B=1, heads=2, head_dim=128, H=40, W=24, w=8,
                                             H_lr=10, W_lr=6),
    "no_guide": Geometry(B=1, heads=2, head_dim=128, H=48, W=48, w=16, H_lr=0, W_lr=0),
    "one_window": Geometry(B=1, heads=2, head_dim=128, H=16, W=16, w=16, H_lr=4, W_lr=4),
    "guide_beyond_grid": Geometry(B=1, heads=2, head_dim=64, H=16, W=16, w=8, H_lr=9, W_lr=7),
    "w32": Geometry(B=1, heads=1, head_dim=128, H=64, W=96, w=32, H_lr=16, W_lr=24),
    "rope_off": Geometry(B=1, heads=2, head_dim=64, H=32, W=48, w=16, H_lr=8, W_lr=12,
                         theta=0.0),
    "tall_single_column": Geometry(B=1, heads=1, head_dim=128, H=160, W=16, w=16, H_lr=40,
                                   W_lr=4),
}


@pytest.mark.parametrize("name", list(FULL_ROW_CASES))
def test_forward_every_row(name):
    g = FULL_ROW_CASES[name]
    say(f"forward every row: {name} {g}")
    q, k, v = config_inputs("tiny")[1:] if name == "tiny" else make_qkv_bits(g, 1234)
    o = from_dev(run_forward(g, q, k, v))
    got = bf16_f64(o)
    for b in range(g.B):
        for h in range(g.heads):
            want = oracle_rows(g, q, k, v, b, h, np.arange(g.L))
            check_close(got[b, :, h], want, f"{name} b{b} h{h}")


def test_forward_custom_scale():
    g = Geometry(B=1, heads=2, head_dim=128, H=32, W=32, w=16, H_lr=8, W_lr=8)
    say("forward custom scale")
    q, k, v = make_qkv_bits(g, 77)
    sc = 0.05
    got = bf16_f64(from_dev(run_forward(g, q, k, v, scale=sc)))
    for h in range(g.heads):
        check_close(got[0, :, h], oracle_rows(g, q, k, v, 0, h, np.arange(g.L), scale=sc),
                    f"scale h{h}")


def stratified_rows(g, rng, n_hi, n_lr):
    """Hi rows from corner, edge and interior windows and window-border tokens; guide rows."""
    nwy, nwx, w = g.H // g.w, g.W // g.w, g.w
    picks = []
    wins = [(0, 0), (0, nwx - 1), (nwy - 1, 0), (nwy - 1, nwx - 1),
            (0, nwx // 2), (nwy // 2, 0), (nwy - 1, nwx // 2), (nwy // 2, nwx - 1),
            (nwy // 2, nwx // 2)]
    for (wy, wx) in wins:
        for (iy, ix) in [(0, 0), (0, w - 1), (w - 1, 0), (w - 1, w - 1), (w // 2, w // 2)]:
            picks.append((wy * w + iy) * g.W + wx * w + ix)
    extra = max(0, n_hi - len(picks))
    picks += list(rng.integers(0, g.N, extra))
    lr = [g.N, g.L - 1] + list(g.N + rng.integers(0, g.M, max(0, n_lr - 2)))
    return np.unique(np.array(picks + lr, dtype=np.int64))


@pytest.mark.parametrize("name,g", [
    # 256 queries of a workgroup span 4 window rows: their Q RoPE factors (4 rows + 64
    # columns) are staged in LDS
    ("w64_factors_in_lds", Geometry(B=1, heads=1, head_dim=128, H=64, W=128, w=64, H_lr=16,
                                    W_lr=32)),
    # 2 rows + 128 columns of factors exceed the stage buffer: the lanes read the fp64 table
    ("w128_factors_from_table", Geometry(B=1, heads=1, head_dim=128, H=128, W=128, w=128,
                                         H_lr=32, W_lr=32)),
])
def test_forward_wide_windows_sampled_rows(name, g):
    say(f"forward wide windows, sampled rows: {name} {g}")
    q, k, v = make_qkv_bits(g, 4321)
    got = bf16_f64(from_dev(run_forward(g, q, k, v)))
    rows = stratified_rows(g, np.random.default_rng(5), 300, 40)
    check_close(got[0, rows, 0], oracle_rows(g, q, k, v, 0, 0, rows), name)


@pytest.mark.parametrize("name,heads_checked,n_hi,n_lr", [
    ("2k", (0, 11, 23), 400, 100),
    ("nonsquare", (0, 23), 300, 60),
    ("4k", (0, 12, 23), 400, 100),
    ("8k", (0, 5, 11, 17, 23), 700, 120),
])
def test_forward_sampled_rows_full_size(name, heads_checked, n_hi, n_lr):
    g, q, k, v = config_inputs(name)
    say(f"forward sampled rows {name}")
    got = from_dev(run_forward(g, q, k, v))
    rng = np.random.default_rng(42)
    for b in range(g.B):
        for h in heads_checked:
            rows = stratified_rows(g, rng, n_hi, n_lr)
            want = oracle_rows(g, q, k, v, b, h, rows)
            check_close(bf16_f64(got[b, rows, h]), want, f"{name} b{b} h{h} ({len(rows)} rows)")


def neighbour_centroid(g):
    """Closed form for the Q = 0 probe: per hi row (wy_mean, wx_mean, guide fraction)."""
    nwy, nwx = g.H // g.w, g.W // g.w
    wy = np.arange(nwy)
    wx = np.arange(nwx)
    # clipped 3-neighbourhoods per axis: count and sum of indices
    cy = np.array([len([a for a in (i - 1, i, i + 1) if 0 <= a < nwy]) for i in wy])
    sy = np.array([sum(a for a in (i - 1, i, i + 1) if 0 <= a < nwy) for i in wy])
    cx = np.array([len([a for a in (i - 1, i, i + 1) if 0 <= a < nwx]) for i in wx])
    sx = np.array([sum(a for a in (i - 1, i, i + 1) if 0 <= a < nwx) for i in wx])
    ww = g.w * g.w
    tot = cy[:, None] * cx[None, :] * ww + g.M                       # [nwy, nwx]
    ey = sy[:, None] * cx[None, :] * ww / tot
    ex = cy[:, None] * sx[None, :] * ww / tot
    ef = g.M / tot
    r = np.arange(g.N)
    ry, rx = (r // g.W) // g.w, (r % g.W) // g.w
    return ey[ry, rx], ex[ry, rx], ef[ry, rx]


@pytest.mark.parametrize("name", ["nonsquare", "8k"])
def test_probe_uniform_weights(name):
    """Q = 0: every allowed key has weight 1/count; V encodes window row/col and guide-ness."""
    import torch
    g = CONFIGS[name]
    say(f"probe Q=0 {name}")
    shape = g.shape()
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    k = to_dev(config_inputs(name)[2]) if name != "8k" else \
        torch.randn(shape, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    v = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    r = torch.arange(g.N, device="cuda")
    v[:, :g.N, :, 0] = ((r // g.W) // g.w).to(torch.bfloat16)[None, :, None]
    v[:, :g.N, :, 1] = ((r % g.W) // g.w).to(torch.bfloat16)[None, :, None]
    v[:, g.N:, :, 2] = 1.0
    o = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ey, ex, ef = neighbour_centroid(g)
    for col, e in ((0, ey), (1, ex), (2, ef)):
        err = np.abs(got[:, :g.N, :, col] - e[None, :, None])
        assert err.max() <= np.abs(e).max() * 2.0 ** -8 + 1e-6, (col, err.max())
    assert np.all(got[:, g.N:, :, 2] == 1.0)
    assert np.all(got[:, g.N:, :, :2] == 0.0)
    assert np.all(got[:, :, :, 3:] == 0.0)


@pytest.mark.parametrize("name", ["tiny", "nonsquare", "8k"])
def test_probe_identity(name):
    """Q = K = 4X: the self logit dominates by > 100 in log2 units, so O = V bit-exactly."""
    import torch
    g, x, _, v = config_inputs(name)
    say(f"probe Q=K=4X {name}")
    xt = to_dev(x) * 4  # exact in bf16
    vt = to_dev(v)
    o = api.forward(xt, xt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    torch.cuda.synchronize()
    same = (o.view(torch.int16) == vt.view(torch.int16))
    frac = same.float().mean().item()
    assert frac == 1.0, frac


def test_probe_constant_value():
    import torch
    g, q, k, _ = config_inputs("nonsquare")
    say("probe V=1")
    v = torch.ones(g.shape(), dtype=torch.bfloat16, device="cuda")
    o = api.forward(to_dev(q), to_dev(k), v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                    theta=g.theta)
    torch.cuda.synchronize()
    assert (o.float() - 1.0).abs().max().item() <= 2.0 ** -8


def test_deterministic_and_timed_matches():
    import torch
    g, q, k, v = config_inputs("2k")
    say("determinism 2k")
    qt, kt, vt = to_dev(q), to_dev(k), to_dev(v)
    ws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim)
    o1 = api.forward(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, workspace=ws)
    o2 = api.forward(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, workspace=ws)
    timer = api.Timer(4)
    o3 = api.forward(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, workspace=ws, timer=timer)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    ms, calls = timer.read()
    assert calls == 1 and ms["attn_hi"] > 0 and ms["prep_hi"] > 0
    timer.close()
