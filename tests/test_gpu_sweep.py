"""A seeded sweep of small random geometries through the forward and the backward, every
row against the fp64 oracle.  It crosses the options the other tests take one or two at a
time: window size 8 or 16, one to three windows per axis, rho 2 to 4, guide grids from
none to past the hi grid, radius 0 to 2, guide modes 0 to 2, text tokens, RoPE on or off,
head dims 64 and 128, one or two batches and heads.

Tolerances as elsewhere: outputs and LSE max-abs <= 2e-2, mean-abs <= 2e-3; gradients
max-abs <= 2e-2 x max |ref|, mean-abs <= 5e-3 x mean |ref|.
"""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import Geometry, make_qkv_bits

from gpu_util import bf16_f64, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def sweep_geometries(n: int = 24, seed: int = 2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        w = int(rng.choice([8, 16]))
        H, W = w * int(rng.integers(1, 4)), w * int(rng.integers(1, 4))
        rho = int(rng.integers(2, 5))
        if rng.random() < 0.2:
            H_lr = W_lr = 0
        else:  # up to two guide rows / columns past the hi grid
            H_lr = int(rng.integers(1, H // rho + 3))
            W_lr = int(rng.integers(1, W // rho + 3))
        out.append(Geometry(
            B=int(rng.integers(1, 3)), heads=int(rng.integers(1, 3)),
            head_dim=int(rng.choice([64, 128])), H=H, W=W, w=w, H_lr=H_lr, W_lr=W_lr, rho=rho,
            theta=float(rng.choice([10000.0, 10000.0, 0.0])), name=f"sweep{i}",
            radius=int(rng.integers(0, 3)), guide_mode=int(rng.integers(0, 3)),
            T=int(rng.choice([0, int(rng.integers(1, 90))]))))
    return out


GEOMS = sweep_geometries()


def check_rel(got, want, what):
    err = np.abs(got - want)
    assert err.max() <= 2e-2 * np.abs(want).max(), (what, err.max())
    assert err.mean() <= 5e-3 * np.abs(want).mean(), (what, err.mean())


@pytest.mark.parametrize("g", GEOMS, ids=[g.name for g in GEOMS])
def test_sweep_forward_backward(g):
    import torch
    say(f"sweep: {g}")
    q, k, v = make_qkv_bits(g, 700 + int(g.name[5:]))
    do = make_qkv_bits(g, 800 + int(g.name[5:]))[0]
    qt, kt, vt, gt = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    kw = dict(rho=g.rho, theta=g.theta, radius=g.radius, guide_mode=g.guide_mode, T=g.T)
    o, lse = api.forward_lse(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, **kw)
    dq, dk, dv = api.backward(qt, kt, vt, o, gt, lse, g.H, g.W, g.w, g.H_lr, g.W_lr, **kw)
    torch.cuda.synchronize()
    qf, kf, vf, gf = (bf16_f64(x) for x in (q, k, v, do))
    want_o = orc.forward(qf, kf, vf, g)
    err = np.abs(bf16_f64(from_dev(o)) - want_o)
    say(f"  out: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    lse_h = lse.cpu().numpy().astype(np.float64)
    rq, rk, rv = orc.backward(qf, kf, vf, gf, g)
    for b in range(g.B):
        for h in range(g.heads):
            e = np.abs(lse_h[b, h] - orc.lse_rows(qf, kf, g, b, h, np.arange(g.L)))
            assert e.max() <= 2e-2 and e.mean() <= 2e-3, ("lse", b, h)
            check_rel(bf16_f64(from_dev(dq)[b, :, h]), rq[b, :, h], f"dq b{b} h{h}")
            check_rel(bf16_f64(from_dev(dk)[b, :, h]), rk[b, :, h], f"dk b{b} h{h}")
            check_rel(bf16_f64(from_dev(dv)[b, :, h]), rv[b, :, h], f"dv b{b} h{h}")
    say("  gradients and lse within tolerance")
