"""uhla_forward_lse and uhla_backward on the GPU vs the fp64 oracle (gradients pinned
against torch autograd and finite differences in the oracle tests).

Tolerances.  LSE: max-abs <= 2e-2, mean-abs <= 2e-3 (natural-log units, from bf16 inputs).
Gradients are compared relative to the oracle gradient's own scale: max-abs error <= 2e-2
x max |ref| and mean-abs error <= 5e-3 x mean |ref|.  The kernels round Q (rotated and
scaled), P and dS to bf16 for the MFMAs (relative 2^-9 each) and store bf16 (2^-9), and the
sums they enter have random signs, so the errors stay a small multiple of 2^-9 of the
gradient's scale.
* every row / every key at small sizes: both head dims, window sizes 8, 16 and 32, radius
  0 / 1 / 2, ragged guide grids, guide positions past the hi grid, no guide tokens, RoPE off,
  text tokens (ragged, several tiles, without guide tokens), guide modes 1 and 2 (rho not
  dividing w, guide cells past the hi grid, radius 2, windows of 8, with text);
* sampled query and key rows at the 2K workload, without and with 512 text tokens and in
  guide modes 1 and 2 (oracle rows of the backward);
* the 8K workload: sampled dQ rows against the oracle and the dV sum rule over all keys;
* determinism.
"""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry, make_qkv_bits

from gpu_util import bf16_f64, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def run_fwd_bwd(g, q, k, v, do):
    import torch
    qt, kt, vt, gt = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = api.forward_lse(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                             radius=g.radius, guide_mode=g.guide_mode, T=g.T)
    dq, dk, dv = api.backward(qt, kt, vt, o, gt, lse, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                              theta=g.theta, radius=g.radius, T=g.T, guide_mode=g.guide_mode)
    torch.cuda.synchronize()
    return lse.cpu().numpy().astype(np.float64), from_dev(dq), from_dev(dk), from_dev(dv)


def check_rel(got, want, what):
    err = np.abs(got - want)
    scale_max, scale_mean = np.abs(want).max(), np.abs(want).mean()
    say(f"{what}: max-abs {err.max():.3e} (ref max {scale_max:.3e}) mean-abs {err.mean():.3e} "
        f"(ref mean {scale_mean:.3e})")
    assert err.max() <= 2e-2 * scale_max, what
    assert err.mean() <= 5e-3 * scale_mean, what


CASES = {
    "d64_w8_r1": Geometry(B=1, heads=2, head_dim=64, H=32, W=32, w=8, H_lr=8, W_lr=8),
    "d128_w16_ragged": Geometry(B=2, heads=2, head_dim=128, H=48, W=32, w=16, H_lr=13, W_lr=9),
    "d128_r0": Geometry(B=1, heads=1, head_dim=128, H=48, W=48, w=16, H_lr=12, W_lr=12, radius=0),
    "d64_r2": Geometry(B=1, heads=2, head_dim=64, H=80, W=48, w=16, H_lr=20, W_lr=12, radius=2),
    "d128_no_guide": Geometry(B=1, heads=2, head_dim=128, H=48, W=48, w=16, H_lr=0, W_lr=0),
    "d128_rope_off": Geometry(B=1, heads=1, head_dim=128, H=32, W=48, w=16, H_lr=8, W_lr=12,
                              theta=0.0),
    "d128_w32": Geometry(B=1, heads=1, head_dim=128, H=64, W=96, w=32, H_lr=16, W_lr=24),
    # guide positions (4i, 4j) up to (40, 32) lie past the 32x32 hi grid: RoPE factors beyond
    # the cos/sin table are evaluated directly
    "d64_guide_beyond_grid": Geometry(B=2, heads=1, head_dim=64, H=32, W=32, w=16, H_lr=11,
                                      W_lr=9),
    # text tokens (rows 0..T-1): a ragged text tile, several text tiles with radius 0, text
    # without guide tokens and with windows of 8
    "d128_text77": Geometry(B=1, heads=2, head_dim=128, H=48, W=32, w=16, H_lr=12, W_lr=8,
                            T=77),
    "d128_text300_r0": Geometry(B=1, heads=1, head_dim=128, H=32, W=48, w=16, H_lr=8, W_lr=12,
                                radius=0, T=300),
    "d64_text_w8_no_guide": Geometry(B=2, heads=1, head_dim=64, H=32, W=32, w=8, H_lr=0, W_lr=0,
                                     T=64),
    # guide modes 1 / 2 (a hi query sees the guide cells of its window / neighbourhood):
    # rho not dividing w, guide cells past the hi grid, radius 2, windows of 8, text
    "d128_mode1": Geometry(B=1, heads=2, head_dim=128, H=48, W=64, w=16, H_lr=12, W_lr=16,
                           guide_mode=1),
    "d64_mode2_rho3": Geometry(B=1, heads=1, head_dim=64, H=48, W=48, w=16, H_lr=14, W_lr=13,
                               rho=3, guide_mode=2),
    "d128_mode2_r2_beyond_grid": Geometry(B=1, heads=1, head_dim=128, H=32, W=64, w=16, H_lr=11,
                                          W_lr=20, radius=2, guide_mode=2),
    "d64_mode1_w8_text": Geometry(B=1, heads=2, head_dim=64, H=32, W=32, w=8, H_lr=8, W_lr=8,
                                  guide_mode=1, T=40),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_every_row(name):
    g = CASES[name]
    say(f"backward every row: {name} {g}")
    q, k, v = make_qkv_bits(g, 111)
    do = make_qkv_bits(g, 112)[0]
    lse, dq, dk, dv = run_fwd_bwd(g, q, k, v, do)
    rq, rk, rv = orc.backward(bf16_f64(q), bf16_f64(k), bf16_f64(v), bf16_f64(do), g)
    for b in range(g.B):
        for h in range(g.heads):
            want_lse = orc.lse_rows(bf16_f64(q), bf16_f64(k), g, b, h, np.arange(g.L))
            err = np.abs(lse[b, h] - want_lse)
            say(f"  lse b{b} h{h}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
            assert err.max() <= 2e-2 and err.mean() <= 2e-3
            check_rel(bf16_f64(dq[b, :, h]), rq[b, :, h], f"{name} dq b{b} h{h}")
            check_rel(bf16_f64(dk[b, :, h]), rk[b, :, h], f"{name} dk b{b} h{h}")
            check_rel(bf16_f64(dv[b, :, h]), rv[b, :, h], f"{name} dv b{b} h{h}")


def test_backward_sampled_rows_2k():
    g = CONFIGS["2k"]
    say("backward sampled rows 2k")
    q, k, v = make_qkv_bits(g, 1)
    do = make_qkv_bits(g, 2)[0]
    _, dq, dk, dv = run_fwd_bwd(g, q, k, v, do)
    rng = np.random.default_rng(5)
    qf, kf, vf, gf = (bf16_f64(x) for x in (q, k, v, do))
    for h in (0, 17):
        q_rows = np.unique(np.concatenate([[0, g.W - 1, g.N - 1, g.N, g.L - 1],
                                           rng.integers(0, g.L, 120)]))
        k_rows = np.unique(np.concatenate([[0, g.N - 1, g.N, g.L - 1], rng.integers(0, g.N, 60),
                                           g.N + rng.integers(0, g.M, 4)]))
        rq, rk, rv = orc.backward_rows(qf, kf, vf, gf, g, 0, h, q_rows, k_rows)
        check_rel(bf16_f64(dq[0, q_rows, h]), rq, f"2k dq h{h}")
        check_rel(bf16_f64(dk[0, k_rows, h]), rk, f"2k dk h{h}")
        check_rel(bf16_f64(dv[0, k_rows, h]), rv, f"2k dv h{h}")


def test_backward_sampled_rows_2k_text():
    g = CONFIGS["2k"].with_(T=512)
    say("backward sampled rows 2k with 512 text tokens")
    q, k, v = make_qkv_bits(g, 11)
    do = make_qkv_bits(g, 12)[0]
    _, dq, dk, dv = run_fwd_bwd(g, q, k, v, do)
    rng = np.random.default_rng(6)
    qf, kf, vf, gf = (bf16_f64(x[:, :, 5:6, :]) for x in (q, k, v, do))
    T, N = g.T, g.N
    q_rows = np.unique(np.concatenate([[0, T - 1, T, T + N - 1, T + N, g.L - 1],
                                       rng.integers(0, T, 10), T + rng.integers(0, N, 40),
                                       T + N + rng.integers(0, g.M, 10)]))
    k_rows = np.unique(np.concatenate([[0, T - 1, T, T + N, g.L - 1], rng.integers(0, T, 6),
                                       T + rng.integers(0, N, 20)]))
    rq, rk, rv = orc.backward_rows(qf, kf, vf, gf, g, 0, 0, q_rows, k_rows)
    check_rel(bf16_f64(dq[0, q_rows, 5]), rq, "2k+text dq h5")
    check_rel(bf16_f64(dk[0, k_rows, 5]), rk, "2k+text dk h5")
    check_rel(bf16_f64(dv[0, k_rows, 5]), rv, "2k+text dv h5")


@pytest.mark.parametrize("mode", [1, 2])
def test_backward_sampled_rows_2k_guide_modes(mode):
    g = CONFIGS["2k"].with_(guide_mode=mode)
    say(f"backward sampled rows 2k, guide mode {mode}")
    q, k, v = make_qkv_bits(g, 21 + mode)
    do = make_qkv_bits(g, 31 + mode)[0]
    _, dq, dk, dv = run_fwd_bwd(g, q, k, v, do)
    rng = np.random.default_rng(mode)
    h = 3 * mode
    qf, kf, vf, gf = (bf16_f64(x[:, :, h:h + 1, :]) for x in (q, k, v, do))
    q_rows = np.unique(np.concatenate([[0, g.N - 1, g.N, g.L - 1], rng.integers(0, g.N, 40),
                                       g.N + rng.integers(0, g.M, 10)]))
    k_rows = np.unique(np.concatenate([[0, g.N, g.L - 1, g.N + 33], rng.integers(0, g.N, 10),
                                       g.N + rng.integers(0, g.M, 12)]))
    rq, rk, rv = orc.backward_rows(qf, kf, vf, gf, g, 0, 0, q_rows, k_rows)
    check_rel(bf16_f64(dq[0, q_rows, h]), rq, f"2k mode {mode} dq h{h}")
    check_rel(bf16_f64(dk[0, k_rows, h]), rk, f"2k mode {mode} dk h{h}")
    check_rel(bf16_f64(dv[0, k_rows, h]), rv, f"2k mode {mode} dv h{h}")


def test_backward_8k_sampled_dq_and_dv_sum():
    """The 8K workload in the launch configuration bench.py --backward times: dQ of sampled
    rows (corner / edge / interior windows, guide rows) against the oracle's rows, and the
    sum rule at full size: every row of P sums to 1, so the sum of dV over all keys equals
    the sum of dO over all queries (per batch, head and dim; bf16 storage of 278 528 dV rows
    and fp32 accumulation keep the difference far below 1e-3 of the sum of |dO|)."""
    from gpu_util import config_inputs
    from test_gpu_forward import stratified_rows
    g, q, k, v = config_inputs("8k")
    say("backward 8k: sampled dQ rows, dV sum rule")
    do = make_qkv_bits(g, 77)[0]
    _, dq, _, dv = run_fwd_bwd(g, q, k, v, do)
    rng = np.random.default_rng(8)
    for h in (0, 23):
        qf, kf, vf, gf = (bf16_f64(x[:, :, h:h + 1, :]) for x in (q, k, v, do))
        rows = stratified_rows(g, rng, 45, 8)
        rq, _, _ = orc.backward_rows(qf, kf, vf, gf, g, 0, 0, rows, [])
        check_rel(bf16_f64(dq[0, rows, h]), rq, f"8k dq h{h} ({len(rows)} rows)")
    for h in range(g.heads):
        sum_dv = bf16_f64(dv[:, :, h, :]).sum(axis=1)   # [B, D]
        gh = bf16_f64(do[:, :, h, :])
        err = np.abs(sum_dv - gh.sum(axis=1)) / np.abs(gh).sum(axis=1)
        assert err.max() <= 1e-3, (h, err.max())
    say(f"8k dV sum rule holds for all {g.heads} heads (last max relative difference {err.max():.3e})")


def test_backward_deterministic():
    g = CASES["d128_w16_ragged"]
    say("backward determinism")
    q, k, v = make_qkv_bits(g, 3)
    do = make_qkv_bits(g, 4)[0]
    a = run_fwd_bwd(g, q, k, v, do)
    b = run_fwd_bwd(g, q, k, v, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
