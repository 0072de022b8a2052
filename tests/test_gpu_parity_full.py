"""Full-size parity gates that bite: checks at the 2K, non-square and 8K workloads whose
tolerance a mask or alignment error cannot hide.

* every row of one head at 2K, every row of the border windows (clipped neighbourhoods)
  of one head per batch at non-square, every row of three bands of windows and the guide
  rows of one head at 4K, and stratified rows of every head at 8K, against the fp64
  oracle at the stated tolerance (max-abs 2e-2, mean-abs 2e-3);
* a sharp gate: Q scaled by 4 (exact in bf16), so each row's softmax concentrates on a few
  keys and dropping or misplacing any visible window moves those rows' outputs by O(1)
  (the oracle pin test_sharp_gate_catches_a_dropped_neighbour measures that effect); the
  tolerance is relative to the output's own scale;
* the backward at 8K in the launch configuration bench.py --backward times: dK and dV of
  sampled hi-res keys (corner, edge and interior windows, window borders) against the
  oracle's row backward on two heads; dK and dV of sampled guide keys (each sums over
  every query row of its head) with dO zero except on about 1000 sampled query rows, so
  that the oracle needs only those rows; and the uniform-weight probe (Q = 0), whose dV has a closed form for every key (guide keys
  included) and whose dK is exactly zero.
"""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, make_qkv_bits

from gpu_util import bf16_f64, config_inputs, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
# sharp gate (Q x 4): relative to the oracle output's own scale
SHARP_MAX_REL, SHARP_MEAN_REL = 2e-2, 1e-2


def forward_dev(g, q, k, v):
    import torch
    o = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    torch.cuda.synchronize()
    return from_dev(o)


def oracle_head_rows(g, q, k, v, b, h, rows):
    sl = lambda x: bf16_f64(x[b:b + 1, :, h:h + 1, :])
    return orc.attention_rows(sl(q), sl(k), sl(v), g, 0, 0, rows)


def check(got, want, what):
    err = np.abs(got - want)
    say(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS, (what, err.max())
    assert err.mean() <= MEAN_ABS, (what, err.mean())


def check_sharp(got, want, what):
    err = np.abs(got - want)
    smax, smean = np.abs(want).max(), np.abs(want).mean()
    say(f"{what}: max-abs {err.max():.3e} (ref max {smax:.3e}) mean-abs {err.mean():.3e} "
        f"(ref mean {smean:.3e})")
    assert err.max() <= SHARP_MAX_REL * smax, (what, err.max(), smax)
    assert err.mean() <= SHARP_MEAN_REL * smean, (what, err.mean(), smean)


def test_forward_every_row_2k_one_head():
    g, q, k, v = config_inputs("2k")
    h = 11
    say(f"forward 2k: every row of head {h}")
    got = forward_dev(g, to_dev(q), to_dev(k), to_dev(v))
    want = oracle_head_rows(g, q, k, v, 0, h, np.arange(g.L))
    check(bf16_f64(got[0, :, h]), want, f"2k h{h} all {g.L} rows")


def border_window_rows(g):
    """Raster indices of every token in the windows of the first and last window rows and
    columns (corner and edge windows: clipped neighbourhoods)."""
    nwy, nwx = g.H // g.w, g.W // g.w
    rows = []
    for wy in range(nwy):
        for wx in range(nwx):
            if wy in (0, nwy - 1) or wx in (0, nwx - 1):
                iy, ix = np.divmod(np.arange(g.w * g.w), g.w)
                rows.append((wy * g.w + iy) * g.W + wx * g.w + ix)
    return np.sort(np.concatenate(rows))


def test_forward_border_windows_nonsquare():
    g, q, k, v = config_inputs("nonsquare")
    say("forward nonsquare: every row of the border windows, one head per batch")
    got = forward_dev(g, to_dev(q), to_dev(k), to_dev(v))
    rows = np.concatenate([border_window_rows(g), np.arange(g.N, g.L)])
    for b, h in ((0, 0), (1, 23)):
        want = oracle_head_rows(g, q, k, v, b, h, rows)
        check(bf16_f64(got[b, rows, h]), want, f"nonsquare b{b} h{h} ({len(rows)} rows)")


def window_band_rows(g, band_rows):
    """Raster indices of every token in the given window rows (all window columns)."""
    nwx = g.W // g.w
    rows = []
    for wy in band_rows:
        for wx in range(nwx):
            iy, ix = np.divmod(np.arange(g.w * g.w), g.w)
            rows.append((wy * g.w + iy) * g.W + wx * g.w + ix)
    return np.sort(np.concatenate(rows))


def test_forward_window_bands_4k():
    """Every row of the top, middle and bottom window rows (corner, edge and interior
    windows, 12 288 hi rows) and every guide row of one head at 4K."""
    g, q, k, v = config_inputs("4k")
    h = 17
    nwy = g.H // g.w
    say(f"forward 4k: every row of window rows 0, {nwy // 2}, {nwy - 1} and the guide rows, head {h}")
    got = forward_dev(g, to_dev(q), to_dev(k), to_dev(v))
    rows = np.concatenate([window_band_rows(g, (0, nwy // 2, nwy - 1)), np.arange(g.N, g.L)])
    want = oracle_head_rows(g, q, k, v, 0, h, rows)
    check(bf16_f64(got[0, rows, h]), want, f"4k h{h} ({len(rows)} rows)")


def test_forward_every_head_8k():
    """Stratified rows (corner, edge and interior windows, window borders, guide rows) of
    every one of the 24 heads at 8K."""
    from test_gpu_forward import stratified_rows
    g, q, k, v = config_inputs("8k")
    say("forward 8k: stratified rows of every head")
    got = forward_dev(g, to_dev(q), to_dev(k), to_dev(v))
    rng = np.random.default_rng(46)
    errs = []
    for h in range(g.heads):
        rows = stratified_rows(g, rng, 90, 20)
        want = oracle_head_rows(g, q, k, v, 0, h, rows)
        err = np.abs(bf16_f64(got[0, rows, h]) - want)
        errs.append((h, len(rows), err.max(), err.mean()))
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (h, err.max(), err.mean())
    say("8k every head: " + ", ".join(f"h{h} {n} rows max-abs {m:.2e}" for h, n, m, _ in errs[::6]))
    say(f"8k every head ({sum(e[1] for e in errs)} rows): max-abs {max(e[2] for e in errs):.3e} "
        f"mean-abs {np.mean([e[3] for e in errs]):.3e}")


def test_sharp_gate_2k_every_row():
    g, q, k, v = config_inputs("2k")
    h = 5
    say(f"sharp gate 2k (Q x 4): every row of head {h}")
    qt = to_dev(q) * 4  # exact in bf16
    got = forward_dev(g, qt, to_dev(k), to_dev(v))
    q4 = from_dev(qt)
    want = oracle_head_rows(g, q4, k, v, 0, h, np.arange(g.L))
    check_sharp(bf16_f64(got[0, :, h]), want, f"sharp 2k h{h}")


def test_sharp_gate_8k_sampled_rows():
    from test_gpu_forward import stratified_rows
    g, q, k, v = config_inputs("8k")
    say("sharp gate 8k (Q x 4): stratified rows of two heads")
    qt = to_dev(q) * 4
    got = forward_dev(g, qt, to_dev(k), to_dev(v))
    q4 = from_dev(qt)
    del qt
    rng = np.random.default_rng(44)
    for h in (3, 20):
        rows = stratified_rows(g, rng, 300, 60)
        want = oracle_head_rows(g, q4, k, v, 0, h, rows)
        check_sharp(bf16_f64(got[0, rows, h]), want, f"sharp 8k h{h} ({len(rows)} rows)")


def run_fwd_bwd(g, qt, kt, vt, gt):
    import torch
    o, lse = api.forward_lse(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
    dq, dk, dv = api.backward(qt, kt, vt, o, gt, lse, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                              theta=g.theta)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_rel(got, want, what):
    err = np.abs(got - want)
    scale_max, scale_mean = np.abs(want).max(), np.abs(want).mean()
    say(f"{what}: max-abs {err.max():.3e} (ref max {scale_max:.3e}) mean-abs {err.mean():.3e} "
        f"(ref mean {scale_mean:.3e})")
    assert err.max() <= 2e-2 * scale_max, what
    assert err.mean() <= 5e-3 * scale_mean, what


def hi_key_rows(g, windows):
    """Border tokens (corners and edge midpoints) and the centre token of each window."""
    w = g.w
    out = []
    for wy, wx in windows:
        for iy, ix in ((0, 0), (0, w - 1), (w - 1, 0), (w - 1, w - 1), (0, w // 2),
                       (w // 2, 0), (w - 1, w // 2), (w // 2, w - 1), (w // 2, w // 2)):
            out.append((wy * w + iy) * g.W + wx * w + ix)
    return np.array(sorted(out), dtype=np.int64)


def test_backward_8k_hi_key_rows():
    """dK and dV rows of hi-res keys at 8K against the oracle's row backward: keys of a
    corner, an edge and an interior window (each key's gradient sums over the 4, 6 or 9
    windows of queries that see it), on heads 0 and 23."""
    g, q, k, v = config_inputs("8k")
    say("backward 8k: sampled hi-key dK / dV rows")
    do = make_qkv_bits(g, 77)[0]
    _, dk, dv = (from_dev(x) for x in run_fwd_bwd(g, to_dev(q), to_dev(k), to_dev(v), to_dev(do)))
    nwy, nwx = g.H // g.w, g.W // g.w
    for h, wins in ((0, [(0, 0), (0, nwx // 2), (nwy // 2, nwx // 2)]),
                    (23, [(nwy - 1, nwx - 1), (nwy // 3, 0)])):
        k_rows = hi_key_rows(g, wins)
        sl = lambda x: bf16_f64(x[:, :, h:h + 1, :])
        _, rk, rv = orc.backward_rows(sl(q), sl(k), sl(v), sl(do), g, 0, 0, [], k_rows)
        check_rel(bf16_f64(dk[0, k_rows, h]), rk, f"8k dk h{h} ({len(k_rows)} hi keys)")
        check_rel(bf16_f64(dv[0, k_rows, h]), rv, f"8k dv h{h} ({len(k_rows)} hi keys)")


def test_backward_8k_sparse_cotangent():
    """dK and dV of guide keys (and of hi keys, and dQ) at 8K against the oracle.  A guide
    key's gradient sums over every query row of its head, so dO is zero except on about
    1000 stratified query rows (corner, edge and interior windows, window borders, random
    hi rows, guide rows); a row with dO = 0 contributes nothing, so the oracle needs only
    those rows' softmax, while the kernels still walk every query tile of the head."""
    from test_gpu_forward import stratified_rows
    g, q, k, v = config_inputs("8k")
    say("backward 8k: sparse cotangent, guide-key and hi-key dK / dV, dQ of live rows")
    rng = np.random.default_rng(79)
    live = stratified_rows(g, rng, 700, 300)
    do = np.zeros_like(q)
    do[:, live] = make_qkv_bits(g, 79)[0][:, live]
    dq, dk, dv = (from_dev(x) for x in run_fwd_bwd(g, to_dev(q), to_dev(k), to_dev(v), to_dev(do)))
    nwy, nwx = g.H // g.w, g.W // g.w
    M, W_lr = g.H_lr * g.W_lr, g.W_lr
    guide = np.array([0, W_lr - 1, M - W_lr, M - 1, (g.H_lr // 2) * W_lr + W_lr // 2]
                     + list(rng.integers(0, M, 11)))
    for h in (0, 23):
        g_rows = np.unique(g.N + guide)
        h_rows = hi_key_rows(g, [(0, 0), (nwy // 2, nwx // 2), (nwy - 1, nwx - 1)])
        k_rows = np.concatenate([h_rows, g_rows])
        q_rows = live[::8]
        sl = lambda x: bf16_f64(x[:, :, h:h + 1, :])
        rq, rk, rv = orc.backward_rows(sl(q), sl(k), sl(v), sl(do), g, 0, 0, q_rows, k_rows)
        nh = len(h_rows)
        check_rel(bf16_f64(dk[0, g_rows, h]), rk[nh:], f"8k dk h{h} ({len(g_rows)} guide keys)")
        check_rel(bf16_f64(dv[0, g_rows, h]), rv[nh:], f"8k dv h{h} ({len(g_rows)} guide keys)")
        check_rel(bf16_f64(dk[0, h_rows, h]), rk[:nh], f"8k dk h{h} ({nh} hi keys, sparse dO)")
        check_rel(bf16_f64(dv[0, h_rows, h]), rv[:nh], f"8k dv h{h} ({nh} hi keys, sparse dO)")
        check_rel(bf16_f64(dq[0, q_rows, h]), rq, f"8k dq h{h} ({len(q_rows)} live rows)")


def test_backward_8k_uniform_probe():
    """Q = 0 at 8K: every allowed pair has weight 1/c_i, so dV of every key (hi and guide)
    has the closed form of tests/probes.py, and dK is exactly zero."""
    import torch
    from probes import uniform_probe_dv
    g = CONFIGS["8k"]
    say("backward 8k: uniform-weight probe (Q = 0), dV of every key")
    _, _, k, v = config_inputs("8k")
    do = make_qkv_bits(g, 78)[0]
    qt = torch.zeros(g.shape(), dtype=torch.bfloat16, device="cuda")
    _, dk, dv = run_fwd_bwd(g, qt, to_dev(k), to_dev(v), to_dev(do))
    assert not torch.any(dk.view(torch.int16) & 0x7fff).item(), "dK must be exactly zero"
    dv_h = from_dev(dv)
    del dk, dv
    for h in range(0, g.heads, 4):
        want = uniform_probe_dv(g, bf16_f64(do[0, :, h]))
        got = bf16_f64(dv_h[0, :, h])
        check_rel(got[:g.N], want[:g.N], f"8k probe dv hi keys h{h}")
        check_rel(got[g.N:], want[g.N:], f"8k probe dv guide keys h{h}")
