"""uhla_forward_text (text tokens in the joint sequence text | hi | guide) on the GPU vs the
fp64 oracle, whose text extension is pinned by enumeration, pair counts, loop attention
and SDPA in the oracle tests.

Tolerance as for uhla_forward: max-abs <= 2e-2 and mean-abs <= 2e-3 (bf16 inputs, fp64
oracle).
* every row at small sizes: text lengths 1, 64, 77 and 300 (ragged key and query tiles),
  both head dims, guide modes 0/1/2, no guide tokens;
* T = 0 reproduces uhla_forward_masked bit for bit;
* closed-form probe Q = 0: every visible key has equal weight, so with V = [key is text]
  each row returns T / (number of keys it sees);
* sampled rows (all text rows among them) at the 2K and 8K workloads with 512 text tokens;
* determinism.
"""
import numpy as np
import pytest

import oracle.uhla_oracle as orc
from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry, make_qkv_bits

from gpu_util import bf16_f64, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def run_text(g, q, k, v):
    import torch
    o = api.forward(to_dev(q), to_dev(k), to_dev(v), g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                    theta=g.theta, radius=g.radius, guide_mode=g.guide_mode, T=g.T)
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


CASES = {
    "d64_T1": Geometry(B=1, heads=2, head_dim=64, H=32, W=32, w=8, H_lr=8, W_lr=8, T=1),
    "d128_T77_ragged": Geometry(B=2, heads=2, head_dim=128, H=48, W=32, w=16, H_lr=13, W_lr=9,
                                T=77),
    "d128_T64_mode1": Geometry(B=1, heads=2, head_dim=128, H=64, W=48, w=16, H_lr=16, W_lr=12,
                               T=64, guide_mode=1),
    "d64_T300_mode2_r2": Geometry(B=1, heads=1, head_dim=64, H=48, W=48, w=16, H_lr=12,
                                  W_lr=12, T=300, guide_mode=2, radius=2),
    "d128_T40_no_guide": Geometry(B=1, heads=2, head_dim=128, H=48, W=32, w=16, H_lr=0,
                                  W_lr=0, T=40),
    "d128_T5_rope_off": Geometry(B=1, heads=1, head_dim=128, H=32, W=32, w=16, H_lr=8, W_lr=8,
                                 T=5, theta=0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_text_every_row(name):
    g = CASES[name]
    say(f"text every row: {name} {g}")
    q, k, v = make_qkv_bits(g, 2468)
    got = bf16_f64(from_dev(run_text(g, q, k, v)))
    for b in range(g.B):
        for h in range(g.heads):
            want = oracle_rows(g, q, k, v, b, h, np.arange(g.L))
            check_close(got[b, :, h], want, f"{name} b{b} h{h}")


def test_text_zero_is_masked_forward():
    import torch
    g = Geometry(B=1, heads=2, head_dim=128, H=48, W=48, w=16, H_lr=12, W_lr=12, guide_mode=2)
    say("text T=0 == masked")
    q, k, v = (to_dev(x) for x in make_qkv_bits(g, 5))
    a = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, guide_mode=2)
    lib = api.load()
    out = torch.empty_like(q)
    ws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim, guide_mode=2)
    st = lib.uhla_forward_text(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), g.B, 0,
                               g.H, g.W, g.w, g.H_lr, g.W_lr, g.rho, g.heads, g.head_dim, 0.0,
                               g.theta, 1, 2, ws.data_ptr(), ws.numel(),
                               torch.cuda.current_stream().cuda_stream, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("mode", [0, 1])
def test_text_probe_uniform_weights(mode):
    """Q = 0: row i returns T / (keys row i sees) in the text-indicator column; the key
    counts come from the oracle's explicit mask (exact integers)."""
    import torch
    g = CONFIGS["2k"].with_(T=512, guide_mode=mode)
    say(f"text probe Q=0 2k T=512 mode {mode}")
    shape = g.shape()
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(shape, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    v = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v[:, :g.T, :, 0] = 1.0
    o = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                    guide_mode=mode, T=g.T)
    got = o[0, :, 0, 0].float().cpu().numpy()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(0, g.T, 7), g.T + rng.integers(0, g.N, 2000),
                                     g.T + g.N + rng.integers(0, g.M, 200)]))
    want = g.T / orc.allowed_key_count(g, rows)
    err = np.abs(got[rows] - want).max()
    say(f"  text fraction max-abs {err:.2e}")
    assert err <= 4e-3


@pytest.mark.parametrize("name,heads_checked,n_hi,n_lr", [("2k", (0, 23), 300, 60),
                                                         ("8k", (0, 11), 300, 60)])
def test_text_sampled_rows(name, heads_checked, n_hi, n_lr):
    g = CONFIGS[name].with_(T=512)
    say(f"text sampled rows {name} T=512")
    q, k, v = make_qkv_bits(g, 1357)
    got = from_dev(run_text(g, q, k, v))
    rng = np.random.default_rng(11)
    for h in heads_checked:
        rows = np.unique(np.concatenate([np.arange(g.T), g.T + rng.integers(0, g.N, n_hi),
                                         g.T + g.N + rng.integers(0, g.M, n_lr)]))
        want = oracle_rows(g, q, k, v, 0, h, rows)
        check_close(bf16_f64(got[0, rows, h]), want, f"{name} T=512 h{h} ({len(rows)} rows)")


def test_text_deterministic():
    g = CASES["d128_T77_ragged"]
    say("text determinism")
    q, k, v = make_qkv_bits(g, 9)
    assert np.array_equal(from_dev(run_text(g, q, k, v)), from_dev(run_text(g, q, k, v)))
