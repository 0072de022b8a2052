"""uhla_forward_noalloc (the forward on the library's static scratch, for callers that
cannot allocate) against uhla_forward: bit-identical outputs on two calls in a row, the
second on a smaller problem, and the size limit rejected before any device work."""
import ctypes

import numpy as np
import pytest

from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, Geometry, make_qkv_bits

from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def test_noalloc_matches_forward_twice_second_smaller():
    import torch
    cases = (Geometry(B=1, heads=8, head_dim=128, H=64, W=64, w=16, H_lr=16, W_lr=16),
             CONFIGS["tiny"])
    for g, seed in zip(cases, (501, 502)):
        need = api.forward_workspace_bytes(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim)
        say(f"noalloc vs forward: {g} (workspace {need} bytes)")
        assert need <= 64 << 20
        q, k, v = (to_dev(x) for x in make_qkv_bits(g, seed))
        ref = api.forward(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta)
        out = torch.full_like(q, float("nan"))
        api.forward_noalloc(q, k, v, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                            out=out)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), ref.view(torch.int16))
        say(f"  bit-identical: {same}")
        assert same


def test_noalloc_rejects_problems_above_its_scratch():
    lib = api.load()
    P = [ctypes.c_void_p(0x10000000 * i) for i in range(1, 5)]
    g = CONFIGS["2k"]  # ~214 MB of scratch
    st = lib.uhla_forward_noalloc(*P, g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.rho, g.heads,
                                  g.head_dim, 0.0, 10000.0, ctypes.c_void_p(0))
    assert st == api.UHLA_ERR_WORKSPACE
    assert b"static scratch" in lib.uhla_last_error_detail()
