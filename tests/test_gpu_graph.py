"""The forward and backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Both paths enqueue only kernel launches on the caller's stream (no allocation, no memset,
no synchronisation), so they can be captured.  The graph is replayed several times with
eager work and synchronisations between the replays (the outputs are cleared eagerly), and
every replay must reproduce the eager results bit for bit.
"""
import pytest

from global_attention_image_amd import api
from global_attention_image_amd.inputs import CONFIGS, make_qkv_bits

from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,mode", [("2k", 0, 0), ("tiny", 40, 1)])
def test_forward_backward_graph_replays(name, T, mode):
    import torch
    g = CONFIGS[name].with_(T=T, guide_mode=mode)
    say(f"graph capture and replay: {name} T={T} guide_mode={mode}")
    q, k, v = make_qkv_bits(g, 5)
    do = make_qkv_bits(g, 6)[0]
    qt, kt, vt, gt = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    dev = qt.device
    fws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim, dev,
                              rho=g.rho, radius=g.radius, guide_mode=mode, T=T)
    nb = api.backward_workspace_bytes(g.B, T, g.H, g.W, g.w, g.H_lr, g.W_lr, g.rho, g.heads,
                                      g.head_dim, g.radius, mode)
    bws = torch.empty(nb, dtype=torch.uint8, device=dev)
    out, lse = torch.empty_like(qt), torch.empty((g.B, g.heads, g.L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(qt), torch.empty_like(qt)

    def step():
        api.forward_lse(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho, theta=g.theta,
                        radius=g.radius, guide_mode=mode, T=T, out=out, lse=lse, workspace=fws)
        api.backward(qt, kt, vt, out, gt, lse, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                     theta=g.theta, radius=g.radius, T=T, guide_mode=mode, dq=dq, dk=dk, dv=dv,
                     workspace=bws)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (out, lse, dq, dk, dv):
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name_x, x, r in zip(("o", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            same = torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                               r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16))
            assert same, (rep, name_x)
    say("  3 replays bit-identical to the eager results")
    del graph
