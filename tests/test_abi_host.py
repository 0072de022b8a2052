"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before anything reaches a GPU.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

from global_attention_image_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uhla.h")

# Fake, 256-byte aligned device addresses: every call below must fail validation on the
# host before these are ever dereferenced or handed to HIP.
P = ctypes.c_void_p(0x10000000)
P2 = ctypes.c_void_p(0x20000000)
P3 = ctypes.c_void_p(0x30000000)
P4 = ctypes.c_void_p(0x40000000)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uhla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return api.load()


def test_header_declares_the_contract_entry_points():
    names = declared_functions()
    for n in ("uhla_window_permute", "uhla_window_unpermute", "uhla_rope_apply", "uhla_forward",
              "uhla_forward_workspace_bytes", "uhla_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (uhla_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    # the binding covers the same set
    assert set(api.EXPORTS) == set(names)


def test_strerror(lib):
    assert lib.uhla_strerror(0) == b"UHLA_OK"
    for s in (1, 2, 3, 4):
        assert lib.uhla_strerror(s).startswith(b"UHLA_ERR_")
    assert lib.uhla_strerror(99) == b"unknown uhla status"


def permute_args(**kw):
    a = dict(src=P, dst=P2, B=1, H=32, W=32, w=8, heads=2, d=64, e=2, stpb=1024, dtpb=1024)
    a.update(kw)
    return (a["src"], a["dst"], a["B"], a["H"], a["W"], a["w"], a["heads"], a["d"], a["e"],
            a["stpb"], a["dtpb"], NULL)


@pytest.mark.parametrize("fn", ["uhla_window_permute", "uhla_window_unpermute"])
@pytest.mark.parametrize("kw,status", [
    (dict(src=NULL), api.UHLA_ERR_ARG),
    (dict(dst=NULL), api.UHLA_ERR_ARG),
    (dict(B=0), api.UHLA_ERR_ARG),
    (dict(w=0), api.UHLA_ERR_ARG),
    (dict(w=5), api.UHLA_ERR_ARG),
    (dict(H=30), api.UHLA_ERR_ARG),
    (dict(heads=0), api.UHLA_ERR_ARG),
    (dict(stpb=1000), api.UHLA_ERR_ARG),
    (dict(dtpb=10), api.UHLA_ERR_ARG),
    (dict(e=8), api.UHLA_ERR_UNSUPPORTED),
    (dict(e=1), api.UHLA_ERR_UNSUPPORTED),
    (dict(dst=ctypes.c_void_p(0x10000000 + 4096)), api.UHLA_ERR_ARG),  # overlap
    (dict(src=ctypes.c_void_p(0x10000001)), api.UHLA_ERR_ARG),  # misaligned
])
def test_permute_rejects(lib, fn, kw, status):
    assert getattr(lib, fn)(*permute_args(**kw)) == status
    assert lib.uhla_last_error_detail() != b""


def rope_args(**kw):
    a = dict(src=P, dst=P2, B=1, H=32, W=32, w=8, order=0, H_lr=8, W_lr=8, rho=4, heads=2, d=64,
             theta=10000.0)
    a.update(kw)
    return (a["src"], a["dst"], a["B"], a["H"], a["W"], a["w"], a["order"], a["H_lr"],
            a["W_lr"], a["rho"], a["heads"], a["d"], a["theta"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(src=NULL), api.UHLA_ERR_ARG),
    (dict(B=0), api.UHLA_ERR_ARG),
    (dict(order=2), api.UHLA_ERR_ARG),
    (dict(order=1, w=5), api.UHLA_ERR_ARG),
    (dict(H_lr=0), api.UHLA_ERR_ARG),
    (dict(rho=0), api.UHLA_ERR_ARG),
    (dict(d=60), api.UHLA_ERR_UNSUPPORTED),
    (dict(dst=ctypes.c_void_p(0x10000000 + 64)), api.UHLA_ERR_ARG),  # partial overlap
    (dict(src=ctypes.c_void_p(0x10000008)), api.UHLA_ERR_ARG),  # misaligned
])
def test_rope_rejects(lib, kw, status):
    assert lib.uhla_rope_apply(*rope_args(**kw)) == status


def fwd_args(**kw):
    a = dict(q=P, k=P2, v=P3, o=P4, B=1, H=32, W=32, w=8, H_lr=8, W_lr=8, rho=4, heads=2, d=64,
             scale=0.0, theta=10000.0, ws=ctypes.c_void_p(0x50000000), wsb=1 << 40)
    a.update(kw)
    return (a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["W"], a["w"], a["H_lr"],
            a["W_lr"], a["rho"], a["heads"], a["d"], a["scale"], a["theta"], a["ws"], a["wsb"],
            NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), api.UHLA_ERR_ARG),
    (dict(o=NULL), api.UHLA_ERR_ARG),
    (dict(B=0), api.UHLA_ERR_ARG),
    (dict(heads=0), api.UHLA_ERR_ARG),
    (dict(w=12), api.UHLA_ERR_ARG),
    (dict(W_lr=0), api.UHLA_ERR_ARG),
    (dict(rho=0), api.UHLA_ERR_ARG),
    (dict(d=96), api.UHLA_ERR_UNSUPPORTED),
    (dict(d=32), api.UHLA_ERR_UNSUPPORTED),
    (dict(H=24, W=24, w=24), api.UHLA_ERR_UNSUPPORTED),
    (dict(H=36, W=36, w=4), api.UHLA_ERR_UNSUPPORTED),
    # 3x3 windows of 96x96 tokens: 9 * 144 key tiles per window, above the 1024-tile table
    (dict(H=384, W=384, w=96, H_lr=0, W_lr=0), api.UHLA_ERR_UNSUPPORTED),
    (dict(B=65536), api.UHLA_ERR_UNSUPPORTED),  # grid dimension limits
    (dict(heads=65536), api.UHLA_ERR_UNSUPPORTED),
    # one head of a 4096 x 8192 grid at head_dim 128: 8 GiB of K (or V) rows per (batch,
    # head), past the kernels' 32-bit tile byte offsets
    (dict(heads=1, H=4096, W=8192, w=16, H_lr=0, W_lr=0, d=128), api.UHLA_ERR_UNSUPPORTED),
    # the same for the guide rows: 2^25 guide tokens of head_dim 128
    (dict(heads=1, H=64, W=64, w=16, H_lr=4096, W_lr=8192, d=128), api.UHLA_ERR_UNSUPPORTED),
    # exactly 4 GiB per (batch, head) region is still addressable: it passes validation
    # and stops at the (too small) workspace
    (dict(heads=1, H=4096, W=4096, w=16, H_lr=0, W_lr=0, d=128, wsb=1000),
     api.UHLA_ERR_WORKSPACE),
    (dict(ws=NULL), api.UHLA_ERR_WORKSPACE),
    (dict(wsb=1000), api.UHLA_ERR_WORKSPACE),
    (dict(o=P), api.UHLA_ERR_ARG),  # aliases q
    (dict(o=ctypes.c_void_p(0x30000000 + 4096)), api.UHLA_ERR_ARG),  # overlaps v
    (dict(ws=ctypes.c_void_p(0x50000010)), api.UHLA_ERR_ARG),  # misaligned workspace
    (dict(ws=P2), api.UHLA_ERR_ARG),  # workspace overlaps k
    (dict(ws=ctypes.c_void_p(0x10000000 + 4096)), api.UHLA_ERR_ARG),  # workspace inside q
])
def test_forward_rejects(lib, kw, status):
    assert lib.uhla_forward(*fwd_args(**kw)) == status


def test_forward_timed_rejects_null_timer(lib):
    assert lib.uhla_forward_timed(*fwd_args(), NULL) == api.UHLA_ERR_ARG
    a = fwd_args()
    assert lib.uhla_forward_masked_timed(*a[:15], 1, 1, *a[15:], NULL) == api.UHLA_ERR_ARG


def test_timer_create_rejects_bad_count(lib):
    h = ctypes.c_void_p()
    assert lib.uhla_timer_create(0, ctypes.byref(h)) == api.UHLA_ERR_ARG


@pytest.mark.parametrize("radius,mode,kw,status", [
    (-1, 0, {}, api.UHLA_ERR_ARG),
    (1, 3, {}, api.UHLA_ERR_ARG),
    (1, -1, {}, api.UHLA_ERR_ARG),
    (1, 1, dict(q=NULL), api.UHLA_ERR_ARG),
    (1, 2, dict(d=96), api.UHLA_ERR_UNSUPPORTED),
    (1, 1, dict(wsb=1000), api.UHLA_ERR_WORKSPACE),
    # radius 4 on a 16x16-window grid: 9x9 windows of 4 tiles = 324 tiles, fine; with 64x64
    # windows (64 tiles each) the 3x3 neighbourhood is 576 and radius 2 is 1600 > 1024
    (2, 0, dict(H=320, W=320, w=64, H_lr=0, W_lr=0), api.UHLA_ERR_UNSUPPORTED),
])
def test_forward_masked_rejects(lib, radius, mode, kw, status):
    a = fwd_args(**kw)
    assert lib.uhla_forward_masked(*a[:15], radius, mode, *a[15:]) == status


def expected_workspace(B, H, W, w, H_lr, W_lr, heads, d, guide_mode=0):
    """Independent restatement of the workspace layout (regions 256-byte aligned): cos/sin
    table, K/V hi rows, K/V guide rows (64-padded), and for guide modes 1 and 2 a copy of
    the guide K/V in 8x8 cell blocks and prepared Q rows (otherwise Q is rotated as the
    attention kernel loads it)."""
    al = lambda x: (x + 255) // 256 * 256
    N, M = H * W, H_lr * W_lr
    Mk = (M + 63) // 64 * 64
    Mb = ((H_lr + 7) // 8) * ((W_lr + 7) // 8) * 64 if (guide_mode and M) else 0
    e, bh = 2, B * heads
    parts = [16 * max(H, W) * (d // 4), bh * N * d * e, bh * N * d * e,
             bh * Mk * d * e, bh * Mk * d * e, bh * Mb * d * e, bh * Mb * d * e]
    if guide_mode and M:  # prepared Q rows (hi, guide) for the guide-locality masks
        parts += [bh * N * d * e, bh * M * d * e]
    return sum(al(p) for p in parts)


GEOMS = [(1, 32, 32, 8, 8, 8, 2, 64), (1, 128, 128, 16, 32, 32, 24, 128),
         (2, 256, 128, 16, 64, 32, 24, 128), (1, 512, 512, 16, 128, 128, 24, 128),
         (1, 48, 16, 16, 5, 3, 3, 128), (1, 16, 16, 16, 0, 0, 1, 64)]


@pytest.mark.parametrize("g", GEOMS)
def test_workspace_bytes(lib, g):
    assert lib.uhla_forward_workspace_bytes(*g) == expected_workspace(*g)


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_masked_workspace_bytes(lib, g, mode):
    B, H, W, w, H_lr, W_lr, heads, d = g
    got = lib.uhla_forward_masked_workspace_bytes(B, H, W, w, H_lr, W_lr, 4, heads, d, 2, mode)
    assert got == expected_workspace(*g, guide_mode=mode)
    if mode == 0:
        assert got == lib.uhla_forward_workspace_bytes(*g)


def expected_text_extra(B, T, H, W, w, H_lr, W_lr, heads, d, guide_mode):
    """Extra workspace bytes with T text tokens: text rows appended to the global-key
    buffers (and to the cell-block buffers) and the split partial results
    (splits = min(ceil(1024 / query blocks), max(1, key tiles // 8)))."""
    al = lambda x: (x + 255) // 256 * 256
    N, M = H * W, H_lr * W_lr
    Mk, Tk, Tq = (M + 63) // 64 * 64, (T + 63) // 64 * 64, (T + 255) // 256 * 256
    Mb = ((H_lr + 7) // 8) * ((W_lr + 7) // 8) * 64 if (guide_mode and M) else 0
    e, bh = 2, B * heads
    qblocks = bh * (Tq // 256)
    splits = min(-(-1024 // qblocks), max(1, (N + Mk + Tk) // 64 // 8)) if T else 0
    grown = [(bh * (Mk + Tk) * d * e, bh * Mk * d * e)] * 2 + \
        [(bh * (Mb + (Tk if Mb else 0)) * d * e, bh * Mb * d * e)] * 2
    extra = sum(al(a) - al(b) for a, b in grown)
    return extra + al(splits * bh * Tq * d * 4) + al(splits * bh * Tq * 8)


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("T,mode", [(0, 0), (1, 0), (77, 1), (512, 2)])
def test_text_workspace_bytes(lib, g, T, mode):
    B, H, W, w, H_lr, W_lr, heads, d = g
    got = lib.uhla_forward_text_workspace_bytes(B, T, H, W, w, H_lr, W_lr, 4, heads, d, 1, mode)
    assert got == expected_workspace(*g, guide_mode=mode) + \
        expected_text_extra(B, T, H, W, w, H_lr, W_lr, heads, d, mode)


def test_forward_text_rejects(lib):
    a = fwd_args()
    f = lib.uhla_forward_text
    assert f(*a[:5], -1, *a[5:15], 1, 0, *a[15:], NULL) == api.UHLA_ERR_ARG
    assert f(*a[:5], 1 << 25, *a[5:15], 1, 0, *a[15:], NULL) == api.UHLA_ERR_UNSUPPORTED
    assert f(*a[:5], 8, *a[5:15], 1, 5, *a[15:], NULL) == api.UHLA_ERR_ARG
    assert lib.uhla_forward_text_workspace_bytes(1, -1, 32, 32, 8, 8, 8, 4, 2, 64, 1, 0) == 0


def test_masked_workspace_bytes_invalid(lib):
    f = lib.uhla_forward_masked_workspace_bytes
    assert f(1, 32, 32, 8, 8, 8, 4, 2, 64, -1, 0) == 0
    assert f(1, 32, 32, 8, 8, 8, 4, 2, 64, 1, 3) == 0
    assert f(1, 32, 32, 8, 8, 8, 0, 2, 64, 1, 1) == 0


def test_workspace_bytes_invalid(lib):
    assert lib.uhla_forward_workspace_bytes(1, 30, 32, 8, 8, 8, 2, 64) == 0
    assert lib.uhla_forward_workspace_bytes(1, 32, 32, 8, 8, 0, 2, 64) == 0
    assert lib.uhla_forward_workspace_bytes(1, 32, 32, 8, 8, 8, 2, 96) == 0


def lse_args(lse=ctypes.c_void_p(0x60000000), **kw):
    a = fwd_args(**kw)
    # uhla_forward_lse(q, k, v, o, lse, B, T, H, W, w, H_lr, W_lr, rho, heads, d, scale, theta,
    #                  radius, guide_mode, ws, bytes, stream)
    return (*a[:4], lse, a[4], 0, *a[5:15], 1, 0, *a[15:])


def test_forward_lse_rejects(lib):
    f = lib.uhla_forward_lse
    assert f(*lse_args(lse=NULL)) == api.UHLA_ERR_ARG
    assert f(*lse_args(lse=ctypes.c_void_p(0x60000002))) == api.UHLA_ERR_ARG  # misaligned
    assert f(*lse_args(lse=ctypes.c_void_p(0x40000000 + 64))) == api.UHLA_ERR_ARG  # inside o
    assert f(*lse_args(lse=ctypes.c_void_p(0x20000000 + 64))) == api.UHLA_ERR_ARG  # inside k
    assert f(*lse_args(q=NULL)) == api.UHLA_ERR_ARG
    assert f(*lse_args(d=96)) == api.UHLA_ERR_UNSUPPORTED


def test_forward_rope_at_load_rejects(lib):
    a = fwd_args()
    f = lib.uhla_forward_rope_at_load
    assert f(*a[:17], NULL, NULL) == api.UHLA_ERR_UNSUPPORTED  # w = 8: windows of 64 tokens
    assert f(*fwd_args(q=NULL)[:17], NULL, NULL) == api.UHLA_ERR_ARG
    assert f(*fwd_args(w=16, wsb=1000)[:17], NULL, NULL) == api.UHLA_ERR_WORKSPACE


# uhla_forward_permute_free(q, k, v, o, B, H, W, w, H_lr, W_lr, rho, heads, d, scale, theta,
#                           ws, bytes, stream, timer): the rejections happen on the host
@pytest.mark.parametrize("kw,status", [
    (dict(w=8), api.UHLA_ERR_UNSUPPORTED),  # a 64-key tile would span parts of 8 window rows
    (dict(H=96, W=96, w=48, H_lr=0, W_lr=0), api.UHLA_ERR_UNSUPPORTED),  # 64 % 48, 48 % 64
    (dict(w=16, q=NULL), api.UHLA_ERR_ARG),
    (dict(w=16, d=96), api.UHLA_ERR_UNSUPPORTED),
    (dict(w=16, H=40), api.UHLA_ERR_ARG),  # w must divide H
    # per-lane chunk offsets within a tile are 32-bit: 4 window rows of 2048 tokens of
    # 1024 heads x 128 dims reach 2^31 bytes ...
    (dict(H=16, W=2048, w=16, H_lr=0, W_lr=0, heads=1024, d=128), api.UHLA_ERR_UNSUPPORTED),
    # ... one head fewer stays below and stops at the (too small) workspace
    (dict(H=16, W=2048, w=16, H_lr=0, W_lr=0, heads=1023, d=128, wsb=1000), api.UHLA_ERR_WORKSPACE),
    (dict(w=16, ws=NULL), api.UHLA_ERR_WORKSPACE),
    (dict(w=16, wsb=1000), api.UHLA_ERR_WORKSPACE),
    (dict(w=16, ws=ctypes.c_void_p(0x50000010)), api.UHLA_ERR_ARG),  # misaligned workspace
    (dict(w=16, o=P), api.UHLA_ERR_ARG),  # aliases q
    (dict(w=16, ws=P3), api.UHLA_ERR_ARG),  # workspace overlaps v
])
def test_forward_permute_free_rejects(lib, kw, status):
    assert lib.uhla_forward_permute_free(*fwd_args(**kw), NULL) == status


@pytest.mark.parametrize("g", [g for g in GEOMS if g[3] >= 16] +
                         [(1, 64, 128, 32, 16, 16, 4, 64), (1, 128, 64, 64, 0, 0, 2, 128),
                          (1, 256, 256, 128, 8, 8, 2, 128)])
def test_forward_permute_free_workspace_bytes(lib, g):
    """The permute-free forward's workspace is the fp64 cos/sin table alone: max(H, W)
    positions x d/4 frequency pairs of (cos, sin), 16 bytes each, 256-byte aligned."""
    B, H, W, w, H_lr, W_lr, heads, d = g
    got = lib.uhla_forward_permute_free_workspace_bytes(B, H, W, w, H_lr, W_lr, 4, heads, d)
    assert got == (16 * max(H, W) * (d // 4) + 255) // 256 * 256


def test_forward_permute_free_workspace_bytes_invalid(lib):
    f = lib.uhla_forward_permute_free_workspace_bytes
    assert f(1, 32, 32, 8, 8, 8, 4, 2, 64) == 0     # w = 8
    assert f(1, 96, 96, 48, 0, 0, 4, 2, 64) == 0    # w = 48
    assert f(1, 40, 32, 16, 8, 8, 4, 2, 64) == 0    # w does not divide H
    assert f(1, 32, 32, 16, 8, 0, 4, 2, 64) == 0    # one guide extent zero
    assert f(1, 32, 32, 16, 8, 8, 4, 2, 96) == 0    # head_dim
    assert f(1, 32, 32, 16, 8, 8, 0, 2, 64) == 0    # rho < 1 with guide tokens
    assert f(0, 32, 32, 16, 8, 8, 4, 2, 64) == 0    # batch


def bwd_args(**kw):
    a = dict(q=P, k=P2, v=P3, o=P4, do=ctypes.c_void_p(0x70000000),
             lse=ctypes.c_void_p(0x80000000), dq=ctypes.c_void_p(0x90000000),
             dk=ctypes.c_void_p(0xa0000000), dv=ctypes.c_void_p(0xb0000000), B=1, T=0, H=32,
             W=32, w=8, H_lr=8, W_lr=8, rho=4, heads=2, d=64, scale=0.0, theta=10000.0,
             radius=1, mode=0, ws=ctypes.c_void_p(0x50000000), wsb=1 << 40)
    a.update(kw)
    return tuple(a[n] for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "B", "T", "H",
                                "W", "w", "H_lr", "W_lr", "rho", "heads", "d", "scale", "theta",
                                "radius", "mode", "ws", "wsb")) + (NULL,)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), api.UHLA_ERR_ARG),
    (dict(lse=NULL), api.UHLA_ERR_ARG),
    (dict(dv=NULL), api.UHLA_ERR_ARG),
    (dict(dq=ctypes.c_void_p(0x90000008)), api.UHLA_ERR_ARG),  # not 16-byte aligned
    (dict(B=0), api.UHLA_ERR_ARG),
    (dict(w=12), api.UHLA_ERR_ARG),
    (dict(W_lr=0), api.UHLA_ERR_ARG),
    (dict(rho=0), api.UHLA_ERR_ARG),
    (dict(radius=-1), api.UHLA_ERR_ARG),
    (dict(T=-1), api.UHLA_ERR_ARG),
    (dict(mode=3), api.UHLA_ERR_ARG),
    # modes 1 / 2: 3x3 windows of 96x96 tokens exceed the tile tables here too
    (dict(mode=2, H=384, W=384, w=96, H_lr=96, W_lr=96), api.UHLA_ERR_UNSUPPORTED),
    (dict(T=1 << 25), api.UHLA_ERR_UNSUPPORTED),
    (dict(d=96), api.UHLA_ERR_UNSUPPORTED),
    (dict(H=36, W=36, w=4), api.UHLA_ERR_UNSUPPORTED),
    (dict(H=384, W=384, w=96, H_lr=0, W_lr=0), api.UHLA_ERR_UNSUPPORTED),
    (dict(ws=NULL), api.UHLA_ERR_WORKSPACE),
    (dict(wsb=1000), api.UHLA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x50000010)), api.UHLA_ERR_ARG),  # misaligned workspace
    (dict(dq=P), api.UHLA_ERR_ARG),  # gradient aliases q
    (dict(dk=ctypes.c_void_p(0x90000000 + 4096)), api.UHLA_ERR_ARG),  # overlaps dq
    (dict(dv=ctypes.c_void_p(0x80000000)), api.UHLA_ERR_ARG),  # overlaps lse
    (dict(dq=ctypes.c_void_p(0x50000000 + 4096)), api.UHLA_ERR_ARG),  # inside the workspace
    (dict(ws=ctypes.c_void_p(0x70000000)), api.UHLA_ERR_ARG),  # workspace overlaps dO
    (dict(ws=ctypes.c_void_p(0x80000000)), api.UHLA_ERR_ARG),  # workspace overlaps lse
])
def test_backward_rejects(lib, kw, status):
    assert lib.uhla_backward(*bwd_args(**kw)) == status


def expected_backward_workspace(B, H, W, w, H_lr, W_lr, heads, d, T=0, guide_mode=0):
    """Independent restatement: cos/sin table, then Q, K, V, dO rows per (b, h) with hi rows,
    then guide rows and text rows each padded to 256 (bf16), then per 64-row tile 64 lse2 and
    64 row dots (fp32), then the text blocks' partial sums; regions 256-byte aligned."""
    al = lambda x: (x + 255) // 256 * 256
    N, M = H * W, H_lr * W_lr
    R = N + (M + 255) // 256 * 256 + (T + 255) // 256 * 256
    bh = B * heads
    # text row blocks split their tile lists: about 1024 workgroups, each >= 8 tiles long;
    # two fp32 partial buffers [splits][B*heads][Tp][d]
    Tp = (T + 255) // 256 * 256
    splits = min(-(-1024 // (bh * (Tp // 256))), max(1, R // 64 // 8)) if T else 0
    part = al(splits * bh * Tp * d * 4)
    # guide modes 1 / 2: guide K and V again in 8x8 cell blocks, block rows padded to 4 blocks
    nbjp = -(-(-(-W_lr // 8)) // 4) * 4
    mb = (-(-H_lr // 8)) * nbjp * 64 if (guide_mode and M) else 0
    cells = al(bh * mb * d * 2)
    return (al(16 * max(H, W) * (d // 4)) + 4 * al(bh * R * d * 2) + al(bh * R // 64 * 512)
            + 2 * part + 2 * cells)


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("T,mode", [(0, 0), (1, 0), (300, 0), (0, 1), (77, 2)])
def test_backward_workspace_bytes(lib, g, T, mode):
    B, H, W, w, H_lr, W_lr, heads, d = g
    f = lib.uhla_backward_workspace_bytes
    assert f(B, T, H, W, w, H_lr, W_lr, 4, heads, d, 1, mode) == \
        expected_backward_workspace(*g, T=T, guide_mode=mode)
    assert f(B, T, H, W, w, H_lr, W_lr, 4, heads, d, -1, mode) == 0
    assert f(B, T, H, W, w, H_lr, W_lr, 4, heads, 96, 1, mode) == 0
    assert f(B, -1, H, W, w, H_lr, W_lr, 4, heads, d, 1, mode) == 0
    assert f(B, T, H, W, w, H_lr, W_lr, 4, heads, d, 1, 3) == 0


@pytest.mark.parametrize("args,status", [
    ((NULL, P2, 16384, 0), api.UHLA_ERR_ARG),
    ((P, NULL, 16384, 0), api.UHLA_ERR_ARG),
    ((P, P2, 0, 0), api.UHLA_ERR_ARG),
    ((P, P2, 16000, 1), api.UHLA_ERR_ARG),   # not a multiple of 16384
    ((P, P2, 16384, 3), api.UHLA_ERR_ARG),
    ((P, P2, 16384, -1), api.UHLA_ERR_ARG),
    ((ctypes.c_void_p(0x10000008), P2, 16384, 0), api.UHLA_ERR_ARG),  # misaligned
    ((P, ctypes.c_void_p(0x10000000 + 8192), 16384, 2), api.UHLA_ERR_ARG),  # overlap
])
def test_copy_probe_rejects(lib, args, status):
    assert lib.uhla_copy_probe(*args, NULL) == status


@pytest.mark.parametrize("w,H,W", [(8, 16, 16), (48, 96, 96)])
def test_binding_reports_the_library_status_for_rejected_sizes(lib, monkeypatch, w, H, W):
    """forward() allocates no workspace for sizes whose workspace query returns 0 and lets
    the entry point say why (here on host tensors: the call is rejected before any pointer
    is used or any GPU call is made)."""
    import torch
    monkeypatch.setattr(api, "_require", lambda t, name, dtype=None: None)
    monkeypatch.setattr(api, "_stream", lambda t: NULL)
    L = H * W + 16
    q = torch.zeros(1, L, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(api.UhlaError) as e:
        api.forward(q, q.clone(), q.clone(), H, W, w, 4, 4, permute_free=True)
    assert e.value.status == api.UHLA_ERR_UNSUPPORTED
