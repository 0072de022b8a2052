"""Thin Python binding of libuhla (ctypes): argument marshalling only.

Every step of the path runs in the HIP library; torch supplies device memory and the
current stream.  If the library is missing, every call raises: there is no fallback.
The entry points mirror ``include/uhla.h`` one to one.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libuhla.so")

UHLA_OK, UHLA_ERR_ARG, UHLA_ERR_UNSUPPORTED, UHLA_ERR_WORKSPACE, UHLA_ERR_HIP = range(5)
STAGES = ("tables", "prep_hi", "prep_lr", "attn_hi", "attn_lr", "unpermute", "attn_text")

EXPORTS = {
    # name: (restype, argtypes)
    "uhla_window_permute": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 7
                            + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "uhla_window_unpermute": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 7
                              + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "uhla_rope_apply": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 10
                        + [ctypes.c_float, ctypes.c_void_p]),
    "uhla_forward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 8),
    "uhla_forward": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                     + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                        ctypes.c_void_p]),
    "uhla_forward_masked_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 11),
    "uhla_forward_masked": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                            + [ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "uhla_forward_masked_timed": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                                  + [ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]),
    "uhla_forward_text_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 12),
    "uhla_forward_text": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 10
                          + [ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "uhla_forward_lse": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 10
                         + [ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "uhla_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 12),
    "uhla_backward": (ctypes.c_int, [ctypes.c_void_p] * 9 + [ctypes.c_int] * 10
                      + [ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "uhla_forward_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                             + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p]),
    "uhla_copy_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]),
    "uhla_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "uhla_last_error_detail": (ctypes.c_char_p, []),
    "uhla_timer_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]),
    "uhla_timer_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "uhla_timer_reset": (ctypes.c_int, [ctypes.c_void_p]),
    "uhla_timer_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "uhla_forward_timed": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                           + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_void_p, ctypes.c_void_p]),
    "uhla_forward_rope_at_load": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                                  + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "uhla_forward_permute_free_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 9),
    "uhla_forward_permute_free": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 9
                                  + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
}

_lib = None


class UhlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        name = lib.uhla_strerror(status).decode()
        detail = lib.uhla_last_error_detail().decode()
        super().__init__(f"{where}: {name} ({detail})")
        self.status = status


def load():
    """Load libuhla.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with "
                           "`python -m global_attention_image_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != UHLA_OK:
        raise UhlaError(status, where)


def _stream(tensor):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(tensor.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def window_permute(src, dst, H, W, w, src_tokens_per_batch=None, dst_tokens_per_batch=None):
    """dst[b, p] = src[b, r(p)] for the H*W hi-res rows; tensors are [B, T, heads, d]."""
    return _permute("uhla_window_permute", src, dst, H, W, w, src_tokens_per_batch,
                    dst_tokens_per_batch)


def window_unpermute(src, dst, H, W, w, src_tokens_per_batch=None, dst_tokens_per_batch=None):
    """dst[b, r(p)] = src[b, p] for the H*W hi-res rows; tensors are [B, T, heads, d]."""
    return _permute("uhla_window_unpermute", src, dst, H, W, w, src_tokens_per_batch,
                    dst_tokens_per_batch)


def _permute(name, src, dst, H, W, w, stpb, dtpb):
    _require(src, "src")
    _require(dst, "dst", src.dtype)
    if src.dim() != 4 or dst.dim() != 4:
        raise ValueError("tensors must be [B, tokens, heads, head_dim]")
    B, Ts, Hh, d = src.shape
    if dst.shape[0] != B or dst.shape[2:] != src.shape[2:]:
        raise ValueError("src and dst must agree in batch, heads and head_dim")
    lib = load()
    st = getattr(lib, name)(_ptr(src), _ptr(dst), B, H, W, w, Hh, d, src.element_size(),
                            Ts if stpb is None else stpb, dst.shape[1] if dtpb is None else dtpb,
                            _stream(src))
    _check(st, name)
    return dst


def rope_apply(src, dst, H, W, H_lr, W_lr, rho=4, theta=10000.0, w=0, hi_order=0):
    """2D axial RoPE on a bf16 [B, H*W + H_lr*W_lr, heads, d] tensor (dst may be src)."""
    import torch
    _require(src, "src", torch.bfloat16)
    _require(dst, "dst", torch.bfloat16)
    if dst.shape != src.shape:
        raise ValueError("shape mismatch")
    B, L, Hh, d = src.shape
    if L != H * W + H_lr * W_lr:
        raise ValueError("token count does not match the grids")
    st = load().uhla_rope_apply(_ptr(src), _ptr(dst), B, H, W, w, hi_order, H_lr, W_lr, rho,
                                Hh, d, float(theta), _stream(src))
    _check(st, "uhla_rope_apply")
    return dst


def forward_noalloc(q, k, v, H, W, w, H_lr, W_lr, rho=4, scale=0.0, theta=10000.0, out=None):
    """uhla_forward with the library's static scratch instead of a workspace (no device
    allocation inside the call; ``out`` must be given to avoid allocating it here)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, torch.bfloat16)
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, L, heads, head_dim] shape")
    B, L, Hh, d = q.shape
    if L != H * W + H_lr * W_lr:
        raise ValueError("token count does not match the grids")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16)
    st = load().uhla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, W, w, H_lr,
                                     W_lr, rho, Hh, d, float(scale), float(theta), _stream(q))
    _check(st, "uhla_forward_noalloc")
    return out


def copy_probe(src, dst, mode):
    """Copy all bytes of ``src`` into ``dst`` (same byte size, a multiple of 16384) through
    load path ``mode`` (0 plain, 1 nontemporal, 2 direct-to-LDS); a measurement aid."""
    _require(src, "src")
    _require(dst, "dst")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must hold the same number of bytes")
    _check(load().uhla_copy_probe(_ptr(src), _ptr(dst), nb, int(mode), _stream(src)),
           "uhla_copy_probe")
    return dst


def forward_workspace_bytes(B, H, W, w, H_lr, W_lr, heads, head_dim) -> int:
    return int(load().uhla_forward_workspace_bytes(B, H, W, w, H_lr, W_lr, heads, head_dim))


def forward_masked_workspace_bytes(B, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                                   guide_mode) -> int:
    return int(load().uhla_forward_masked_workspace_bytes(B, H, W, w, H_lr, W_lr, rho, heads,
                                                          head_dim, radius, guide_mode))


def forward_text_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                                 guide_mode) -> int:
    return int(load().uhla_forward_text_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads,
                                                        head_dim, radius, guide_mode))


def workspace_bytes_for(B, H, W, w, H_lr, W_lr, heads, head_dim, rho=4, radius=1, guide_mode=0,
                        T=0, permute_free=False) -> int:
    """Workspace bytes of the forward entry point that forward() selects for these options
    (0 when the library rejects the sizes)."""
    if permute_free:
        n = load().uhla_forward_permute_free_workspace_bytes(B, H, W, w, H_lr, W_lr, rho, heads,
                                                             head_dim)
    elif T:
        n = forward_text_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                                         guide_mode)
    elif radius == 1 and guide_mode == 0:
        n = forward_workspace_bytes(B, H, W, w, H_lr, W_lr, heads, head_dim)
    else:
        n = forward_masked_workspace_bytes(B, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                                           guide_mode)
    return int(n)


def alloc_workspace(B, H, W, w, H_lr, W_lr, heads, head_dim, device="cuda", rho=4, radius=1,
                    guide_mode=0, T=0, permute_free=False):
    import torch
    n = workspace_bytes_for(B, H, W, w, H_lr, W_lr, heads, head_dim, rho=rho, radius=radius,
                            guide_mode=guide_mode, T=T, permute_free=permute_free)
    if n == 0:
        raise ValueError("invalid geometry")
    return torch.empty(n, dtype=torch.uint8, device=device)


class Timer:
    """HIP-event stage timer (see uhla_timer_* in uhla.h)."""

    def __init__(self, max_calls: int):
        self.h = ctypes.c_void_p()
        _check(load().uhla_timer_create(max_calls, ctypes.byref(self.h)), "uhla_timer_create")

    def reset(self):
        _check(load().uhla_timer_reset(self.h), "uhla_timer_reset")

    def read(self):
        ms = (ctypes.c_double * len(STAGES))()
        calls = ctypes.c_int()
        _check(load().uhla_timer_read(self.h, ms, len(STAGES), ctypes.byref(calls)),
               "uhla_timer_read")
        return {s: ms[i] for i, s in enumerate(STAGES)}, calls.value

    def close(self):
        if self.h:
            load().uhla_timer_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward(q, k, v, H, W, w, H_lr, W_lr, rho=4, scale=0.0, theta=10000.0, out=None,
            workspace=None, timer: Timer | None = None, radius=1, guide_mode=0, T=0,
            rope_at_load=False, permute_free=False):
    """Hierarchical local attention forward on bf16 [B, T + H*W + H_lr*W_lr, heads, d] tensors.

    radius / guide_mode select the mask variants of uhla_forward_masked and T > 0 the text
    tokens of uhla_forward_text (rows 0..T-1); with the defaults uhla_forward is called.
    rope_at_load selects uhla_forward_rope_at_load (K rotated at every K tile load) and
    permute_free uhla_forward_permute_free (no K/V prep pass), both for the default mask
    only.  A timer records per-stage durations (uhla_forward_timed /
    uhla_forward_masked_timed / uhla_forward_text / uhla_forward_rope_at_load /
    uhla_forward_permute_free).  Sizes the library rejects get no workspace, and the
    entry point's status is raised as UhlaError."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, torch.bfloat16)
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, L, heads, head_dim] shape")
    B, L, Hh, d = q.shape
    if L != T + H * W + H_lr * W_lr:
        raise ValueError("token count does not match the grids")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16)
    if (rope_at_load or permute_free) and (T or radius != 1 or guide_mode != 0):
        raise ValueError("rope_at_load and permute_free cover the default mask only")
    if rope_at_load and permute_free:
        raise ValueError("choose one of rope_at_load and permute_free")
    if workspace is None and workspace_bytes_for(B, H, W, w, H_lr, W_lr, Hh, d, rho=rho,
                                                 radius=radius, guide_mode=guide_mode, T=T,
                                                 permute_free=permute_free) > 0:
        workspace = alloc_workspace(B, H, W, w, H_lr, W_lr, Hh, d, q.device, rho=rho,
                                    radius=radius, guide_mode=guide_mode, T=T,
                                    permute_free=permute_free)
    lib = load()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, W, w, H_lr, W_lr, rho, Hh, d,
            float(scale), float(theta))
    # sizes the library rejects have no workspace: the entry point reports why
    tail = (_ptr(workspace) if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, _stream(q))
    if rope_at_load:
        st = lib.uhla_forward_rope_at_load(*args, *tail, timer.h if timer is not None else None)
        _check(st, "uhla_forward_rope_at_load")
        return out
    if permute_free:
        st = lib.uhla_forward_permute_free(*args, *tail, timer.h if timer is not None else None)
        _check(st, "uhla_forward_permute_free")
        return out
    if T:
        st = lib.uhla_forward_text(*args[:5], int(T), *args[5:], int(radius), int(guide_mode),
                                   *tail, timer.h if timer is not None else None)
        _check(st, "uhla_forward_text")
        return out
    if radius != 1 or guide_mode != 0:
        if timer is None:
            st = lib.uhla_forward_masked(*args, int(radius), int(guide_mode), *tail)
        else:
            st = lib.uhla_forward_masked_timed(*args, int(radius), int(guide_mode), *tail,
                                               timer.h)
        _check(st, "uhla_forward_masked")
        return out
    if timer is None:
        st = lib.uhla_forward(*args, *tail)
    else:
        st = lib.uhla_forward_timed(*args, *tail, timer.h)
    _check(st, "uhla_forward")
    return out


def forward_lse(q, k, v, H, W, w, H_lr, W_lr, rho=4, scale=0.0, theta=10000.0, radius=1,
                guide_mode=0, T=0, out=None, lse=None, workspace=None):
    """uhla_forward_lse: the forward plus the per-row natural-log sum of exp of the scaled
    scores, fp32 [B, heads, L].  Returns (out, lse)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, torch.bfloat16)
    B, L, Hh, d = q.shape
    if L != T + H * W + H_lr * W_lr:
        raise ValueError("token count does not match the grids")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hh, L), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(out, "out", torch.bfloat16)
    _require(lse, "lse", torch.float32)
    if workspace is None:
        workspace = alloc_workspace(B, H, W, w, H_lr, W_lr, Hh, d, q.device, rho=rho,
                                    radius=radius, guide_mode=guide_mode, T=T)
    st = load().uhla_forward_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T, H, W, w,
                                 H_lr, W_lr, rho, Hh, d, float(scale), float(theta), int(radius),
                                 int(guide_mode), _ptr(workspace), workspace.numel(), _stream(q))
    _check(st, "uhla_forward_lse")
    return out, lse


def backward_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                             guide_mode=0) -> int:
    return int(load().uhla_backward_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads,
                                                    head_dim, radius, guide_mode))


def backward(q, k, v, o, do, lse, H, W, w, H_lr, W_lr, rho=4, scale=0.0, theta=10000.0,
             radius=1, T=0, guide_mode=0, dq=None, dk=None, dv=None, workspace=None):
    """uhla_backward: (dq, dk, dv) bf16 for the output gradient do (T text tokens in rows
    0..T-1; radius and guide_mode as in the forward)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _require(t, n, torch.bfloat16)
    _require(lse, "lse", torch.float32)
    B, L, Hh, d = q.shape
    if L != T + H * W + H_lr * W_lr:
        raise ValueError("token count does not match the grids")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if workspace is None:
        n = backward_workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, Hh, d, radius, guide_mode)
        if n == 0:
            raise ValueError("invalid geometry")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = load().uhla_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, int(T), H, W, w, H_lr, W_lr, rho, Hh, d,
                              float(scale), float(theta), int(radius), int(guide_mode),
                              _ptr(workspace),
                              workspace.numel(), _stream(q))
    _check(st, "uhla_backward")
    return dq, dk, dv
