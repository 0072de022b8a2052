"""Plain fp64 CPU oracle for UltraGen's hierarchical local attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP path: it is the method's definition written out in numpy,
slowly and in float64, so that a reader can check it against the pages by eye.

Citation keys: [UltraGen/<lang> §n] is the gist.science summary page "UltraGen:
Efficient Ultra-High-Resolution Image Generation with Hierarchical Local Attention"
in the named language edition (it, fr, es, ar, ko), section n of its technical summary.

What the pages fix, and the readings taken where they are silent:

* Window-first token order: hi-res tokens are split into fixed, non-overlapping
  w x w windows and reordered window by window, so each attention block is one
  spatial window ([UltraGen/it §2], [UltraGen/fr §2.A], [UltraGen/ar §2.A]).  Reading:
  windows are enumerated row-major over the window grid, tokens raster inside a window.
* Mask ([UltraGen/ar §2.B], [UltraGen/es §2]): a hi-res window attends to itself, to
  its adjacent windows and to every low-res guide token; guide tokens attend to each
  other.  Readings: "adjacent" is the clipped 3x3 neighbourhood (no wrap); guide
  queries see no hi-res key.  Variants: a neighbourhood radius other than 1, and
  [UltraGen/it §2]'s narrower wording (a window looks at the *corresponding* guide
  tokens): the guide tokens whose scaled position lies in the window (or in its
  neighbourhood).
* Positions ([UltraGen/ar §2.B]): guide-token position indices are scaled by rho
  (4) onto the hi-res grid.  Reading: integer positions (rho*i, rho*j), no offset.
* RoPE ([UltraGen/fr §2.A]: relative positional embeddings).  Readings: 2D axial RoPE,
  half of the head dims per axis (y first), adjacent pairs (2k, 2k+1) rotated by
  pos * theta**(-2k/d_axis), theta = 10000; applied to Q and K, not V.
* Text tokens (optional, T > 0): the joint sequence is text | hi-res | guide
  ([UltraGen/it §2], [UltraGen/fr §2.C]).  Readings (the plain MMDiT joint attention):
  text queries attend to every key, every query attends to every text key; text tokens
  sit at position (0, 0), so RoPE leaves them unrotated.
* Attention: softmax(Q K^T / sqrt(d)) V over the allowed keys.  Every row has at least
  w*w allowed keys, so no row is empty.
* Backward (training the guide path, [UltraGen/it §2] LoRA fine-tuning, [UltraGen/ar §2.C]):
  the gradients of that function with respect to the un-rotated Q, K and V, written out
  from the chain rule; LSE is the natural log of each row's sum of exp(scaled scores).

parity pinned: every function here is checked by tests marked "not gpu" against brute
force, closed forms, invariants or library routines (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------------
# Window-first permutation  ([UltraGen/it §2], [UltraGen/fr §2.A], [UltraGen/ar §2.A])
# ---------------------------------------------------------------------------------

def window_first_source_index(H: int, W: int, w: int) -> np.ndarray:
    """r[p] = raster index of the token placed at window-first position p.

    p = win * w*w + t;  win = wy * (W // w) + wx  (row-major over windows);
    t = iy * w + ix (raster inside the window);  r = (wy*w + iy) * W + (wx*w + ix).
    """
    if H % w or W % w:
        raise ValueError("window size must divide the grid")
    p = np.arange(H * W, dtype=np.int64)
    win, t = np.divmod(p, w * w)
    wy, wx = np.divmod(win, W // w)
    iy, ix = np.divmod(t, w)
    return (wy * w + iy) * W + (wx * w + ix)


def window_permute(x: np.ndarray, H: int, W: int, w: int) -> np.ndarray:
    """Raster -> window-first along axis 1 (the token axis) of ``[B, N, ...]``."""
    r = window_first_source_index(H, W, w)
    return x[:, r]


def window_unpermute(x: np.ndarray, H: int, W: int, w: int) -> np.ndarray:
    """Window-first -> raster along axis 1: out[:, r[p]] = x[:, p]."""
    r = window_first_source_index(H, W, w)
    out = np.empty_like(x)
    out[:, r] = x
    return out


# ---------------------------------------------------------------------------------
# Positions  ([UltraGen/ar §2.B]: guide positions scaled by rho onto the hi-res grid)
# ---------------------------------------------------------------------------------

def hi_positions(H: int, W: int):
    """(y, x) of hi-res raster tokens 0..H*W-1."""
    r = np.arange(H * W, dtype=np.int64)
    return r // W, r % W


def lr_positions(H_lr: int, W_lr: int, rho: int):
    """(y, x) of guide raster tokens: (rho * i, rho * j)."""
    s = np.arange(H_lr * W_lr, dtype=np.int64)
    return rho * (s // W_lr), rho * (s % W_lr)


def token_positions(geom):
    """(y, x) for all L tokens of the joint [text | hi | lr] sequence: text tokens at
    (0, 0), hi and guide tokens raster."""
    T = getattr(geom, "T", 0)
    yh, xh = hi_positions(geom.H, geom.W)
    yl, xl = lr_positions(geom.H_lr, geom.W_lr, geom.rho)
    z = np.zeros(T, dtype=np.int64)
    return np.concatenate([z, yh, yl]), np.concatenate([z, xh, xl])


# ---------------------------------------------------------------------------------
# 2D axial RoPE
# ---------------------------------------------------------------------------------

def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_k = theta ** (-2k / d_axis), k = 0 .. d_axis/2 - 1, d_axis = head_dim / 2."""
    d_axis = head_dim // 2
    k = np.arange(d_axis // 2, dtype=np.float64)
    return theta ** (-2.0 * k / d_axis)


def rope_rotate(x: np.ndarray, pos_y: np.ndarray, pos_x: np.ndarray, theta: float) -> np.ndarray:
    """Rotate ``x[..., T, heads, d]`` (fp64) by token positions (pos_y, pos_x) of length T.

    Dims [0, d/2) rotate by the y position, dims [d/2, d) by the x position.  Within an
    axis block, pair (2k, 2k+1) = (a, b) becomes (a cos phi - b sin phi, a sin phi + b cos phi)
    with phi = pos * omega_k.
    """
    d = x.shape[-1]
    if d % 4:
        raise ValueError("head_dim must be a multiple of 4 for 2D axial RoPE")
    d_axis = d // 2
    omega = rope_frequencies(d, theta)
    out = np.empty(x.shape, dtype=np.float64)
    for axis_block, pos in ((0, pos_y), (1, pos_x)):
        phi = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]  # [T, d_axis/2]
        c = np.cos(phi)[:, None, :]  # broadcast over heads
        s = np.sin(phi)[:, None, :]
        lo = axis_block * d_axis
        a = x[..., lo:lo + d_axis:2].astype(np.float64)
        b = x[..., lo + 1:lo + d_axis:2].astype(np.float64)
        out[..., lo:lo + d_axis:2] = a * c - b * s
        out[..., lo + 1:lo + d_axis:2] = a * s + b * c
    return out


def rope_joint(x: np.ndarray, geom) -> np.ndarray:
    """RoPE on a full ``[B, L, heads, d]`` tensor in the [text | hi | lr] layout."""
    py, px = token_positions(geom)
    return rope_rotate(x, py, px, geom.theta)


# ---------------------------------------------------------------------------------
# Mask  ([UltraGen/ar §2.B] attention-mask bullets; [UltraGen/es §2])
# ---------------------------------------------------------------------------------

def mask_block(geom, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Explicit boolean mask entries for query rows ``rows`` and key columns ``cols`` of the
    [text | hi | lr] sequence (both raster indices into the L tokens).

    hi q -> hi k : allowed iff the windows differ by at most ``radius`` in both axes
                   (radius 1: the clipped 3x3 neighbourhood of the pages);
    hi q -> lr k : guide_mode 0: always; 1: iff the guide token's scaled position
                   (rho*i, rho*j) lies in the query's window; 2: iff it lies in a window
                   of the query's neighbourhood (scaled positions outside the hi-res grid
                   belong to no window);
    lr q -> lr k : always;   lr q -> hi k : never;
    text q -> any k, and any q -> text k : always.
    """
    rows = np.asarray(rows, dtype=np.int64)
    key = np.asarray(cols, dtype=np.int64)
    T = getattr(geom, "T", 0)
    N, w = geom.N, geom.w
    r = getattr(geom, "radius", 1)
    mode = getattr(geom, "guide_mode", 0)
    key_is_text = key < T
    key_is_hi = (key >= T) & (key < T + N)
    key_is_lr = key >= T + N
    kh = np.where(key_is_hi, key - T, 0)
    ky, kx = kh // geom.W, kh % geom.W
    q_is_text = rows < T
    q_is_hi = (rows >= T) & (rows < T + N)
    q_is_lr = rows >= T + N
    qh = np.where(q_is_hi, rows - T, 0)
    qy, qx = qh // geom.W, qh % geom.W
    near = (np.abs(qy[:, None] // w - ky[None, :] // w) <= r) & \
           (np.abs(qx[:, None] // w - kx[None, :] // w) <= r)
    hi_hi = q_is_hi[:, None] & key_is_hi[None, :] & near
    if mode == 0:
        hi_lr = q_is_hi[:, None] & key_is_lr[None, :]
    else:
        s = np.where(key_is_lr, key - T - N, 0)
        gy = geom.rho * (s // max(geom.W_lr, 1))
        gx = geom.rho * (s % max(geom.W_lr, 1))
        inside = key_is_lr & (gy < geom.H) & (gx < geom.W)
        reach = 0 if mode == 1 else r
        close = (np.abs(qy[:, None] // w - gy[None, :] // w) <= reach) & \
                (np.abs(qx[:, None] // w - gx[None, :] // w) <= reach)
        hi_lr = q_is_hi[:, None] & inside[None, :] & close
    lr_lr = q_is_lr[:, None] & key_is_lr[None, :]
    text = q_is_text[:, None] | key_is_text[None, :]
    return hi_hi | hi_lr | lr_lr | text


def mask_rows(geom, rows: np.ndarray) -> np.ndarray:
    """Explicit boolean mask rows over all L keys for query rows ``rows`` (the rules of
    ``mask_block``)."""
    return mask_block(geom, rows, np.arange(geom.L, dtype=np.int64))


# ---------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------

def masked_softmax_attention(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
                             mask: np.ndarray, scale: float, return_probs: bool = False):
    """Dense softmax attention for a block of query rows of one (batch, head).

    q_rows [R, d], k [L, d], v [L, d], mask [R, L] (True = allowed).  S = q k^T * scale,
    masked entries -inf, subtract row max, exp, normalise, P v.
    """
    s = (q_rows @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    return (o, p) if return_probs else o


def rotated_qk(q: np.ndarray, k: np.ndarray, geom, b: int, h: int):
    """RoPE-rotated fp64 Q and K rows of one (batch, head): [L, d] each."""
    py, px = token_positions(geom)
    qbh = q[b, :, h:h + 1, :].astype(np.float64)
    kbh = k[b, :, h:h + 1, :].astype(np.float64)
    if geom.theta > 0:
        qbh = rope_rotate(qbh, py, px, geom.theta)
        kbh = rope_rotate(kbh, py, px, geom.theta)
    return qbh[:, 0, :], kbh[:, 0, :]


def attention_rows(q, k, v, geom, b: int, h: int, rows, block: int = 512, qk=None):
    """Oracle output rows (raster index ``rows``) of one (batch, head), fp64 ``[R, d]``.

    ``qk`` may carry the already rotated (Q, K) of this (b, h) to avoid recomputing it.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qr, kr = qk if qk is not None else rotated_qk(q, k, geom, b, h)
    vv = v[b, :, h, :].astype(np.float64)
    out = np.empty((len(rows), q.shape[-1]), dtype=np.float64)
    for s in range(0, len(rows), block):
        blk = rows[s:s + block]
        out[s:s + len(blk)] = masked_softmax_attention(qr[blk], kr, vv, mask_rows(geom, blk),
                                                       geom.scale)
    return out


def forward(q, k, v, geom, block: int = 512) -> np.ndarray:
    """Full oracle forward: fp64 ``[B, L, heads, d]`` in the [text | hi | lr] layout.

    Permute -> attend -> unpermute leaves the result in raster order, and the mask is
    defined on positions, so the oracle attends in raster order directly.
    """
    B, L, Hh, d = q.shape
    out = np.empty((B, L, Hh, d), dtype=np.float64)
    rows = np.arange(L)
    for b in range(B):
        for h in range(Hh):
            out[b, :, h, :] = attention_rows(q, k, v, geom, b, h, rows, block)
    return out


def allowed_key_count(geom, rows) -> np.ndarray:
    """Number of allowed keys for each query row (from the explicit mask)."""
    return mask_rows(geom, rows).sum(axis=1)

# ---------------------------------------------------------------------------------
# Backward (gradients of the forward above) and the per-row log-sum-exp
# ---------------------------------------------------------------------------------

def rope_rotate_inverse(x: np.ndarray, pos_y: np.ndarray, pos_x: np.ndarray,
                        theta: float) -> np.ndarray:
    """The transpose (= inverse) of rope_rotate: each pair rotated by -phi."""
    d = x.shape[-1]
    d_axis = d // 2
    omega = rope_frequencies(d, theta)
    out = np.empty(x.shape, dtype=np.float64)
    for axis_block, pos in ((0, pos_y), (1, pos_x)):
        phi = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]
        c = np.cos(phi)[:, None, :]
        s = np.sin(phi)[:, None, :]
        lo = axis_block * d_axis
        a = x[..., lo:lo + d_axis:2].astype(np.float64)
        b = x[..., lo + 1:lo + d_axis:2].astype(np.float64)
        out[..., lo:lo + d_axis:2] = a * c + b * s
        out[..., lo + 1:lo + d_axis:2] = -a * s + b * c
    return out


def lse_rows(q, k, geom, b: int, h: int, rows, block: int = 512, qk=None) -> np.ndarray:
    """log sum_j exp(scale * q_i . k_j) over the allowed keys j of each query row i."""
    rows = np.asarray(rows, dtype=np.int64)
    qr, kr = qk if qk is not None else rotated_qk(q, k, geom, b, h)
    out = np.empty(len(rows), dtype=np.float64)
    for s0 in range(0, len(rows), block):
        blk = rows[s0:s0 + block]
        sc = (qr[blk] @ kr.T) * geom.scale
        sc = np.where(mask_rows(geom, blk), sc, -np.inf)
        mx = sc.max(axis=1)
        out[s0:s0 + len(blk)] = mx + np.log(np.exp(sc - mx[:, None]).sum(axis=1))
    return out


def backward(q, k, v, do, geom):
    """Gradients (dQ, dK, dV), fp64 ``[B, L, heads, d]``, of O = forward(q, k, v, geom) for the
    output gradient ``do``.  Per (batch, head), with rotated Q~, K~ and the scale s:
    P = softmax(s Q~ K~^T + mask), dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)),
    dQ~ = s dS K~, dK~ = s dS^T Q~; dQ and dK rotate dQ~ and dK~ back (transpose of RoPE)."""
    B, L, Hh, d = q.shape
    py, px = token_positions(geom)
    dq = np.empty((B, L, Hh, d))
    dk = np.empty((B, L, Hh, d))
    dv = np.empty((B, L, Hh, d))
    mask = mask_rows(geom, np.arange(L))
    for b in range(B):
        for h in range(Hh):
            qr, kr = rotated_qk(q, k, geom, b, h)
            vv = v[b, :, h].astype(np.float64)
            g = do[b, :, h].astype(np.float64)
            _, p = masked_softmax_attention(qr, kr, vv, mask, geom.scale, return_probs=True)
            dv[b, :, h] = p.T @ g
            dp = g @ vv.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dqr = geom.scale * (ds @ kr)
            dkr = geom.scale * (ds.T @ qr)
            if geom.theta > 0:
                dqr = rope_rotate_inverse(dqr[:, None, :], py, px, geom.theta)[:, 0, :]
                dkr = rope_rotate_inverse(dkr[:, None, :], py, px, geom.theta)[:, 0, :]
            dq[b, :, h] = dqr
            dk[b, :, h] = dkr
    return dq, dk, dv


def backward_rows(q, k, v, do, geom, b: int, h: int, q_rows, k_rows, block: int = 512):
    """Rows of the backward of one (batch, head) without the full L x L matrices:
    (dQ[q_rows], dK[k_rows], dV[k_rows]), fp64.

    The arithmetic of ``backward`` restricted to the query rows that matter: the rows in
    ``q_rows`` and every query row whose mask row allows one of ``k_rows`` and whose dO
    row is not zero (a key's gradients sum over those rows only; every other entry of its
    column of P dO and dS is zero).  For each block of those rows: P = masked softmax of the row block over all L
    keys, dP = dO V^T, dS = P * (dP - rowsum(dP * P)); dV[k] and dK~[k] sum P[:, k] dO and
    s dS[:, k] Q~ over the block, dQ~ = s dS K~; dQ, dK rotate back."""
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    L = q.shape[1]
    py, px = token_positions(geom)
    qr, kr = rotated_qk(q, k, geom, b, h)
    vv = v[b, :, h].astype(np.float64)
    g = do[b, :, h].astype(np.float64)
    need = np.zeros(L, dtype=bool)
    need[q_rows] = True
    if len(k_rows):
        # a row with dO = 0 has dP = 0, a zero row dot and so dS = 0: it adds nothing to
        # any key's dK or dV, and is skipped (exact)
        live = np.any(g != 0, axis=1)
        for s0 in range(0, L, 8 * block):
            blk = np.arange(s0, min(L, s0 + 8 * block))
            need[blk] |= mask_block(geom, blk, k_rows).any(axis=1) & live[blk]
    rows = np.nonzero(need)[0]
    dq = np.zeros((len(q_rows), q.shape[-1]))
    dk = np.zeros((len(k_rows), q.shape[-1]))
    dv = np.zeros((len(k_rows), q.shape[-1]))
    for s0 in range(0, len(rows), block):
        blk = rows[s0:s0 + block]
        _, p = masked_softmax_attention(qr[blk], kr, vv, mask_rows(geom, blk), geom.scale,
                                        return_probs=True)
        dp = g[blk] @ vv.T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dv += p[:, k_rows].T @ g[blk]
        dk += geom.scale * (ds[:, k_rows].T @ qr[blk])
        for i, r in enumerate(blk):
            hit = np.nonzero(q_rows == r)[0]
            if len(hit):
                dq[hit] = geom.scale * (ds[i] @ kr)
    if geom.theta > 0:
        dq = rope_rotate_inverse(dq[:, None, :], py[q_rows], px[q_rows], geom.theta)[:, 0, :]
        dk = rope_rotate_inverse(dk[:, None, :], py[k_rows], px[k_rows], geom.theta)[:, 0, :]
    return dq, dk, dv
