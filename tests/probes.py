"""Closed forms of the uniform-weight probe (Q = 0) used as full-size checks.

With Q = 0 every score is 0, so each query row spreads its weight evenly over the keys its
mask row allows: P[i, j] = 1 / c_i on allowed pairs, c_i = the row's allowed-key count
(the mask of [UltraGen/ar §2.B]: a hi-res query sees the clipped 3x3 neighbourhood of
windows, w*w keys each, and every guide token; a guide query sees every guide token).
Hence the backward's dV[j] = sum over the queries i that see key j of dO[i] / c_i.  These
sums are written out here from window aggregates; tests/test_oracle_pins.py pins them
against the oracle's backward on small grids."""
import numpy as np


def window_counts(geom):
    """Allowed-key count of a hi query in each window, [n_wy, n_wx] (default mask)."""
    nwy, nwx = geom.H // geom.w, geom.W // geom.w
    cy = np.array([sum(0 <= a < nwy for a in (i - 1, i, i + 1)) for i in range(nwy)])
    cx = np.array([sum(0 <= a < nwx for a in (i - 1, i, i + 1)) for i in range(nwx)])
    return cy[:, None] * cx[None, :] * geom.w * geom.w + geom.M


def uniform_probe_dv(geom, do):
    """dV of every key of one (batch, head) for Q = 0 and output gradient ``do`` [L, d]
    (fp64), in the [hi | guide] layout (no text tokens), default mask."""
    H, W, w, N, M = geom.H, geom.W, geom.w, geom.N, geom.M
    nwy, nwx = H // w, W // w
    d = do.shape[-1]
    hi = do[:N].reshape(nwy, w, nwx, w, d)
    win_sum = hi.sum(axis=(1, 3))                                  # [nwy, nwx, d]
    contrib = win_sum / window_counts(geom)[:, :, None]            # sum_i dO_i / c_i per window
    # each key window collects the contributions of its clipped 3x3 neighbourhood
    pad = np.zeros((nwy + 2, nwx + 2, d))
    pad[1:-1, 1:-1] = contrib
    nb = sum(pad[1 + dy:1 + dy + nwy, 1 + dx:1 + dx + nwx] for dy in (-1, 0, 1) for dx in (-1, 0, 1))
    dv = np.empty((N + M, d))
    dv[:N] = np.broadcast_to(nb[:, None, :, None, :], (nwy, w, nwx, w, d)).reshape(N, d)
    if M:
        dv[N:] = contrib.sum(axis=(0, 1)) + do[N:].sum(axis=0) / M
    return dv
