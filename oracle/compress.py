"""Spatial token compression: keep sets and nearest-kept maps.

Source: PaperDaily review, section 2 (Flash): in the compressed layers each
frame keeps every other position along rows and columns (about a quarter of
the spatial positions) together with the edge rows and columns; the time axis,
text and audio are never subsampled; every dropped position takes the update of
the nearest kept position of the same frame. The tokendh.com article, training
section, states the same 2x spatial subsampling with boundary rows/columns kept.

Readings (the pages give no formula):
  * kept rows K(n, s) = {r : r mod s == 0} U {n - 1}; same for columns; the
    kept set of a frame is the product K_H x K_W, in raster (t, h, w) order.
  * "nearest" is per axis, argmin |r - k| over k in K, ties to the lower k.
    For a product keep set this is the 2D nearest kept position (checked by
    brute force in the tests).
"""
from __future__ import annotations

import numpy as np


def keep_axis(n: int, s: int = 2) -> list:
    """Kept indices along one axis of length n with stride s, ascending."""
    if n < 1 or s < 1:
        raise ValueError("n and s must be >= 1")
    return [r for r in range(n) if r % s == 0 or r == n - 1]


def nearest_axis(n: int, s: int = 2) -> list:
    """For every r in [0, n): the kept index nearest to r (ties -> lower)."""
    kept = keep_axis(n, s)
    out = []
    for r in range(n):
        best = None
        for k in kept:  # ascending, so strict '<' keeps the lower index on ties
            if best is None or abs(r - k) < abs(r - best):
                best = k
        out.append(best)
    return out


def keep_dims(H: int, W: int, s: int = 2) -> tuple:
    return len(keep_axis(H, s)), len(keep_axis(W, s))


def keep_index(T: int, H: int, W: int, s: int = 2) -> np.ndarray:
    """int32 [T*Hk*Wk]: flat video position t*H*W + h*W + w of each kept slot,
    in raster order of (t, h, w)."""
    kh, kw = keep_axis(H, s), keep_axis(W, s)
    out = [t * H * W + h * W + w for t in range(T) for h in kh for w in kw]
    return np.asarray(out, dtype=np.int32)


def nearest_kept_map(T: int, H: int, W: int, s: int = 2) -> np.ndarray:
    """int32 [T*H*W]: for each video position (raster order) the kept slot j
    (index into keep_index) of (t, nearest_h(h), nearest_w(w))."""
    kh, kw = keep_axis(H, s), keep_axis(W, s)
    nh, nw = nearest_axis(H, s), nearest_axis(W, s)
    rank_h = {k: i for i, k in enumerate(kh)}
    rank_w = {k: i for i, k in enumerate(kw)}
    Hk, Wk = len(kh), len(kw)
    col = np.asarray([rank_w[nw[w]] for w in range(W)], dtype=np.int64)
    row = np.asarray([rank_h[nh[h]] for h in range(H)], dtype=np.int64)
    t = np.arange(T, dtype=np.int64)
    slot = t[:, None, None] * (Hk * Wk) + row[None, :, None] * Wk + col[None, None, :]
    return slot.reshape(-1).astype(np.int32)


def kept_coords(T: int, H: int, W: int, s: int = 2) -> np.ndarray:
    """int64 [T*Hk*Wk, 3]: original (t, h, w) of each kept slot (compressed
    tokens keep their original coordinates)."""
    kh, kw = keep_axis(H, s), keep_axis(W, s)
    return np.asarray([(t, h, w) for t in range(T) for h in kh for w in kw], dtype=np.int64).reshape(-1, 3)


def history_frames(n_hist: int) -> list:
    """Bounded long-video history (tokendh.com article, long-video section;
    PaperDaily review, section 3): of the n_hist latent frames generated so
    far (0 = the first), the first frame stays at full spatial resolution, the
    two most recent are sampled at stride 2 and up to eight frames before them
    at stride 4; frames in the middle beyond that are dropped (the first and
    the most recent are kept). Returns [(frame, stride)] in frame order."""
    if n_hist < 0:
        raise ValueError("n_hist must be >= 0")
    if n_hist == 0:
        return []
    recent = [f for f in (n_hist - 2, n_hist - 1) if f >= 1]
    middle = list(range(max(1, n_hist - 2 - 8), n_hist - 2))
    return [(0, 1)] + [(f, 4) for f in middle] + [(f, 2) for f in recent]


def history_index(n_hist: int, H: int, W: int) -> np.ndarray:
    """int32: flat positions f*H*W + h*W + w, in the [n_hist, H, W] grid of
    the history latents, of the history tokens, frame by frame in raster
    order. Reading: a frame at stride s keeps rows and columns that are
    multiples of s (plain stride sampling, without the compression's extra
    edge row and column: then the whole history holds exactly two full frames
    of tokens when H and W are multiples of 4, the budget the pages state)."""
    out = []
    for f, s in history_frames(n_hist):
        out += [f * H * W + h * W + w for h in range(0, H, s) for w in range(0, W, s)]
    return np.asarray(out, dtype=np.int32)
