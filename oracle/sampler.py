"""Few-step flow-matching sampler over a stack of Flash blocks.

Sources:
  * tokendh.com article, training section: flow matching mixes clean data and
    noise by time and learns the velocity; video and audio use separate noise
    clocks, with printed clean times for four evaluations at native 768p
    (video 0, 0.027, 0.0769, 0.2; audio 0, 0.1, 0.25, 0.5). Flash keeps 42 of
    the 50 layers and runs 3 evaluations: layers 1-2 on the full sequence,
    the middle 26 compressed, the last 14 at full resolution.
  * PaperDaily review, section 2: same schedule of layers and evaluations.
  * tokendh.com article, long-video section, and PaperDaily review, section
    3: long videos are generated chunk by chunk; the last frame of a chunk is
    shared as the fixed first frame of the next, which predicts 5 new latent
    frames (17 new pixel frames) from it, with the bounded history of the
    earlier frames as context.

Readings:
  * clean time t runs from 0 (noise) to 1 (clean); one Euler step per
    evaluation, x <- x + (t_{k+1} - t_k) * v, with v the stack output on the
    video and audio rows (there is no final projection in this block form);
    text rows are re-fed unchanged;
  * schedule: t_k = u / (u + shift (1 - u)), u = k / N, t_N = 1. With N = 4
    it gives exactly the printed clocks for shift 12 (video) and shift 3
    (audio); this closed form is a fit, not printed on the pages;
  * long video (no decoder or encoder here): the shared boundary is the
    previous chunk's last latent frame itself (the pages re-encode the
    decoded RGB frame); it sits at target position 0 and keeps its value
    (its velocity is not applied, d.n_fixed = 1); the history is every
    earlier frame, of which the block sees the bounded selection
    (compress.history_index); time positions run on across chunks (history
    frame f at f, target frame k at n_hist + k); each chunk carries its own
    audio tokens, with no audio history.
"""
from __future__ import annotations

import numpy as np

from .block import block_forward
from .compress import history_index


def flow_schedule(n_evals: int, shift: float) -> np.ndarray:
    """Clean times t_0..t_N (N = n_evals), fp64."""
    u = np.arange(n_evals + 1, dtype=np.float64) / n_evals
    return u / (u + shift * (1.0 - u))


def flash_layer_flags(n_full_head: int = 2, n_compressed: int = 26, n_full_tail: int = 14) -> np.ndarray:
    """Per layer: 1 if compressed. Default: the Flash 2 / 26 / 14 schedule."""
    return np.asarray([0] * n_full_head + [1] * n_compressed + [0] * n_full_tail, dtype=np.uint8)


def _scatter_ctrl(rows, ctrl_idx, d):
    """Packed control-token rows back into a [Tc, H, W, D] grid (other positions zero)."""
    g = np.zeros((d.n_ctrl * d.H * d.W, d.d_model))
    g[np.asarray(ctrl_idx, dtype=np.int64)] = rows
    return g.reshape(d.n_ctrl, d.H, d.W, d.d_model)


def stack_sample(x_text, x_video, x_audio, layers, flags, t_video, t_audio, d, x_ctrl=None, ctrl_idx=None,
                 store=None):
    """Run len(t_video) - 1 evaluations of the layer stack with Euler updates.

    Every compressed layer is applied literally (gather the kept tokens,
    compute, broadcast the nearest-kept update onto the full features).
    Control frames (x_ctrl, optionally only the tokens at ctrl_idx) are
    re-fed unchanged every evaluation, like text. The first d.n_fixed video
    frames keep their value (no Euler update).
    store: the block's rounding model (tests only; block_core), also applied
    to the updated state as "state".
    Returns the final (x_video, x_audio) in fp64."""
    t_video = np.asarray(t_video, dtype=np.float64)
    t_audio = t_video if t_audio is None else np.asarray(t_audio, dtype=np.float64)
    xt = np.asarray(x_text, dtype=np.float64)
    xv = np.asarray(x_video, dtype=np.float64)
    xa = np.asarray(x_audio, dtype=np.float64)
    for k in range(len(t_video) - 1):
        zt, zv, za, zc = xt, xv, xa, x_ctrl
        first = True
        for w, c in zip(layers, flags):
            if zc is None:
                zt, zv, za = block_forward(zt, zv, za, w, d, compress=bool(c), store=store)
            elif ctrl_idx is None:
                zt, zv, za, zc = block_forward(zt, zv, za, w, d, compress=bool(c), x_ctrl=zc, store=store)
            else:
                # the selected tokens, packed after the first layer
                zin = zc if first else _scatter_ctrl(zc, ctrl_idx, d)
                zt, zv, za, zc = block_forward(zt, zv, za, w, d, compress=bool(c), x_ctrl=zin, ctrl_idx=ctrl_idx,
                                               store=store)
            first = False
        step = (t_video[k + 1] - t_video[k]) * zv
        step[:getattr(d, "n_fixed", 0)] = 0.0
        xv = xv + step
        xa = xa + (t_audio[k + 1] - t_audio[k]) * za
        if store is not None:
            xv, xa = store("state", xv), store("state", xa)
    return xv, xa


def long_video_sample(x_text, first_video, new_video, audio, layers, flags, t_video, t_audio, d, store=None):
    """Chunk-by-chunk long video.

    first_video [T, H, W, D]: noise of the first chunk (no history, every
    frame denoised). new_video: one [T - 1, H, W, D] noise block per later
    chunk. audio: one [n_audio, D] noise block per chunk. d: the chunk's
    block dimensions (T frames per chunk, n_ctrl / ctrl_offset / n_fixed are
    set here). A later chunk is [boundary | new frames]: the boundary is the
    last frame made so far, held fixed; its history is every frame before it,
    read through the bounded selection history_index(n_hist, H, W).
    store: the block's rounding model (tests only; stack_sample).
    Returns (frames [T + (chunks - 1)(T - 1), H, W, D], [audio per chunk])."""
    v, a = stack_sample(x_text, first_video, audio[0], layers, flags, t_video, t_audio,
                        d.with_(n_ctrl=0, ctrl_offset=0, n_fixed=0), store=store)
    frames, audio_out = list(v), [a]
    for noise, an in zip(new_video, audio[1:]):
        n_hist = len(frames) - 1                 # frames before the boundary
        target = np.concatenate([frames[-1][None], np.asarray(noise, dtype=np.float64)])
        dc = d.with_(n_ctrl=n_hist, ctrl_offset=n_hist, n_fixed=1)
        v, a = stack_sample(x_text, target, an, layers, flags, t_video, t_audio, dc,
                            x_ctrl=np.stack(frames[:n_hist]), ctrl_idx=history_index(n_hist, d.H, d.W), store=store)
        frames += list(v[1:])
        audio_out.append(a)
    return np.stack(frames), audio_out
