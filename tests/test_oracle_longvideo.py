"""Pins of the oracle's chunk-by-chunk long video (CPU only).

The pages (tokendh.com article, long-video section; PaperDaily review,
section 3) generate a long video chunk by chunk: the last frame of a chunk is
the fixed first frame of the next, which adds new frames with the bounded
history of the earlier frames as context. Pins: identity blocks give the
closed form of the Euler steps on every new frame and leave each boundary
frame untouched; a later chunk depends on the earlier frames only through the
history selection; held-fixed frames keep their value in the sampler."""
import numpy as np
import pytest

import oracle as O
from dit_synth import BlockDims

from test_oracle_block import rand_inputs

pytestmark = pytest.mark.cpu

D = BlockDims("long", d_model=32, n_heads=2, head_dim=16, d_ffn=48, T=3, H=4, W=5, n_text=3, n_audio=2,
              rope=(4, 6, 6), dtype="f32", seed=0)


def noise(d, n_chunks, seed=1):
    g = np.random.default_rng(seed)
    first = g.standard_normal((d.T, d.H, d.W, d.d_model))
    new = [g.standard_normal((d.T - 1, d.H, d.W, d.d_model)) for _ in range(n_chunks - 1)]
    audio = [g.standard_normal((d.n_audio, d.d_model)) for _ in range(n_chunks)]
    return first, new, audio


def test_identity_blocks_closed_form():
    """Zero projections: every block is the identity and the velocity is the
    state, so a denoised frame is its noise times prod(1 + dt); a boundary
    frame passes through its chunk unchanged."""
    d = D
    x, w = rand_inputs(d, wscale=0.0)
    tv, ta = O.flow_schedule(3, 12.0), O.flow_schedule(3, 3.0)
    first, new, audio = noise(d, 4)
    frames, aud = O.long_video_sample(x["x_text"], first, new, audio, [w, w], [0, 1], tv, ta, d)
    gv, ga = np.prod(1 + np.diff(tv)), np.prod(1 + np.diff(ta))
    assert frames.shape == (d.T + 3 * (d.T - 1), d.H, d.W, d.d_model)
    np.testing.assert_allclose(frames[:d.T], first * gv, rtol=1e-12)
    for c, nz in enumerate(new):
        s = d.T + c * (d.T - 1)
        np.testing.assert_allclose(frames[s:s + d.T - 1], nz * gv, rtol=1e-12)
    for a, an in zip(aud, audio):
        np.testing.assert_allclose(a, an * ga, rtol=1e-12)


def test_fixed_frames_keep_their_value():
    # one evaluation: both runs start from the same state, so the frames that
    # are not held move identically (over more evaluations the held frames'
    # values feed back through attention)
    d = D.with_(n_fixed=2)
    x, w = rand_inputs(d)
    tv = O.flow_schedule(1, 12.0)
    v, a = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], [w], [1], tv, None, d)
    np.testing.assert_array_equal(v[:2], x["x_video"][:2])
    assert np.abs(v[2] - x["x_video"][2]).max() > 1e-6
    v0, a0 = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], [w], [1], tv, None, d.with_(n_fixed=0))
    np.testing.assert_allclose(v[2:], v0[2:], rtol=0, atol=1e-12)   # the others are unaffected
    np.testing.assert_allclose(a, a0, rtol=0, atol=1e-12)


def test_later_chunk_sees_only_the_history_selection():
    """14 chunks of 1 new frame: the last chunk has 13 history frames, of
    which frames 1 and 2 are no longer selected. Re-running it with those
    frames replaced gives the same result; replacing a selected frame does
    not."""
    d = D.with_(T=2)
    x, w = rand_inputs(d, seed=3)
    tv = O.flow_schedule(2, 12.0)
    first, new, audio = noise(d, 14, seed=4)
    frames, aud = O.long_video_sample(x["x_text"], first, new, audio, [w], [1], tv, None, d)
    n_hist = len(frames) - 2
    assert n_hist == 13 and set(range(n_hist)) - {f for f, _ in O.history_frames(n_hist)} == {1, 2}
    target = np.concatenate([frames[n_hist][None], new[-1]])
    dc = d.with_(n_ctrl=n_hist, ctrl_offset=n_hist, n_fixed=1)
    idx = O.history_index(n_hist, d.H, d.W)

    def last_chunk(hist):
        return O.stack_sample(x["x_text"], target, audio[-1], [w], [1], tv, None, dc, x_ctrl=hist, ctrl_idx=idx)

    hist = frames[:n_hist].copy()
    v, a = last_chunk(hist)
    np.testing.assert_allclose(v[1:], frames[n_hist + 1:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a, aud[-1], rtol=0, atol=1e-12)
    hist[1:3] = np.random.default_rng(5).standard_normal(hist[1:3].shape)
    v2, _ = last_chunk(hist)
    np.testing.assert_allclose(v2, v, rtol=0, atol=1e-12)
    hist[0] += 1.0
    v3, _ = last_chunk(hist)
    assert np.abs(v3[1:] - v[1:]).max() > 1e-6
