"""Pins of the oracle's control frames (CPU only).

Control frames sit a fixed positive time offset before the target frames
(tokendh.com article, backbone section; PaperDaily review, section 1). The
pins: with the offset equal to the number of control frames and no audio,
the block with control frames is the plain block over the frames
[control | video] in another token order (the block is permutation
equivariant given the coordinates); moving every time position together
changes nothing when no text is present (rotary logits between rotated
tokens depend on differences only); stride 1 keeps
every token; and the offset does change the result."""
import numpy as np
import pytest

import oracle as O
from dit_synth import BlockDims

from test_oracle_block import rand_inputs

pytestmark = pytest.mark.cpu

CTRL = BlockDims("ctrl", d_model=32, n_heads=2, head_dim=16, d_ffn=48, T=2, H=5, W=6, n_text=3, n_audio=2,
                 rope=(4, 6, 6), dtype="f32", seed=0, n_ctrl=2, ctrl_offset=2)


def ctrl_input(d, seed=5):
    return np.random.default_rng(seed).standard_normal((d.n_ctrl, d.H, d.W, d.d_model))


def test_ctrl_block_is_plain_block_over_control_then_video():
    d = CTRL.with_(n_audio=0)
    x, w = rand_inputs(d)
    xc = ctrl_input(d)
    yt, yv, ya, yc = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False, x_ctrl=xc)
    # plain block: one video of n_ctrl + T frames, control frames first (times 0..Tc-1, then Tc..)
    dp = d.with_(T=d.n_ctrl + d.T, n_ctrl=0, ctrl_offset=0)
    pt, pv, pa = O.block_forward(x["x_text"], np.concatenate([xc, x["x_video"]], axis=0), x["x_audio"], w, dp,
                                 False)
    np.testing.assert_allclose(yt, pt, rtol=0, atol=1e-12)
    np.testing.assert_allclose(yc, pv[:d.n_ctrl], rtol=0, atol=1e-12)
    np.testing.assert_allclose(yv, pv[d.n_ctrl:], rtol=0, atol=1e-12)


@pytest.mark.parametrize("compress", [False, True])
def test_ctrl_block_invariant_to_a_common_time_shift(compress):
    # text tokens do not rotate, so their logits with the rotated tokens do
    # depend on absolute time positions: no text here
    d = CTRL.with_(H=6, W=7, n_text=0)
    x, w = rand_inputs(d)
    xc = ctrl_input(d)
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress, x_ctrl=xc)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress, x_ctrl=xc, t_shift=5)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-10)


def test_ctrl_stride1_equals_uncompressed():
    d = CTRL
    x, w = rand_inputs(d)
    xc = ctrl_input(d)
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False, x_ctrl=xc)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, True, stride=1, x_ctrl=xc)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-12)


def test_ctrl_offset_matters_and_is_required():
    d = CTRL
    x, w = rand_inputs(d)
    xc = ctrl_input(d)
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False, x_ctrl=xc)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d.with_(ctrl_offset=3), False, x_ctrl=xc)
    assert max(np.abs(u - v).max() for u, v in zip(a, b)) > 1e-6
    with pytest.raises(ValueError):
        O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d.with_(ctrl_offset=0), False, x_ctrl=xc)
    with pytest.raises(ValueError):
        O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False)


def test_ctrl_stack_refeeds_control_frames():
    """Zero projections: every block is the identity, so the stack's velocity
    is the state itself whatever the control frames hold."""
    d = CTRL
    x, w = rand_inputs(d, wscale=0.0)
    xc = ctrl_input(d)
    tv = O.flow_schedule(3, 12.0)
    v, a = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], [w, w], [0, 1], tv, None, d, x_ctrl=xc)
    np.testing.assert_allclose(v, x["x_video"] * np.prod(1 + np.diff(tv)), rtol=1e-12)
    np.testing.assert_allclose(a, x["x_audio"] * np.prod(1 + np.diff(tv)), rtol=1e-12)
