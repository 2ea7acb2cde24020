"""Pins of the bounded long-video history (CPU only): the properties the pages
state for it (tokendh.com article, long-video section; PaperDaily review,
section 3) and the block's handling of a selected token list."""
import numpy as np
import pytest

import oracle as O
from dit_synth import BlockDims

from test_oracle_block import rand_inputs

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("n", range(0, 40))
def test_history_frames_properties(n):
    fr = O.history_frames(n)
    frames = [f for f, _ in fr]
    assert frames == sorted(set(frames)) and all(0 <= f < n for f in frames)
    if n == 0:
        assert fr == []
        return
    assert fr[0] == (0, 1)                                   # the first frame, full resolution
    strides = dict(fr)
    assert [strides[f] for f in range(max(1, n - 2), n)] == [2] * len(range(max(1, n - 2), n))  # two most recent
    s4 = [f for f, s in fr if s == 4]
    assert len(s4) <= 8 and s4 == list(range(n - 2 - len(s4), n - 2))   # contiguous, right before the recent two
    assert len(s4) == min(8, max(0, n - 3))                  # as many as exist, up to eight
    dropped = set(range(n)) - set(frames)
    assert dropped == set(range(1, max(1, n - 10)))          # only middle frames are ever dropped


@pytest.mark.parametrize("H,W", [(8, 12), (32, 60), (48, 84)])
def test_history_budget_is_two_frames(H, W):
    """H, W multiples of 4: never more than two full frames of tokens, exactly
    two once the history is full, whatever its length."""
    counts = [len(O.history_index(n, H, W)) for n in range(0, 60)]
    assert max(counts) == 2 * H * W
    assert all(c == 2 * H * W for c in counts[11:])


def test_history_index_positions():
    H, W = 10, 13
    idx = O.history_index(15, H, W)
    assert len(idx) == len(set(idx.tolist())) and idx.min() >= 0 and idx.max() < 15 * H * W
    f, rem = idx // (H * W), idx % (H * W)
    h, w = rem // W, rem % W
    st = dict(O.history_frames(15))
    for fi, hi, wi in zip(f, h, w):
        s = st[int(fi)]
        assert hi % s == 0 and wi % s == 0
    for fr, s in O.history_frames(15):
        assert (f == fr).sum() == len(range(0, H, s)) * len(range(0, W, s))
    assert np.all(np.diff(idx) > 0)                          # frame by frame, raster order


CTRL = BlockDims("hist", d_model=32, n_heads=2, head_dim=16, d_ffn=48, T=2, H=8, W=8, n_text=3, n_audio=2,
                 rope=(4, 6, 6), dtype="f32", seed=0, n_ctrl=5, ctrl_offset=5)


def test_block_with_all_control_tokens_listed_equals_whole_frames():
    d = CTRL
    x, w = rand_inputs(d)
    xc = np.random.default_rng(3).standard_normal((d.n_ctrl, d.H, d.W, d.d_model))
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False, x_ctrl=xc)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, False, x_ctrl=xc,
                        ctrl_idx=np.arange(d.n_ctrl * d.H * d.W))
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[3].reshape(-1, d.d_model), b[3], rtol=0, atol=1e-12)


@pytest.mark.parametrize("compress", [False, True])
def test_history_tokens_carry_their_coordinates(compress):
    """Listing the history tokens in another order permutes their outputs and
    leaves every other output unchanged (coordinates travel with the rows)."""
    d = CTRL
    x, w = rand_inputs(d)
    xc = np.random.default_rng(4).standard_normal((d.n_ctrl, d.H, d.W, d.d_model))
    idx = O.history_index(d.n_ctrl, d.H, d.W)
    perm = np.random.default_rng(5).permutation(len(idx))
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress, x_ctrl=xc, ctrl_idx=idx)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress, x_ctrl=xc, ctrl_idx=idx[perm])
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[3][perm], b[3], rtol=0, atol=1e-12)
    # and the history does reach the outputs
    c = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress, x_ctrl=2 * xc, ctrl_idx=idx)
    assert np.abs(a[1] - c[1]).max() > 1e-6
