"""dit_block_forward_noalloc (the block on the library's static per-device
scratch array, for callers that cannot allocate) against dit_block_forward
(caller workspace): bit-identical outputs on calls in a row, each later call
on a smaller input (the scratch keeps the earlier call's contents); a block
whose workspace exceeds the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest

from cases import SMALL_FP8
from dit_synth import CONFIGS
from helpers import gpu_weights, inputs, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")
from video_diffusion_transformer_flash_amd import _lib  # noqa: E402


def run_both(d, compress):
    x, w = inputs(d)
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gw, _ = gpu_weights(w, d.dtype)
    keep = V.keep_index(d.T, d.H, d.W) if compress else None
    nk = V.nearest_kept_map(d.T, d.H, d.W) if compress else None
    a = V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk)
    b = V.block_forward_noalloc(dims, xt, xv, xa, gw, compress, keep, nk)
    torch.cuda.synchronize()
    return [to_numpy(t) for t in a], [to_numpy(t) for t in b]


def test_noalloc_equals_block_forward_on_shrinking_calls():
    # full width, 294 tokens uncompressed: 101 MiB of the 128 MiB scratch,
    # with the K-split tail of the O and down projections; then smaller ones
    cases = [(CONFIGS["540p_off"].with_(name="full_width_294", T=2, H=9, W=15, n_text=16, n_audio=8), False),
             (SMALL_FP8, False),
             (SMALL_FP8.with_(T=1, H=5, W=7, n_text=3, n_audio=2), True)]
    for d, compress in cases:
        print(f"noalloc {d.name} {d.T}x{d.H}x{d.W} compress={compress}", flush=True)
        a, b = run_both(d, compress)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_noalloc_refuses_past_the_scratch():
    d = CONFIGS["540p_on"]
    dims = V.make_dims(d)
    need = V.block_workspace_size(dims, True)
    assert need > 128 << 20
    fake = ctypes.c_void_p(1 << 20)
    w = _lib.BlockWeights(*([fake] * 7))
    st = V.lib().dit_block_forward_noalloc(ctypes.byref(dims), fake, fake, fake, ctypes.byref(w), 1, fake, fake, fake,
                                          fake, fake, None)
    assert st == _lib.DIT_EWORKSPACE
