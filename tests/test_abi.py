"""CPU checks of the C ABI: the library loads, exports every symbol declared in
include/vdtflash.h, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdtflash.h")

V = pytest.importorskip("video_diffusion_transformer_flash_amd")
from video_diffusion_transformer_flash_amd import _lib  # noqa: E402
from dit_synth import CONFIGS  # noqa: E402


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = V.lib()
    names = declared_symbols()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_keep_dims_matches_oracle():
    for s in (1, 2, 3, 4):
        for H in range(1, 40):
            for W in (1, 2, 7, 60):
                assert V.keep_dims(H, W, s) == O.keep_dims(H, W, s)


def _dims(**kw):
    d = V.make_dims(CONFIGS["540p_on"])
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), _lib.DIT_EUNSUPPORTED),
    (dict(rope_t=30), _lib.DIT_EINVAL),
    (dict(rope_t=31, rope_h=49), _lib.DIT_EINVAL),
    (dict(d_model=5377), _lib.DIT_EINVAL),
    (dict(T=0), _lib.DIT_EINVAL),
    (dict(stride=0), _lib.DIT_EINVAL),
    (dict(act_dtype=_lib.DIT_F32), _lib.DIT_EUNSUPPORTED),       # f32 activations with bf16 weights
    (dict(w_dtype=7), _lib.DIT_EUNSUPPORTED),
    (dict(d_model=5376 + 64), _lib.DIT_EUNSUPPORTED),          # bf16 path wants multiples of 128
    (dict(n_ctrl=1, ctrl_offset=0), _lib.DIT_EINVAL),          # control frames need a positive offset
    (dict(n_ctrl=-1), _lib.DIT_EINVAL),
    (dict(ctrl_offset=-2), _lib.DIT_EINVAL),
    (dict(n_fixed=-1), _lib.DIT_EINVAL),
    (dict(n_fixed=7), _lib.DIT_EINVAL),                          # more fixed frames than T = 6
    (dict(T=8, H=1024, W=1025), _lib.DIT_EUNSUPPORTED),         # past 2^23 tokens on the MFMA path
    (dict(T=1024, H=1024, W=1025), _lib.DIT_EINVAL),            # past 2^30 tokens
])
def test_dims_rejected(bad, code):
    n = ctypes.c_size_t()
    assert V.lib().dit_block_workspace_size(ctypes.byref(_dims(**bad)), 1, ctypes.byref(n)) == code


def test_token_bound_is_the_mfma_paths_only():
    """2^23 + tokens: refused on the bf16 path, accepted by the f32 path."""
    n = ctypes.c_size_t()
    big = dict(T=8, H=1024, W=1025)
    assert V.lib().dit_block_workspace_size(ctypes.byref(_dims(**big)), 0, ctypes.byref(n)) == _lib.DIT_EUNSUPPORTED
    f32 = _dims(act_dtype=_lib.DIT_F32, w_dtype=_lib.DIT_F32, **big)
    assert V.lib().dit_block_workspace_size(ctypes.byref(f32), 0, ctypes.byref(n)) == _lib.DIT_OK
    assert n.value > 0


def test_block_forward_rejects_before_launch():
    lib = V.lib()
    d = _dims()
    w = _lib.BlockWeights()
    # null weights / inputs: EINVAL, nothing launched (no GPU needed)
    st = lib.dit_block_forward(ctypes.byref(d), None, None, None, ctypes.byref(w), 1, None, None, None, None, None,
                               None, 0, None)
    assert st == _lib.DIT_EINVAL
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    wf = _lib.BlockWeights(*([fake] * 7))
    # compressed without keep / nk
    st = lib.dit_block_forward(ctypes.byref(d), fake, fake, fake, ctypes.byref(wf), 1, None, None, fake, fake, fake,
                               ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL
    # workspace too small
    st = lib.dit_block_forward(ctypes.byref(d), fake, fake, fake, ctypes.byref(wf), 1, fake, fake, fake, fake, fake,
                               ws, 1024, None)
    assert st == _lib.DIT_EWORKSPACE
    # misaligned input pointer
    st = lib.dit_block_forward(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 8), fake, fake, ctypes.byref(wf), 0,
                               None, None, fake, fake, fake, ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL


def test_other_entry_points_reject():
    lib = V.lib()
    assert lib.dit_keep_index(0, 4, 4, 2, ctypes.c_void_p(1 << 20), None) == _lib.DIT_EINVAL
    assert lib.dit_nearest_kept_map(1, 4, 4, 0, ctypes.c_void_p(1 << 20), None) == _lib.DIT_EINVAL
    assert lib.dit_keep_index(1, 4, 4, 2, None, None) == _lib.DIT_EINVAL
    assert lib.dit_quantize_fp8(None, 0, 16, None, None, None) == _lib.DIT_EINVAL
    assert lib.dit_quantize_fp8(ctypes.c_void_p(1 << 20), 2, 16, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20),
                                None) == _lib.DIT_EUNSUPPORTED
    assert lib.dit_broadcast_residual(4, 0, 64, 1, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), 0,
                                      ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None) == _lib.DIT_EINVAL
    assert lib.dit_broadcast_residual(4, 2, 64, 1, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), 2,
                                      ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None) == _lib.DIT_EUNSUPPORTED
    n = ctypes.c_size_t()
    assert lib.dit_attention_workspace_size(10, 2, 96, 1, ctypes.byref(n)) == _lib.DIT_EUNSUPPORTED
    d = _dims()
    assert lib.dit_stack_sample(ctypes.byref(d), None, 3, None, 1, None, None, None, None, None, None, None, None, 0,
                                None) == _lib.DIT_EINVAL
    assert lib.dit_status_str(_lib.DIT_EWORKSPACE) == b"workspace too small"


def test_workspace_grows_with_sequence():
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    d = _dims()
    V.lib().dit_block_workspace_size(ctypes.byref(d), 1, ctypes.byref(a))
    V.lib().dit_block_workspace_size(ctypes.byref(d), 0, ctypes.byref(b))
    assert 0 < a.value < b.value


def test_control_frame_entry_points_reject():
    """The plain calls refuse dims with control frames, the *_ctrl calls dims
    without them; a control workspace covers the extra rows."""
    lib = V.lib()
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    wf = _lib.BlockWeights(*([fake] * 7))
    dc = _dims(n_ctrl=2, ctrl_offset=3)
    st = lib.dit_block_forward(ctypes.byref(dc), fake, fake, fake, ctypes.byref(wf), 0, None, None, fake, fake, fake,
                               ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL
    d0 = _dims()
    st = lib.dit_block_forward_ctrl(ctypes.byref(d0), fake, fake, fake, None, 0, fake, ctypes.byref(wf), 0, None,
                                    None, fake, fake, fake, fake, ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL
    # missing control pointers
    st = lib.dit_block_forward_ctrl(ctypes.byref(dc), fake, fake, None, None, 0, fake, ctypes.byref(wf), 0, None,
                                    None, fake, fake, None, fake, ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL
    # a token list longer than the control grid
    st = lib.dit_block_forward_ctrl(ctypes.byref(dc), fake, fake, fake, fake, 2 * 34 * 60 + 1, fake,
                                    ctypes.byref(wf), 0, None, None, fake, fake, fake, fake, ws, 1 << 40, None)
    assert st == _lib.DIT_EINVAL
    assert lib.dit_stack_sample(ctypes.byref(dc), None, 0, None, 1, None, None, fake, fake, fake, None, None, ws,
                                1 << 40, None) == _lib.DIT_EINVAL
    assert lib.dit_stack_sample_ctrl(ctypes.byref(d0), None, 0, None, 1, None, None, fake, fake, fake, None, 0, fake,
                                     None, None, ws, 1 << 40, None) == _lib.DIT_EINVAL
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    lib.dit_block_workspace_size(ctypes.byref(d0), 1, ctypes.byref(a))
    lib.dit_block_workspace_size(ctypes.byref(dc), 1, ctypes.byref(b))
    assert b.value > a.value


def test_history_count_matches_oracle():
    lib = V.lib()
    n = ctypes.c_int32()
    for nh in (0, 1, 2, 3, 4, 11, 12, 25):
        for H, W in ((8, 12), (34, 60), (5, 7)):
            assert lib.dit_history_count(nh, H, W, ctypes.byref(n)) == _lib.DIT_OK
            assert n.value == len(O.history_index(nh, H, W))
    assert lib.dit_history_count(-1, 4, 4, ctypes.byref(n)) == _lib.DIT_EINVAL
    assert lib.dit_history_index(3, 0, 4, None, None) == _lib.DIT_EINVAL


def test_long_video_workspace_and_refusals():
    """The long-video workspace covers the history index list and the largest
    chunk's stack workspace sized for its history tokens (far below a stack
    sized for every earlier position); bad arguments are refused on the host."""
    lib = V.lib()
    d = _dims(T=6)
    fl = (ctypes.c_uint8 * 4)(0, 1, 1, 0)
    flp = ctypes.cast(fl, ctypes.c_void_p)
    n = ctypes.c_size_t()
    assert lib.dit_long_video_workspace_size(ctypes.byref(d), flp, 4, 1, ctypes.byref(n)) == _lib.DIT_OK
    one = n.value
    s0 = ctypes.c_size_t()
    assert lib.dit_stack_workspace_size(ctypes.byref(d), flp, 4, ctypes.byref(s0)) == _lib.DIT_OK
    assert one == s0.value
    assert lib.dit_long_video_workspace_size(ctypes.byref(d), flp, 4, 5, ctypes.byref(n)) == _lib.DIT_OK
    five = n.value
    # the last chunk has 6 + 3 * 5 - 1 = 20 earlier frames; its history keeps frame 0, two frames at
    # stride 2 and eight at stride 4
    cnt = ctypes.c_int32()
    lib.dit_history_count(20, d.H, d.W, ctypes.byref(cnt))
    assert cnt.value == len(O.history_index(20, d.H, d.W))
    full = ctypes.c_size_t()
    dl = _dims(T=6, n_ctrl=20, ctrl_offset=20, n_fixed=1)
    lib.dit_stack_workspace_size(ctypes.byref(dl), flp, 4, ctypes.byref(full))
    assert one < five < full.value
    es = 2
    grow_tokens = (five - one) / (d.d_model * es)
    assert grow_tokens >= 2 * cnt.value    # the full-resolution and the packed state both hold the history rows
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    wf = (_lib.BlockWeights * 4)(*[_lib.BlockWeights(*([fake] * 7)) for _ in range(4)])
    tv = (ctypes.c_float * 4)(1.0, 0.6, 0.3, 0.0)
    tvp = ctypes.cast(tv, ctypes.c_void_p)
    call = lambda dd, chunks, frames, wsb: lib.dit_long_video_sample(  # noqa: E731
        ctypes.byref(dd), wf, 4, flp, 3, tvp, None, fake, chunks, frames, fake, fake, fake, ws, wsb, None)
    assert call(d, 0, fake, 1 << 40) == _lib.DIT_EINVAL                        # no chunks
    assert call(_dims(T=1), 2, fake, 1 << 40) == _lib.DIT_EINVAL               # a later chunk needs T >= 2
    assert call(_dims(T=6, n_ctrl=1, ctrl_offset=1), 2, fake, 1 << 40) == _lib.DIT_EINVAL
    assert call(_dims(T=6, n_fixed=1), 2, fake, 1 << 40) == _lib.DIT_EINVAL
    assert call(d, 5, None, 1 << 40) == _lib.DIT_EINVAL                        # no frames
    assert call(d, 5, fake, five - 256) == _lib.DIT_EWORKSPACE
