"""GPU parity of the block and the sampler with control frames (a fixed
positive time offset before the target frames) against the fp64 oracle, and
the permutation equivalence with the plain block on the GPU itself.

Bars as for the plain block: 1e-4 (fp32), 2e-2 (bf16) on max|err|/RMS; fp8
blocks and the stacks: 1.5 x the case's noise floor (tests/floors.py)."""
import numpy as np
import pytest

import oracle as O
from cases import CTRL_BF16, CTRL_F32, CTRL_FP8, CTRL_STACK, HIST, HIST_STACK, LONG_VIDEO
from dit_synth import round_bf16
from helpers import check_parity, gpu_weights, inputs, oracle_weights, rel_err, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")

CONFIGS = {"bf16": CTRL_BF16, "fp8": CTRL_FP8, "f32": CTRL_F32}


def run_gpu(d, x, w, compress):
    dims = V.make_dims(d)
    xt, xv, xa, xc = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio", "x_ctrl"))
    gw, _ = gpu_weights(w, d.dtype)
    keep = V.keep_index(d.T, d.H, d.W, d.stride) if compress else None
    nk = V.nearest_kept_map(d.T, d.H, d.W, d.stride) if compress else None
    yt, yv, ya, yc = V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk, x_ctrl=xc)
    torch.cuda.synchronize()
    return [to_numpy(yt), to_numpy(yv), to_numpy(ya), to_numpy(yc)]


def check(got, ref, dtype, case=None):
    check_parity(got, ref, dtype, case if dtype == "fp8" else None)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("compress", [False, True])
def test_ctrl_block_vs_oracle(dtype, compress):
    d = CONFIGS[dtype]
    print(f"ctrl block {d.name} compress={compress}", flush=True)
    x, w = inputs(d)
    got = run_gpu(d, x, w, compress)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], oracle_weights(w, dtype), d, compress,
                          x_ctrl=x["x_ctrl"])
    check(got, list(ref), dtype, f"ctrl_fp8_{'on' if compress else 'off'}")


def test_ctrl_block_is_plain_block_over_control_then_video_on_gpu():
    """Offset = number of control frames, no audio: the block with control
    frames equals the plain block on the frames [control | video] (another
    token order of the same sequence and coordinates)."""
    d = CTRL_F32.with_(n_audio=0, n_ctrl=2, ctrl_offset=2)
    x, w = inputs(d)
    yt, yv, ya, yc = run_gpu(d, x, w, False)
    dp = d.with_(T=d.n_ctrl + d.T, n_ctrl=0, ctrl_offset=0)
    dims = V.make_dims(dp)
    xv = torch_act(np.concatenate([x["x_ctrl"], x["x_video"]], axis=0), "f32")
    xt, xa = torch_act(x["x_text"], "f32"), torch_act(x["x_audio"], "f32")
    gw, _ = gpu_weights(w, "f32")
    pt, pv, pa = V.block_forward(dims, xt, xv, xa, gw, False)
    torch.cuda.synchronize()
    pv = to_numpy(pv)
    assert rel_err([yt, yc, yv], [to_numpy(pt), pv[:d.n_ctrl], pv[d.n_ctrl:]]) <= 1e-5


def test_ctrl_stack_vs_oracle():
    d = CTRL_STACK
    flags = [0, 1, 1, 0]
    tv, ta = O.flow_schedule(3, 12.0), O.flow_schedule(3, 3.0)
    print(f"ctrl stack flags={flags}", flush=True)
    x, _ = inputs(d)
    layers = [inputs(d, layer=l)[1] for l in range(len(flags))]
    dims = V.make_dims(d)
    xt, xv, xa, xc = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio", "x_ctrl"))
    gl = [gpu_weights(lw, d.dtype)[0] for lw in layers]
    keep, nk = V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W)
    xc0 = to_numpy(xc).copy()
    V.stack_sample(dims, gl, flags, tv, ta, xt, xv, xa, keep, nk, x_ctrl=xc)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(xc), xc0)   # control frames are inputs only
    ref = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], [oracle_weights(lw, "bf16") for lw in layers], flags,
                         tv.astype(np.float32), ta.astype(np.float32), d, x_ctrl=x["x_ctrl"])
    check_parity([to_numpy(xv), to_numpy(xa)], list(ref), "bf16", "ctrl_stack_bf16")


# ---------------------------------------------------------------- bounded long-video history
@pytest.mark.parametrize("n_hist,H,W", [(0, 4, 4), (1, 9, 15), (3, 9, 15), (12, 9, 15), (25, 34, 60), (40, 5, 7)])
def test_history_index_bit_exact(n_hist, H, W):
    got = V.history_index(n_hist, H, W)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.history_index(n_hist, H, W))


def run_gpu_hist(d, x, w, compress):
    dims = V.make_dims(d)
    xt, xv, xa, xc = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio", "x_ctrl"))
    gw, _ = gpu_weights(w, d.dtype)
    keep = V.keep_index(d.T, d.H, d.W, d.stride) if compress else None
    nk = V.nearest_kept_map(d.T, d.H, d.W, d.stride) if compress else None
    idx = V.history_index(d.n_ctrl, d.H, d.W)
    yt, yv, ya, yc = V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk, x_ctrl=xc, ctrl_idx=idx)
    torch.cuda.synchronize()
    return [to_numpy(yt), to_numpy(yv), to_numpy(ya), to_numpy(yc)]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("compress", [False, True])
def test_history_block_vs_oracle(dtype, compress):
    """A chunk of 2 frames after 12 history frames (first full, 8 at stride 4,
    2 at stride 2), the history tokens read through their position list."""
    d = HIST.with_(dtype=dtype)
    print(f"history block {dtype} compress={compress}", flush=True)
    x, w = inputs(d)
    got = run_gpu_hist(d, x, w, compress)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], oracle_weights(w, dtype), d, compress,
                          x_ctrl=x["x_ctrl"], ctrl_idx=O.history_index(d.n_ctrl, d.H, d.W))
    check(got, list(ref), dtype, f"hist_fp8_{'on' if compress else 'off'}")


def test_history_stack_vs_oracle():
    d = HIST_STACK
    flags = [0, 1, 0]
    tv = O.flow_schedule(3, 12.0)
    print(f"history stack flags={flags}", flush=True)
    x, _ = inputs(d)
    layers = [inputs(d, layer=l)[1] for l in range(len(flags))]
    dims = V.make_dims(d)
    xt, xv, xa, xc = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio", "x_ctrl"))
    gl = [gpu_weights(lw, d.dtype)[0] for lw in layers]
    keep, nk = V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W)
    idx = V.history_index(d.n_ctrl, d.H, d.W)
    V.stack_sample(dims, gl, flags, tv, None, xt, xv, xa, keep, nk, x_ctrl=xc, ctrl_idx=idx)
    torch.cuda.synchronize()
    ref = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], [oracle_weights(lw, "bf16") for lw in layers], flags,
                         tv.astype(np.float32), None, d, x_ctrl=x["x_ctrl"],
                         ctrl_idx=O.history_index(d.n_ctrl, d.H, d.W))
    check_parity([to_numpy(xv), to_numpy(xa)], list(ref), "bf16", "hist_stack_bf16")


# ---------------------------------------------------------------- chunk-by-chunk long video
def test_long_video_vs_oracle():
    """5 chunks of 3 frames (the first; then a boundary frame held fixed and
    2 new frames, with up to 8 history frames read through the bounded
    selection), 4 layers (2 compressed), 3 evaluations."""
    d = LONG_VIDEO
    flags = [0, 1, 1, 0]
    tv, ta = O.flow_schedule(3, 12.0), O.flow_schedule(3, 3.0)
    x, _ = inputs(d)
    layers = [inputs(d, layer=l)[1] for l in range(len(flags))]
    g = np.random.default_rng(99)
    first = x["x_video"]
    new = [round_bf16(g.standard_normal((d.T - 1, d.H, d.W, d.d_model)).astype(np.float32)) for _ in range(4)]
    audio = [x["x_audio"]] + [round_bf16(g.standard_normal((d.n_audio, d.d_model)).astype(np.float32))
                              for _ in range(4)]
    print("long video: 5 chunks", flush=True)
    dims = V.make_dims(d)
    gl = [gpu_weights(lw, d.dtype)[0] for lw in layers]
    keep, nk = V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W)
    xt = torch_act(x["x_text"], d.dtype)
    ga = [torch_act(a, d.dtype) for a in audio]
    frames = V.long_video_sample(dims, gl, flags, tv, ta, xt, torch_act(first, d.dtype),
                                 [torch_act(n, d.dtype) for n in new], ga, keep, nk)
    # the first chunk alone gives the same first frames, boundary included (later chunks hold it fixed)
    f0, a0 = torch_act(first, d.dtype), torch_act(audio[0], d.dtype)
    V.stack_sample(dims, gl, flags, tv, ta, xt, f0, a0, keep, nk)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(frames[:d.T]), to_numpy(f0))
    ref_f, ref_a = O.long_video_sample(x["x_text"], first, new, audio, [oracle_weights(lw, "bf16") for lw in layers],
                                       flags, tv.astype(np.float32), ta.astype(np.float32), d)
    check_parity([to_numpy(frames)] + [to_numpy(a) for a in ga], [ref_f] + list(ref_a), "bf16", "long_video_bf16")
    # the library's chunk loop equals the chunks composed from dit_stack_sample_ctrl calls, bit for bit
    T = d.T
    fr = torch.empty_like(frames)
    fr[:T].copy_(torch_act(first, d.dtype))
    for c, n in enumerate(new):
        fr[T + c * (T - 1):T + (c + 1) * (T - 1)].copy_(torch_act(n, d.dtype))
    ca = [torch_act(a, d.dtype) for a in audio]
    V.stack_sample(dims, gl, flags, tv, ta, xt, fr[:T], ca[0], keep, nk)
    for c in range(1, len(audio)):
        n_hist = T + (c - 1) * (T - 1) - 1
        dc = V.make_dims(d)
        dc.n_ctrl, dc.ctrl_offset, dc.n_fixed = n_hist, n_hist, 1
        V.stack_sample(dc, gl, flags, tv, ta, xt, fr[n_hist:n_hist + T], ca[c], keep, nk, x_ctrl=fr[:n_hist],
                       ctrl_idx=V.history_index(n_hist, d.H, d.W))
    torch.cuda.synchronize()
    assert torch.equal(fr, frames)
    assert all(torch.equal(a, b) for a, b in zip(ca, ga))
