"""GPU parity of dit_stack_sample (flow-matching Euler sampler over a stack of
blocks with compressed spans) against the oracle, which applies every
compressed layer literally (per-layer gather and broadcast).

Bars: fp32 1e-4 on max|err|/RMS; bf16 and fp8 stacks (a bf16 state rounded
after every block and every Euler step; fp8: e4m3 codes): 1.5 x the case's
noise floor on max|err|/RMS and on the RMS error (tests/floors.py)."""
import numpy as np
import pytest

import oracle as O
from cases import FLASH42, STACK_FLAGS, STACK_SMALL, STACK_WIDE, STACK_WIDE_FLAGS
from helpers import check_parity, gpu_weights, inputs, oracle_weights, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")


def run(d, flags, tv, ta):
    x, _ = inputs(d)
    layers = [inputs(d, layer=l)[1] for l in range(len(flags))]
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gl = [gpu_weights(w, d.dtype)[0] for w in layers]
    keep = V.keep_index(d.T, d.H, d.W)
    nk = V.nearest_kept_map(d.T, d.H, d.W)
    V.stack_sample(dims, gl, flags, tv, ta, xt, xv, xa, keep, nk)
    torch.cuda.synchronize()
    return x, layers, (to_numpy(xv), to_numpy(xa))


def oracle_stack(d, x, layers, flags, tv, ta):
    ow = [oracle_weights(w, d.dtype) for w in layers]
    return O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], ow, flags, tv, ta, d)


@pytest.mark.parametrize("dtype", ["fp8", "bf16", "f32"])
def test_stack_vs_oracle(dtype):
    d = STACK_SMALL.with_(dtype=dtype, d_ffn=512 if dtype != "f32" else 704)
    if dtype == "f32":
        d = d.with_(head_dim=64, n_heads=4, rope=(16, 24, 24))
    flags = STACK_FLAGS
    tv = O.flow_schedule(3, 12.0).astype(np.float32)
    ta = O.flow_schedule(3, 3.0).astype(np.float32)
    print(f"stack {dtype} flags={flags}", flush=True)
    x, layers, got = run(d, flags, tv, ta)
    ref = oracle_stack(d, x, layers, flags, tv, ta)
    check_parity(list(got), list(ref), dtype, None if dtype == "f32" else f"stack_small_{dtype}")


def test_stack_wide_fp8():
    """Full Flash width, 4 layers (full, compressed, compressed, full), 3 evaluations."""
    d = STACK_WIDE
    tv = O.flow_schedule(3, 12.0).astype(np.float32)
    print(f"stack wide fp8 flags={STACK_WIDE_FLAGS}", flush=True)
    x, layers, got = run(d, STACK_WIDE_FLAGS, tv, None)
    ref = oracle_stack(d, x, layers, STACK_WIDE_FLAGS, tv, None)
    check_parity(list(got), list(ref), "fp8", "stack_wide_fp8")


def test_flash42_fp8_stack():
    """The Flash schedule: 42 layers (2 full, 26 compressed, 14 full), 3
    evaluations, fp8 projections, at width 1024 on a 2 x 16 x 30 grid; every
    element of the final video and audio state."""
    d = FLASH42
    flags = list(O.flash_layer_flags())
    assert len(flags) == 42 and sum(flags) == 26 and flags[:2] == [0, 0] and flags[-14:] == [0] * 14
    tv = O.flow_schedule(3, 12.0).astype(np.float32)
    print("flash42 fp8 stack", flush=True)
    x, layers, got = run(d, flags, tv, None)
    ref = oracle_stack(d, x, layers, flags, tv, None)
    check_parity(list(got), list(ref), "fp8", "flash42_fp8")


def test_stack_zero_evals_and_layers():
    d = STACK_SMALL.with_(dtype="bf16")
    x, _ = inputs(d)
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    v0, a0 = to_numpy(xv), to_numpy(xa)
    V.stack_sample(dims, [], [], [0.0], None, xt, xv, xa)
    assert np.array_equal(to_numpy(xv), v0) and np.array_equal(to_numpy(xa), a0)
    # no layers: the velocity is the state itself -> x * (1 + dt), rounded to bf16
    V.stack_sample(dims, [], [], [0.0, 0.5], None, xt, xv, xa)
    assert np.max(np.abs(to_numpy(xv) - 1.5 * v0)) <= 1.5 * np.abs(v0).max() * 2 ** -8
