"""GPU parity of dit_stack_sample (flow-matching Euler sampler over a stack of
blocks with compressed spans) against the oracle, which applies every
compressed layer literally (per-layer gather and broadcast)."""
import numpy as np
import pytest

import oracle as O
from dit_synth import BlockDims
from helpers import FP8_MAX_BOUND, gpu_weights, inputs, oracle_weights, rel_err, rms_err, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")

SMALL = BlockDims("stack_small", d_model=256, n_heads=2, head_dim=128, d_ffn=512, T=2, H=9, W=15, n_text=16,
                  n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=7)
# stack bars: 6e-2 for the bf16-residual stacks (fp8 or bf16 projections; the
# bf16 residual stream is rounded after every block), 1e-4 for fp32
TOL = {"bf16": 6e-2, "fp8": 6e-2, "f32": 1e-4}
WIDE = BlockDims("stack_wide", d_model=5376, n_heads=56, head_dim=128, d_ffn=14336, T=2, H=6, W=10, n_text=16,
                 n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=9)


def run(d, flags, tv, ta, n_layers_seed=0):
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


@pytest.mark.parametrize("dtype", ["fp8", "bf16", "f32"])
def test_stack_vs_oracle(dtype):
    d = SMALL.with_(dtype=dtype, d_ffn=512 if dtype != "f32" else 704)
    if dtype == "f32":
        d = d.with_(head_dim=64, n_heads=4, rope=(16, 24, 24))
    flags = [0, 1, 1, 1, 0, 1]
    tv = O.flow_schedule(3, 12.0)
    ta = O.flow_schedule(3, 3.0)
    print(f"stack {dtype} flags={flags}", flush=True)
    x, layers, got = run(d, flags, tv, ta)
    ow = [oracle_weights(w, dtype) for w in layers]
    ref = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], ow, flags, tv.astype(np.float32),
                         ta.astype(np.float32), d)
    check(got, ref, dtype)


def check(got, ref, dtype):
    err = rel_err(list(got), list(ref))
    rerr = rms_err(list(got), list(ref))
    print(f"  max|err|/rms = {err:.3e}, rms err = {rerr:.3e}")
    if dtype == "fp8":
        assert rerr <= TOL["fp8"] and err <= FP8_MAX_BOUND
    else:
        assert err <= TOL[dtype]


def test_stack_wide_fp8():
    """Full Flash width, 4 layers (full, compressed, compressed, full), 3 evaluations."""
    d = WIDE
    flags = [0, 1, 1, 0]
    tv = O.flow_schedule(3, 12.0)
    print(f"stack wide fp8 flags={flags}", flush=True)
    x, layers, got = run(d, flags, tv, None)
    ow = [oracle_weights(w, "fp8") for w in layers]
    ref = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], ow, flags, tv.astype(np.float32), None, d)
    check(got, ref, "fp8")


def test_stack_zero_evals_and_layers():
    d = SMALL.with_(dtype="bf16")
    x, _ = inputs(d)
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    v0, a0 = to_numpy(xv), to_numpy(xa)
    V.stack_sample(dims, [], [], [0.0], None, xt, xv, xa)
    assert np.array_equal(to_numpy(xv), v0) and np.array_equal(to_numpy(xa), a0)
    # no layers: the velocity is the state itself -> x * (1 + dt), rounded to bf16
    V.stack_sample(dims, [], [], [0.0, 0.5], None, xt, xv, xa)
    assert np.max(np.abs(to_numpy(xv) - 1.5 * v0)) <= 1.5 * np.abs(v0).max() * 2 ** -8
