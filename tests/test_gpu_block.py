"""GPU parity of dit_block_forward against the fp64 oracle.

Metric: max |gpu - oracle| over every output element / RMS of the oracle
outputs. Bars: 1e-4 for the fp32 block, 2e-2 for bf16; fp8 projections: 6e-2
on the RMS error, the max error within the e4m3 code-flip bound (helpers.py). Small configurations compare every element; the full
540p / 768p configurations compare sampled rows that the oracle evaluates one
by one (keys and values still come from the whole sequence)."""
import numpy as np
import pytest

import oracle as O
from dit_synth import CONFIGS, SWEEP_FRAMES, BlockDims
from helpers import FP8_MAX_BOUND, gpu_weights, inputs, oracle_weights, rel_err, rms_err, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}

# small bf16 / fp8 blocks: several GEMM and attention tiles and a ragged tail
SMALL_BF16 = BlockDims("small_bf16", d_model=512, n_heads=4, head_dim=128, d_ffn=1024, T=2, H=9, W=15, n_text=16,
                       n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=5)
SMALL_FP8 = SMALL_BF16.with_(name="small_fp8", dtype="fp8", seed=6)
# full Flash width on a small grid: the fp8 code-flip noise scales with
# 1/sqrt(width), so this is the fp8 block at the width the stack runs at
WIDE_FP8 = BlockDims("wide_fp8", T=2, H=6, W=10, n_text=16, n_audio=8, dtype="fp8", seed=8, d_model=5376, n_heads=56,
                     head_dim=128, d_ffn=14336, rope=(32, 48, 48))
# 9 token x 4 feature tiles of 256 x 256 in the O and down projections when
# uncompressed: fewer tiles than compute units, so those projections run
# entirely as K slices plus the slice-sum pass (compressed: 3 token tiles,
# too few to split, the plain path)
SPLIT_BF16 = BlockDims("split_bf16", d_model=1024, n_heads=8, head_dim=128, d_ffn=2048, T=2, H=32, W=32, n_text=16,
                       n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=9)
SPLIT_FP8 = SPLIT_BF16.with_(name="split_fp8", dtype="fp8", seed=10)


def run_gpu(d, x, w, compress, stride=None):
    dims = V.make_dims(d, stride)
    s = d.stride if stride is None else stride
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gw, codes = gpu_weights(w, d.dtype)
    keep = V.keep_index(d.T, d.H, d.W, s) if compress else None
    nk = V.nearest_kept_map(d.T, d.H, d.W, s) if compress else None
    yt, yv, ya = V.block_forward(dims, xt, xv, xa, gw, compress, keep, nk)
    torch.cuda.synchronize()
    return [to_numpy(yt), to_numpy(yv), to_numpy(ya)], codes


def check_full(d, compress, stride=None):
    print(f"block {d.name} compress={compress} stride={stride}", flush=True)
    x, w = inputs(d)
    got, codes = run_gpu(d, x, w, compress, stride)
    if codes:
        for k, (c, s) in codes.items():
            rc, rs = O.quantize_weight_fp8(w[k])
            assert np.array_equal(c.cpu().numpy().reshape(-1), rc.reshape(-1)) and np.float32(s.item()) == rs
    ow = oracle_weights(w, d.dtype)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, stride)
    err = rel_err(got, ref)
    rerr = rms_err(got, ref)
    print(f"  max|err|/rms = {err:.3e}, rms err = {rerr:.3e} (bar {TOL[d.dtype]})")
    assert np.all(np.isfinite(np.concatenate([g.ravel() for g in got])))
    if d.dtype == "fp8":
        assert rerr <= TOL["fp8"] and err <= FP8_MAX_BOUND
    else:
        assert err <= TOL[d.dtype]
    return got, ref


@pytest.mark.parametrize("compress", [False, True])
def test_tiny_fp32(compress):
    check_full(CONFIGS["tiny"], compress)


@pytest.mark.parametrize("compress", [False, True])
def test_small_bf16(compress):
    check_full(SMALL_BF16, compress)


@pytest.mark.parametrize("compress", [False, True])
def test_small_fp8(compress):
    check_full(SMALL_FP8, compress)


@pytest.mark.parametrize("compress", [False, True])
def test_wide_fp8(compress):
    check_full(WIDE_FP8, compress)


@pytest.mark.parametrize("d", [SPLIT_BF16, SPLIT_FP8], ids=lambda d: d.name)
@pytest.mark.parametrize("compress", [False, True])
def test_k_split_tail(d, compress):
    check_full(d, compress)


@pytest.mark.parametrize("name", ["tiny", "small_bf16"])
def test_stride1_equals_uncompressed(name):
    d = CONFIGS["tiny"] if name == "tiny" else SMALL_BF16
    x, w = inputs(d)
    a, _ = run_gpu(d, x, w, False)
    b, _ = run_gpu(d, x, w, True, stride=1)
    # kept rows are every row; the output is x + (y - x) instead of y
    assert rel_err(b, a) <= (1e-6 if d.dtype == "f32" else 1e-2)


def test_degenerate_grids_bf16():
    for T, H, W, nt, na in [(1, 1, 1, 0, 0), (1, 2, 2, 3, 0), (2, 3, 1, 0, 5), (1, 2, 97, 1, 1)]:
        d = SMALL_BF16.with_(name=f"deg{T}x{H}x{W}", T=T, H=H, W=W, n_text=nt, n_audio=na)
        for compress in (False, True):
            check_full(d, compress)


def test_deterministic_and_in_place():
    d = SMALL_BF16
    x, w = inputs(d)
    a, _ = run_gpu(d, x, w, True)
    b, _ = run_gpu(d, x, w, True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # in place: outputs alias the inputs
    dims = V.make_dims(d)
    xt, xv, xa = (torch_act(x[k], d.dtype) for k in ("x_text", "x_video", "x_audio"))
    gw, _ = gpu_weights(w, d.dtype)
    V.block_forward(dims, xt, xv, xa, gw, True, V.keep_index(d.T, d.H, d.W), V.nearest_kept_map(d.T, d.H, d.W),
                    out=(xt, xv, xa))
    for u, v in zip(a, (to_numpy(xt), to_numpy(xv), to_numpy(xa))):
        assert np.array_equal(u, v)


def sampled(d, compress, n_video=96, seed=0):
    g = np.random.default_rng(seed)

    def pick(n, k, fixed):
        return np.unique(np.concatenate([g.integers(0, n, k), fixed])) if n else np.zeros(0, np.int64)

    sv = pick(d.n_video, n_video, [0, d.n_video - 1, d.W - 1])
    st = pick(d.n_text, 8, [d.n_text - 1])
    sa = pick(d.n_audio, 8, [d.n_audio - 1])
    return {"text": st, "video": sv, "audio": sa}


def check_sampled(d, compress):
    print(f"block {d.name} compress={compress} (sampled rows)", flush=True)
    x, w = inputs(d)
    got, _ = run_gpu(d, x, w, compress)
    smp = sampled(d, compress)
    ow = oracle_weights(w, d.dtype)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, sample=smp)
    D = d.d_model
    gs = [got[0][smp["text"]], got[1].reshape(-1, D)[smp["video"]], got[2][smp["audio"]]]
    err, rerr = rel_err(gs, ref), rms_err(gs, ref)
    print(f"  max|err|/rms = {err:.3e}, rms err = {rerr:.3e} over {sum(len(v) for v in smp.values())} rows")
    if d.dtype == "fp8":
        assert rerr <= TOL["fp8"] and err <= FP8_MAX_BOUND
    else:
        assert err <= TOL[d.dtype]
    # every output finite
    assert all(np.all(np.isfinite(a)) for a in got)


@pytest.mark.parametrize("name,compress", [("540p_on", True), ("540p_off", False), ("768p", True), ("768p", False)])
def test_full_size_sampled(name, compress):
    check_sampled(CONFIGS[name], compress)


@pytest.mark.parametrize("T", SWEEP_FRAMES)
@pytest.mark.parametrize("compress", [True, False])
def test_sweep_768p_sampled(T, compress):
    """The 768p grid at 2, 8 and 32 latent frames (sequence-length sweep;
    2794 to 129668 tokens), sampled rows against the oracle."""
    check_sampled(CONFIGS["768p"].with_(name=f"768p_T{T}", T=T), compress)


# Many tokens at a narrow width: the QKV and gate/up projections run more than
# two rounds of 256 x 256 tiles with a partial last round. bf16: 46104 tokens
# (543 and 724 tiles) and the compressed 16-frame grid (561 and 748), sampled
# rows; fp8 (per-tensor scales need the whole tensor): 10968 tokens with 8
# heads (516 and 688 tiles), every element.
LONG_BF16 = BlockDims("long_bf16", d_model=256, n_heads=2, head_dim=128, d_ffn=512, T=4, H=96, W=120, n_text=16,
                      n_audio=8, rope=(32, 48, 48), dtype="bf16", seed=21)
LONG_FP8 = BlockDims("long_fp8", d_model=256, n_heads=8, head_dim=128, d_ffn=2048, T=2, H=72, W=76, n_text=16,
                     n_audio=8, rope=(32, 48, 48), dtype="fp8", seed=22)


LONG_CASES = [(LONG_BF16, False), (LONG_BF16.with_(name="long_bf16_c16", T=16, seed=23), True)]


@pytest.mark.parametrize("d,compress", LONG_CASES, ids=["long_bf16", "long_bf16_c16"])
def test_many_tokens_sampled(d, compress):
    check_sampled(d, compress)


def test_many_tokens_fp8():
    check_full(LONG_FP8, False)


# The light decoder's widths (2048, 16 heads of 128, FFN 8192) as a video-only
# block: every element on a small grid, sampled rows on the 540p latent grid
# that the decoder timing runs at.
DECODER_SMALL = CONFIGS["decoder"].with_(name="decoder_small", T=2, H=9, W=15, seed=12)


def test_decoder_width_small():
    check_full(DECODER_SMALL, False)


def test_decoder_width_sampled():
    check_sampled(CONFIGS["decoder"], False)
