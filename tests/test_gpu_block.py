"""GPU parity of dit_block_forward against the fp64 oracle.

Metric: max |gpu - oracle| over every output element / RMS of the oracle
outputs. Bars: 1e-4 for the fp32 block, 2e-2 for bf16; fp8 projections:
1.5 x the case's noise floor on max|err|/RMS and on the RMS error
(tests/floors.py). Every configuration is compared on every output element,
except the 768p grid uncompressed (24836 tokens), its frame sweep and the
46k-token narrow block, which compare sampled rows that the oracle evaluates
one by one (keys and values still come from the whole sequence)."""
import numpy as np
import pytest

import floors as FL
import oracle as O
from dit_synth import CONFIGS, SWEEP_FRAMES
from cases import DEG_FP8, C5_BLOCK, LONG_BF16, LONG_FP8, SMALL_BF16, SMALL_FP8, SPLIT_BF16, SPLIT_FP8, WIDE_FP8
from helpers import check_parity, gpu_weights, inputs, oracle_weights, rel_err, to_numpy, torch_act

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")


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


def check_full(d, compress, stride=None, case=None):
    """Every output element against the oracle; fp8 cases use the floor of
    `case` (default: the configuration name with _on / _off)."""
    print(f"block {d.name} compress={compress} stride={stride}", flush=True)
    x, w = inputs(d)
    got, codes = run_gpu(d, x, w, compress, stride)
    if codes:
        for k, (c, s) in codes.items():
            rc, rs = O.quantize_weight_fp8(w[k])
            assert np.array_equal(c.cpu().numpy().reshape(-1), rc.reshape(-1)) and np.float32(s.item()) == rs
        del codes
    ow = oracle_weights(w, d.dtype)
    del w
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, stride)
    if d.dtype == "fp8":
        check_parity(got, ref, "fp8", case or f"{d.name}_{'on' if compress else 'off'}")
    else:
        check_parity(got, ref, d.dtype)
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


@pytest.mark.parametrize("stride", [3, 4])
def test_other_strides_bf16(stride):
    """Compression at strides 3 and 4 (kept rows and columns 0, s, 2s, ...
    plus the last; each kept slot's update reaches a rectangle of up to s x s
    positions)."""
    check_full(SMALL_BF16.with_(name=f"small_bf16_s{stride}", H=10, W=17), True, stride=stride)


def test_degenerate_grids_bf16():
    for T, H, W, nt, na in [(1, 1, 1, 0, 0), (1, 2, 2, 3, 0), (2, 3, 1, 0, 5), (1, 2, 97, 1, 1)]:
        d = SMALL_BF16.with_(name=f"deg{T}x{H}x{W}", T=T, H=H, W=W, n_text=nt, n_audio=na)
        for compress in (False, True):
            check_full(d, compress)


@pytest.mark.parametrize("compress", [False, True])
@pytest.mark.parametrize("d", DEG_FP8[1:], ids=lambda d: d.name)
def test_degenerate_grids_fp8(d, compress):
    """Low-bit projections on text beside a 2 x 2 grid and on audio beside a
    one-column grid (tensors far smaller than a tile)."""
    check_full(d, compress)


@pytest.mark.parametrize("compress", [False, True])
def test_single_token_fp8(compress):
    """One token. Its rounding model flips no e4m3 code, so its floor is the
    bf16 storage alone; the GPU's own accumulation can still put a value that
    lies within rounding reach of a code boundary on the other side (that
    code is as correct). The GPU must match the oracle within the floor bar,
    either as is or under one such admissible decision."""
    d = DEG_FP8[0]
    print(f"block {d.name} compress={compress}", flush=True)
    x, w = inputs(d)
    got, _ = run_gpu(d, x, w, compress)
    ow = oracle_weights(w, d.dtype)
    case = f"{d.name}_{'on' if compress else 'off'}"
    mb, rb = FL.bar(case)
    cands = [("none", O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress))]
    cands += list(FL.admissible_flips(d, x, ow, compress))
    errs = sorted((FL.errors(got, ref), key) for key, ref in cands)
    (mx, rm), key = errs[0]
    print(f"  {len(cands) - 1} admissible single code decisions; closest: {key}, max|err|/rms {mx:.3e} "
          f"(bar {mb:.3e}), rms err {rm:.3e} (bar {rb:.3e})")
    assert mx <= mb and rm <= rb


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_inputs_give_zero_outputs(dtype):
    """All-zero activations: the norms give zero rows, attention averages zero
    values, and every e4m3 tensor has amax 0 (scale 1, zero codes), so every
    output is exactly zero, as in the oracle."""
    d = (SMALL_FP8 if dtype == "fp8" else SMALL_BF16).with_(name=f"zero_{dtype}")
    x, w = inputs(d)
    x = {k: np.zeros_like(v) for k, v in x.items()}
    for compress in (False, True):
        got, _ = run_gpu(d, x, w, compress)
        ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], oracle_weights(w, d.dtype), d, compress)
        for g_, r_ in zip(got, ref):
            assert not np.any(r_)
            assert not np.any(g_) and np.all(np.isfinite(g_))


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
    """bf16 only (the low-bit scales need every row)."""
    print(f"block {d.name} compress={compress} (sampled rows)", flush=True)
    x, w = inputs(d)
    got, _ = run_gpu(d, x, w, compress)
    smp = sampled(d, compress)
    ow = oracle_weights(w, d.dtype)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, sample=smp)
    D = d.d_model
    gs = [got[0][smp["text"]], got[1].reshape(-1, D)[smp["video"]], got[2][smp["audio"]]]
    print(f"  {sum(len(v) for v in smp.values())} rows")
    check_parity(gs, ref, d.dtype)
    # every output finite
    assert all(np.all(np.isfinite(a)) for a in got)


@pytest.mark.parametrize("name,compress", [("540p_on", True), ("540p_off", False), ("768p", True)])
def test_full_size_every_element(name, compress):
    """The 540p grid compressed (3736 tokens) and not (12628), the 768p grid
    compressed (7094): every output element (text, all 12240 / 24192 video
    positions, audio) against the oracle."""
    check_full(CONFIGS[name], compress)


def test_768p_uncompressed_sampled():
    check_sampled(CONFIGS["768p"], False)


@pytest.mark.parametrize("compress", [True, False], ids=["on", "off"])
def test_fp8_block_at_stack_layer_sizes(compress):
    """The fp8 block at the two layer shapes of the 42-layer stack (540p grid:
    3736 tokens compressed, 12628 not), every element."""
    check_full(C5_BLOCK, compress, case=f"c5_block_{'on' if compress else 'off'}")


# the 768p sequence-length sweep: every element up to 9244 tokens, sampled
# rows beyond (32900 and 35044-129668 tokens)
SWEEP_FULL = [(2, True), (2, False), (8, True)]
SWEEP_SAMPLED = [(8, False), (32, True), (32, False)]
assert sorted(SWEEP_FULL + SWEEP_SAMPLED) == sorted((T, c) for T in SWEEP_FRAMES for c in (True, False))


@pytest.mark.parametrize("T,compress", SWEEP_FULL, ids=lambda v: str(v))
def test_sweep_768p_every_element(T, compress):
    """The 768p grid at 2 latent frames (2794 / 8708 tokens) and 8 frames
    compressed (9244): every output element against the oracle."""
    check_full(CONFIGS["768p"].with_(name=f"768p_T{T}", T=T), compress)


@pytest.mark.parametrize("T,compress", SWEEP_SAMPLED, ids=lambda v: str(v))
def test_sweep_768p_sampled(T, compress):
    """The 768p grid at 8 frames uncompressed (32900 tokens) and 32 frames
    (35044 / 129668), sampled rows against the oracle."""
    check_sampled(CONFIGS["768p"].with_(name=f"768p_T{T}", T=T), compress)


# Many tokens at a narrow width (cases.py): bf16 46104 tokens (543 and 724
# tiles) and the compressed 16-frame grid (561 and 748), sampled rows; fp8
# (per-tensor scales need the whole tensor): 10968 tokens, every element.
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
