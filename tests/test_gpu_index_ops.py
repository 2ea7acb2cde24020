"""GPU parity of the compression index maps and the bandwidth-bound ops
against the oracle: keep_index / nearest_kept_map bit-exact, gather
bit-exact, broadcast-residual and fp8 weight codes bit-exact at the kernels'
precision, standalone attention within tolerance (also with sharp logits)."""
import numpy as np
import pytest

import oracle as O
from dit_synth import CONFIGS, SWEEP_FRAMES, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
V = pytest.importorskip("video_diffusion_transformer_flash_amd")


def _idx(T, H, W, s):
    print(f"index maps T={T} H={H} W={W} stride={s}", flush=True)
    keep = V.keep_index(T, H, W, s).cpu().numpy()
    nk = V.nearest_kept_map(T, H, W, s).cpu().numpy()
    assert np.array_equal(keep, O.keep_index(T, H, W, s)), (T, H, W, s)
    assert np.array_equal(nk, O.nearest_kept_map(T, H, W, s)), (T, H, W, s)


@pytest.mark.parametrize("name", ["tiny", "540p_on", "768p", "stack"])
def test_index_maps_configs(name):
    d = CONFIGS[name]
    _idx(d.T, d.H, d.W, 2)


@pytest.mark.parametrize("T", SWEEP_FRAMES)
def test_index_maps_frame_sweep(T):
    _idx(T, 48, 84, 2)


def test_index_maps_random_grids():
    g = np.random.default_rng(0)
    for _ in range(60):
        H, W = int(g.integers(1, 98)), int(g.integers(1, 98))
        T = int(g.integers(1, 4))
        s = int(g.choice([1, 2, 3, 4]))
        _idx(T, H, W, s)
    for H, W in [(1, 1), (1, 2), (2, 1), (2, 2), (3, 3), (97, 97)]:
        _idx(2, H, W, 2)


# (T, H, W, D): one 16-byte chunk per row on a single position; fewer chunks
# than threads; the 540p compressed block's rows (several chunks per thread);
# the 768p grid at 8 frames (more chunks than one pass of the grid covers)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 8), (3, 34, 60, 384), (6, 34, 60, 5376), (8, 48, 80, 5376)])
def test_gather_kept_bit_exact(dtype, shape):
    T, H, W, D = shape
    if dtype == "f32" and D == 8:
        D = 4
    print(f"gather {dtype} T={T} H={H} W={W} D={D}", flush=True)
    x = np.random.default_rng(1).standard_normal((T, H, W, D), dtype=np.float32)
    if dtype == "bf16":
        x = round_bf16(x)
    tx = torch.from_numpy(x).cuda()
    tx = tx.to(torch.bfloat16) if dtype == "bf16" else tx
    keep = V.keep_index(T, H, W, 2)
    got = V.gather_kept(tx, keep).float().cpu().numpy()
    ref = x.reshape(-1, D)[O.keep_index(T, H, W, 2)]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ddtype", ["f32", "bf16"])
@pytest.mark.parametrize("grid", [(2, 9, 15), (6, 34, 60), (1, 1, 1), (2, 2, 5)])
def test_broadcast_residual_bit_exact(dtype, ddtype, grid):
    T, H, W = grid
    D = 256
    g = np.random.default_rng(2)
    x = g.standard_normal((T * H * W, D)).astype(np.float32)
    if dtype == "bf16":
        x = round_bf16(x)
    nkept = len(O.keep_index(T, H, W))
    delta = (0.5 * g.standard_normal((nkept, D))).astype(np.float32)
    if ddtype == "bf16":
        delta = round_bf16(delta)
    nk = O.nearest_kept_map(T, H, W)
    ref = (x + delta[nk]).astype(np.float32)      # fp32 add, then the storage rounding
    if dtype == "bf16":
        ref = round_bf16(ref)
    tx = torch.from_numpy(x).cuda()
    tx = tx.to(torch.bfloat16) if dtype == "bf16" else tx
    td = torch.from_numpy(delta).cuda()
    td = td.to(torch.bfloat16) if ddtype == "bf16" else td
    out = V.broadcast_residual(tx, td, V.nearest_kept_map(T, H, W, 2))
    assert np.array_equal(out.float().cpu().numpy(), ref)
    # in place
    V.broadcast_residual(tx, td, V.nearest_kept_map(T, H, W, 2), out=tx)
    assert np.array_equal(tx.float().cpu().numpy(), ref)


def test_fp8_weight_codes_bit_exact():
    # every bf16 bit pattern scaled into range, plus a configuration-shaped weight
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    vals = bits[np.isfinite(bits)].astype(np.float32)
    for w in (vals, (np.random.default_rng(3).standard_normal((512, 384)) / np.sqrt(384)).astype(np.float32),
              np.zeros(64, np.float32), np.asarray([1e-30, -3e-5, 2.5, -7.0] * 4, np.float32)):
        codes, scale = V.quantize_fp8(torch.from_numpy(np.ascontiguousarray(w)).cuda())
        rc, rs = O.quantize_weight_fp8(w)
        assert np.float32(scale.item()) == rs
        assert np.array_equal(codes.cpu().numpy().reshape(-1), rc.reshape(-1))
    # bf16 source gives the same codes as its fp32 value
    w = round_bf16(np.random.default_rng(4).standard_normal(4096).astype(np.float32))
    c1, _ = V.quantize_fp8(torch.from_numpy(w).cuda().to(torch.bfloat16))
    rc, _ = O.quantize_weight_fp8(w)
    assert np.array_equal(c1.cpu().numpy(), rc)


# bf16 bar: P and the output are stored in bf16 (2^-9 relative each), the max
# |o| is about 4.5x its RMS, so max|err|/RMS <= 2 * 2^-9 * 4.5 * (1 + slack) = 3e-2
@pytest.mark.parametrize("dtype,tol", [("f32", 1e-4), ("bf16", 3e-2)])
@pytest.mark.parametrize("S", [1, 63, 64, 65, 129, 300, 1000])
@pytest.mark.parametrize("sharp", [1.0, 8.0])
def test_attention_standalone(dtype, tol, S, sharp):
    nh, dh = 3, (64 if dtype == "f32" else 128)
    g = np.random.default_rng(S)
    q, k, v = (g.standard_normal((S, nh * dh)).astype(np.float32) for _ in range(3))
    q *= sharp
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    tt = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16 if dtype == "bf16" else torch.float32)  # noqa: E731
    out = V.attention(tt(q), tt(k), tt(v), nh, 1.0 / np.sqrt(dh)).float().cpu().numpy()
    ref = O.attention(q.reshape(S, nh, dh).astype(np.float64), k.reshape(S, nh, dh).astype(np.float64),
                      v.reshape(S, nh, dh).astype(np.float64)).reshape(S, nh * dh)
    err = np.max(np.abs(out - ref)) / np.sqrt(np.mean(ref ** 2))
    print(f"attention {dtype} S={S} sharp={sharp}: {err:.2e}")
    assert err <= tol
