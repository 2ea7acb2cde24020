"""Pins of the oracle sampler (CPU only): the printed noise clocks and layer
schedule (tests/golden), Euler closed forms, and the equality of per-layer
compression with gather-once / broadcast-once over a compressed span."""
import os

import numpy as np
import pytest

import oracle as O
from oracle.block import BlockWeights, block_core, token_coords
from dit_synth import BlockDims
from dit_synth.configs import FLASH, FLASH_EVALS, FLASH_LAYERS

pytestmark = pytest.mark.cpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")

TINY = BlockDims("tiny-stack", d_model=16, n_heads=2, head_dim=8, d_ffn=24, T=2, H=5, W=4,
                 n_text=2, n_audio=3, rope=(2, 2, 4), dtype="f32", seed=0)


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_printed_noise_clocks():
    rows = _read_table("noise_clocks_768p.txt")
    video = [float(r[1]) for r in rows]
    audio = [float(r[2]) for r in rows]
    tv = O.flow_schedule(4, 12.0)
    ta = O.flow_schedule(4, 3.0)
    for printed, got in zip(video, tv[:4]):
        digits = len(str(printed).split(".")[1]) if "." in str(printed) else 0
        assert round(got, digits) == printed
    for printed, got in zip(audio, ta[:4]):
        assert got == pytest.approx(printed, abs=1e-15)
    assert tv[-1] == 1.0 and ta[-1] == 1.0
    assert np.all(np.diff(tv) > 0) and np.all(np.diff(ta) > 0)
    # three-evaluation Flash schedule from the same closed form
    np.testing.assert_allclose(O.flow_schedule(3, 12.0), [0, 1 / 25, 1 / 7, 1], rtol=1e-15)


def test_printed_layer_schedule():
    g = {k: float(v) for k, v in _read_table("flash_schedule.txt")}
    flags = O.flash_layer_flags()
    assert len(flags) == g["flash_layers"] == sum(FLASH_LAYERS) <= g["standard_layers"]
    assert flags[:int(g["full_head"])].sum() == 0
    assert flags.sum() == g["compressed"]
    assert flags[-int(g["full_tail"]):].sum() == 0
    assert FLASH_EVALS == g["flash_evals"]
    assert FLASH["d_model"] == g["hidden"] and FLASH["n_heads"] == g["heads"]
    assert FLASH["head_dim"] == g["head_dim"] and FLASH["d_ffn"] == g["ffn"]


def _rand_layers(d, n, seed, scale=1.0):
    g = np.random.default_rng(seed)
    D, I, F = d.d_model, d.inner, d.d_ffn
    return [BlockWeights(g1=1 + 0.2 * g.standard_normal(D), wqkv=scale * g.standard_normal((3 * I, D)) / np.sqrt(D),
                         wo=scale * g.standard_normal((D, I)) / np.sqrt(I), g2=1 + 0.2 * g.standard_normal(D),
                         wgate=scale * g.standard_normal((F, D)) / np.sqrt(D),
                         wup=scale * g.standard_normal((F, D)) / np.sqrt(D),
                         wdown=scale * g.standard_normal((D, F)) / np.sqrt(F)) for _ in range(n)]


def _inputs(d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((d.n_text, d.d_model)), g.standard_normal((d.T, d.H, d.W, d.d_model)),
            g.standard_normal((d.n_audio, d.d_model)))


def test_euler_closed_form_identity_blocks():
    """All projections zero: every block is the identity, so the velocity is
    the state itself and x_N = x_0 * prod(1 + dt_k), separately per clock."""
    d = TINY
    layers = [BlockWeights(g1=np.ones(16), wqkv=np.zeros((48, 16)), wo=np.zeros((16, 16)), g2=np.ones(16),
                           wgate=np.zeros((24, 16)), wup=np.zeros((24, 16)), wdown=np.zeros((16, 24)))] * 4
    flags = [0, 1, 1, 0]
    xt, xv, xa = _inputs(d, 1)
    tv, ta = O.flow_schedule(3, 12.0), O.flow_schedule(3, 3.0)
    yv, ya = O.stack_sample(xt, xv, xa, layers, flags, tv, ta, d)
    np.testing.assert_allclose(yv, xv * np.prod(1 + np.diff(tv)), rtol=1e-14)
    np.testing.assert_allclose(ya, xa * np.prod(1 + np.diff(ta)), rtol=1e-14)
    # no evaluation: identity
    yv, ya = O.stack_sample(xt, xv, xa, layers, flags, tv[:1], None, d)
    np.testing.assert_array_equal(yv, xv)
    np.testing.assert_array_equal(ya, xa)


def test_single_eval_equals_block_chain():
    d = TINY
    layers = _rand_layers(d, 3, 2)
    flags = [0, 1, 0]
    xt, xv, xa = _inputs(d, 3)
    t = np.asarray([0.2, 0.45])
    yv, ya = O.stack_sample(xt, xv, xa, layers, flags, t, None, d)
    zt, zv, za = xt, xv, xa
    for w, c in zip(layers, flags):
        zt, zv, za = O.block_forward(zt, zv, za, w, d, compress=bool(c))
    np.testing.assert_allclose(yv, xv + 0.25 * zv, rtol=1e-13)
    np.testing.assert_allclose(ya, xa + 0.25 * za, rtol=1e-13)


def test_per_layer_equals_per_span_broadcast():
    """A span of compressed layers applied one by one (oracle) equals:
    gather the kept tokens once, run the span as plain blocks on the kept
    sequence (original coordinates), then broadcast the summed update once."""
    d = TINY
    layers = _rand_layers(d, 4, 4)
    xt, xv, xa = _inputs(d, 5)
    zt, zv, za = xt, xv, xa
    for w in layers:
        zt, zv, za = O.block_forward(zt, zv, za, w, d, compress=True)
    D = d.d_model
    keep = O.keep_index(d.T, d.H, d.W)
    nk = O.nearest_kept_map(d.T, d.H, d.W)
    coords, kinds = token_coords(d, compressed=True)
    X0 = np.concatenate([xt, xv.reshape(-1, D)[keep], xa])
    X = X0
    for w in layers:
        X = block_core(X, coords, kinds, w, d)
    nv = len(keep)
    delta = X[d.n_text:d.n_text + nv] - X0[d.n_text:d.n_text + nv]
    span_v = xv.reshape(-1, D) + delta[nk]
    np.testing.assert_allclose(zv.reshape(-1, D), span_v, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(zt, X[:d.n_text], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(za, X[-d.n_audio:], rtol=1e-10, atol=1e-10)


def test_lowbit_stack_runs_and_stays_close():
    """fp8 projections: the quantisation-mirroring stack differs from the exact
    stack (quantisation is applied) but stays the same order of magnitude on a
    tiny model (width 16, so few terms average the e4m3 rounding out)."""
    d = TINY
    layers = _rand_layers(d, 4, 6)
    lowbit = []
    for w in layers:
        q = {}
        for f in ("wqkv", "wo", "wgate", "wup", "wdown"):
            codes, s = O.quantize_weight_fp8(getattr(w, f).astype(np.float32))
            q[f] = O.e4m3_decode(codes).reshape(getattr(w, f).shape) * float(s)
        lowbit.append(BlockWeights(g1=w.g1, g2=w.g2, lowbit=True, **q))
    xt, xv, xa = _inputs(d, 7)
    t = O.flow_schedule(3, 12.0)
    flags = [0, 1, 1, 0]
    ev, ea = O.stack_sample(xt, xv, xa, layers, flags, t, None, d)
    qv, qa = O.stack_sample(xt, xv, xa, lowbit, flags, t, None, d)
    rms = np.sqrt(np.mean(np.concatenate([ev.ravel(), ea.ravel()]) ** 2))
    err = max(np.abs(qv - ev).max(), np.abs(qa - ea).max()) / rms
    assert 0 < err < 0.6
