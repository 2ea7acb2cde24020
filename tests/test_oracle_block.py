"""Pins of the oracle block (CPU only): closed forms, invariants, special cases
and brute force, chosen so that a dropped term, a sign or index slip or a
transposed operand in the oracle fails at least one of them."""
import numpy as np
import pytest

import oracle as O
from oracle.block import KIND_AUDIO, KIND_TEXT, KIND_VIDEO, BlockWeights, block_core, token_coords
from dit_synth import BlockDims

pytestmark = pytest.mark.cpu

SMALL = BlockDims("small", d_model=32, n_heads=2, head_dim=16, d_ffn=48, T=2, H=5, W=7,
                  n_text=3, n_audio=2, rope=(4, 6, 6), dtype="f32", seed=0)


def rand_inputs(d, seed=0, wscale=1.0):
    g = np.random.default_rng(seed)
    D, I, F = d.d_model, d.inner, d.d_ffn
    x = {"x_text": g.standard_normal((d.n_text, D)), "x_video": g.standard_normal((d.T, d.H, d.W, D)),
         "x_audio": g.standard_normal((d.n_audio, D))}
    w = BlockWeights(g1=1 + 0.3 * g.standard_normal(D), wqkv=wscale * g.standard_normal((3 * I, D)) / np.sqrt(D),
                     wo=wscale * g.standard_normal((D, I)) / np.sqrt(I), g2=1 + 0.3 * g.standard_normal(D),
                     wgate=wscale * g.standard_normal((F, D)) / np.sqrt(D),
                     wup=wscale * g.standard_normal((F, D)) / np.sqrt(D),
                     wdown=wscale * g.standard_normal((D, F)) / np.sqrt(F))
    return x, w


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form():
    g = np.random.default_rng(1)
    m, eps = 37, 1e-2                                     # large eps makes a dropped eps visible
    x = g.standard_normal((5, m)) * np.arange(1, 6)[:, None]
    y = O.rmsnorm(x, np.ones(m), eps)
    ms = (x ** 2).mean(axis=1)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # per-row scale invariance (eps -> 0) and per-channel gains
    y0 = O.rmsnorm(x, np.ones(m), 0.0)
    np.testing.assert_allclose(O.rmsnorm(7.0 * x, np.ones(m), 0.0), y0, rtol=1e-13)
    gains = np.linspace(0.5, 2.0, m)
    np.testing.assert_allclose(O.rmsnorm(x, gains, 0.0), y0 * gains, rtol=1e-13)


# ---------------------------------------------------------------- RoPE
def _unit(S, nh, dh, idx):
    x = np.zeros((S, nh, dh))
    x[:, :, idx] = 1.0
    return x


def test_rope_unit_vector_closed_form():
    bands, base = (4, 6, 6), 10000.0
    coords = np.asarray([[3, 5, 2]])
    kinds = np.asarray([KIND_VIDEO])
    # band h (offset 4, width 6), pair i=1 -> dims (6, 7), theta = base^(-2/6)
    y = O.rope_rotate(_unit(1, 1, 16, 6), coords, kinds, bands, base)
    ang = 5 * base ** (-2.0 / 6)
    expect = np.zeros(16)
    expect[6], expect[7] = np.cos(ang), np.sin(ang)
    np.testing.assert_allclose(y[0, 0], expect, atol=1e-15)
    # the second member of a pair turns to (-sin, cos)
    y = O.rope_rotate(_unit(1, 1, 16, 7), coords, kinds, bands, base)
    expect = np.zeros(16)
    expect[6], expect[7] = -np.sin(ang), np.cos(ang)
    np.testing.assert_allclose(y[0, 0], expect, atol=1e-15)
    # band t pair 0 turns by t (theta 1); band w pair 2 by w * base^(-4/6)
    y = O.rope_rotate(_unit(1, 1, 16, 0), coords, kinds, bands, base)
    assert y[0, 0, 0] == pytest.approx(np.cos(3.0)) and y[0, 0, 1] == pytest.approx(np.sin(3.0))
    y = O.rope_rotate(_unit(1, 1, 16, 14), coords, kinds, bands, base)
    a = 2 * base ** (-4.0 / 6)
    assert y[0, 0, 14] == pytest.approx(np.cos(a)) and y[0, 0, 15] == pytest.approx(np.sin(a))


def test_rope_invariants():
    g = np.random.default_rng(2)
    bands, base = (4, 6, 6), 10000.0
    S = 9
    x = g.standard_normal((S, 2, 16))
    coords = g.integers(0, 40, size=(S, 3))
    kinds = np.asarray([KIND_TEXT] * 3 + [KIND_VIDEO] * 4 + [KIND_AUDIO] * 2)
    y = O.rope_rotate(x, coords, kinds, bands, base)
    # pair norms preserved
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    # text untouched; audio h and w bands untouched
    np.testing.assert_array_equal(y[:3], x[:3])
    np.testing.assert_array_equal(y[7:, :, 4:], x[7:, :, 4:])
    # position 0 is the identity
    y0 = O.rope_rotate(x, np.zeros_like(coords), kinds, bands, base)
    np.testing.assert_allclose(y0, x, atol=0)
    # logits depend on relative positions only: shift every t by a constant
    q = O.rope_rotate(x, coords, kinds, bands, base)
    k = O.rope_rotate(x[::-1].copy(), coords[::-1], kinds[::-1], bands, base)
    shifted = coords.copy()
    shifted[:, 0] += 11
    q2 = O.rope_rotate(x, shifted, kinds, bands, base)
    k2 = O.rope_rotate(x[::-1].copy(), shifted[::-1], kinds[::-1], bands, base)
    vid_aud = slice(3, 9)
    l1 = np.einsum("qhd,khd->hqk", q[vid_aud], k[:6])
    l2 = np.einsum("qhd,khd->hqk", q2[vid_aud], k2[:6])
    np.testing.assert_allclose(l1, l2, atol=1e-12)


# ---------------------------------------------------------------- attention
def test_attention_special_cases():
    g = np.random.default_rng(3)
    S, nh, dh = 11, 2, 8
    k = g.standard_normal((S, nh, dh))
    v = g.standard_normal((S, nh, dh))
    # q = 0 -> mean of v
    o = O.attention(np.zeros((S, nh, dh)), k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13)
    # single key -> its value
    o = O.attention(g.standard_normal((1, nh, dh)), k[:1], v[:1])
    np.testing.assert_allclose(o, v[:1], rtol=1e-13)
    # a query aligned with one key by a large margin returns that key's value
    kk = np.zeros((S, nh, dh))
    kk[4, :, 0] = 1.0
    qq = np.zeros((S, nh, dh))
    qq[:, :, 0] = 400.0
    o = O.attention(qq, kk, v)
    np.testing.assert_allclose(o, np.broadcast_to(v[4], o.shape), atol=1e-9)
    # jointly permuting keys and values changes nothing; permuting queries permutes rows
    q = g.standard_normal((S, nh, dh))
    perm = g.permutation(S)
    np.testing.assert_allclose(O.attention(q, k[perm], v[perm]), O.attention(q, k, v), rtol=1e-12)
    np.testing.assert_allclose(O.attention(q[perm], k, v), O.attention(q, k, v)[perm], rtol=1e-12)


def test_attention_brute_force_loops():
    g = np.random.default_rng(4)
    S, nh, dh = 7, 2, 4
    q, k, v = (g.standard_normal((S, nh, dh)) for _ in range(3))
    ref = np.zeros((S, nh, dh))
    for h in range(nh):
        for i in range(S):
            logits = [sum(q[i, h, c] * k[j, h, c] for c in range(dh)) / np.sqrt(dh) for j in range(S)]
            e = [np.exp(l_) for l_ in logits]
            z = sum(e)
            for c in range(dh):
                ref[i, h, c] = sum(e[j] / z * v[j, h, c] for j in range(S))
    np.testing.assert_allclose(O.attention(q, k, v, chunk=3), ref, rtol=1e-12)


# ---------------------------------------------------------------- block
def _zero_like(w, **keep):
    z = {f: np.zeros_like(getattr(w, f)) for f in ("wqkv", "wo", "wgate", "wup", "wdown")}
    z.update(keep)
    return BlockWeights(g1=w.g1, g2=w.g2, **z)


@pytest.mark.parametrize("compress", [False, True])
def test_block_zero_projections_identity(compress):
    x, w = rand_inputs(SMALL)
    for wz in (_zero_like(w), _zero_like(w, wqkv=w.wqkv, wgate=w.wgate, wup=w.wup)):  # all 0; Wo = Wd = 0
        yt, yv, ya = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], wz, SMALL, compress)
        np.testing.assert_array_equal(yt, x["x_text"])
        np.testing.assert_array_equal(yv, x["x_video"])
        np.testing.assert_array_equal(ya, x["x_audio"])


def test_block_permutation_closed_form():
    """Wq = Wk = 0 (uniform attention), Wv, Wo, Wg, Wu, Wd scaled permutations:
    the output follows from indexing alone, without any matrix product."""
    d = SMALL.with_(d_model=32, n_heads=2, head_dim=16, d_ffn=32)
    g = np.random.default_rng(5)
    D = d.d_model
    x, _ = rand_inputs(d, 6)
    pv, po, pg, pu, pd = (g.permutation(D) for _ in range(5))
    P = lambda p, c=1.0: c * np.eye(D)[p]                    # noqa: E731  (P x)[n] = c * x[p[n]]
    g1 = 1 + 0.2 * g.standard_normal(D)
    g2 = 1 + 0.2 * g.standard_normal(D)
    w = BlockWeights(g1=g1, wqkv=np.concatenate([np.zeros((2 * D, D)), P(pv, 0.7)]), wo=P(po, 1.3), g2=g2,
                     wgate=P(pg, 2.0), wup=P(pu, 0.5), wdown=P(pd, 0.9))
    yt, yv, ya = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress=False)
    X = np.concatenate([x["x_text"], x["x_video"].reshape(-1, D), x["x_audio"]])
    n1 = X / np.sqrt((X ** 2).mean(1, keepdims=True) + d.eps) * g1
    vbar = 0.7 * n1.mean(0)[pv]                               # uniform attention -> mean of v
    h = X + 1.3 * vbar[po][None, :]
    n2 = h / np.sqrt((h ** 2).mean(1, keepdims=True) + d.eps) * g2
    a = 2.0 * n2[:, pg]
    u = a / (1 + np.exp(-a)) * (0.5 * n2[:, pu])
    y = h + 0.9 * u[:, pd]
    np.testing.assert_allclose(np.concatenate([yt, yv.reshape(-1, D), ya]), y, rtol=1e-12, atol=1e-12)


def test_stride1_compression_equals_uncompressed():
    x, w = rand_inputs(SMALL, 7)
    a = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, SMALL, compress=False)
    b = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, SMALL, compress=True, stride=1)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-12)


def test_compressed_text_audio_match_block_on_kept_sequence():
    d = SMALL
    x, w = rand_inputs(d, 8)
    yt, yv, ya = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress=True)
    keep = O.keep_index(d.T, d.H, d.W)
    X = np.concatenate([x["x_text"], x["x_video"].reshape(-1, d.d_model)[keep], x["x_audio"]])
    coords, kinds = token_coords(d, compressed=True)
    y = block_core(X, coords, kinds, w, d)
    np.testing.assert_allclose(yt, y[:d.n_text], rtol=1e-13)
    np.testing.assert_allclose(ya, y[-d.n_audio:], rtol=1e-13)
    # kept video rows come out as the block output itself
    np.testing.assert_allclose(yv.reshape(-1, d.d_model)[keep], y[d.n_text:d.n_text + len(keep)], rtol=1e-12,
                               atol=1e-12)


def test_compressed_broadcast_brute_force():
    """Attention off (Wq = Wk = Wv = Wo = 0): each token's update is its own
    feed-forward term, so every video position must receive exactly the update
    of the kept position nearest to it (found here by brute force)."""
    d = SMALL.with_(H=6, W=5)
    x, w = rand_inputs(d, 9)
    w = _zero_like(w, wgate=w.wgate, wup=w.wup, wdown=w.wdown)
    _, yv, _ = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress=True)
    kh, kw = O.keep_axis(d.H), O.keep_axis(d.W)
    xv = x["x_video"]
    for t in range(d.T):
        for hh in range(d.H):
            for ww in range(d.W):
                a = min(kh, key=lambda k: (abs(k - hh), k))
                b = min(kw, key=lambda k: (abs(k - ww), k))
                src = xv[t, a, b][None, :]
                n2 = O.rmsnorm(src, w.g2, d.eps)
                upd = O.swiglu(n2, w.wgate, w.wup) @ w.wdown.T
                np.testing.assert_allclose(yv[t, hh, ww], xv[t, hh, ww] + upd[0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("compress", [False, True])
def test_sampled_rows_equal_full(compress):
    d = SMALL
    x, w = rand_inputs(d, 10)
    full = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress)
    st, sv, sa = np.asarray([0, 2]), np.asarray([0, 5, 17, d.n_video - 1]), np.asarray([1])
    yt, yv, ya = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], w, d, compress,
                                 sample={"text": st, "video": sv, "audio": sa})
    np.testing.assert_allclose(yt, full[0][st], rtol=1e-12)
    np.testing.assert_allclose(yv, full[1].reshape(-1, d.d_model)[sv], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ya, full[2][sa], rtol=1e-12)


def test_lowbit_identity_weights_quantise_input():
    """Low-bit projections: with identity weights the product returns the
    e4m3-quantised input times its per-tensor scale."""
    g = np.random.default_rng(11)
    a = g.standard_normal((6, 16))
    y = O.block.linear(a, np.eye(16), lowbit=True)
    vals, s = O.fp8.quantize_act_fp8(a)
    np.testing.assert_allclose(y, vals * s, rtol=1e-15)
    assert np.max(np.abs(y - a)) <= np.abs(a).max() * 2 ** -4
