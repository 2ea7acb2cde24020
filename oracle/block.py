"""One joint text + video + audio Flash DiT block, plain fp64 numpy.

Sources:
  * tokendh.com article, backbone section: one shared denoiser over text,
    video and audio tokens; block width 5376, 56 heads of 128, feed-forward
    width 14336; tokens carry 3D rotary positions.
  * tokendh.com article, training section and PaperDaily review, section 2:
    the compressed layers compute attention and the feed-forward update on the
    kept video tokens (plus all text and audio tokens), and every video
    position adds the update of its nearest kept position of the same frame to
    its own full-resolution features.

Readings of the points the pages leave open (each one a choice, listed with
the reasons in the design notes):
  * block form: pre-RMSNorm, no biases, no modulation, one weight set shared by
    all modalities: h = X + Attn(RMSNorm(X) g1) Wo^T,
    y = h + (silu(n2 Wg^T) * (n2 Wu^T)) Wd^T with n2 = RMSNorm(h) g2;
  * RMSNorm: x / sqrt(mean(x^2) + eps) * g over the hidden axis;
  * attention: softmax(q k^T / sqrt(head_dim)) v per head over the whole joint
    sequence, no mask;
  * rotary embedding: each head splits into bands (t, h, w) in that order;
    inside a band of width d, pair (2i, 2i+1) turns by pos * base**(-2i/d)
    as (a, b) -> (a cos - b sin, a sin + b cos); q and k rotate, v does not.
    Video tokens use (t, h, w) (compressed tokens keep their original
    coordinates), audio token j rotates only its t band by position j, text
    does not rotate;
  * "the update" of a kept token is y - X (attention plus feed-forward);
  * sequence order [text | video (t, h, w raster) | control | audio].

Control frames (tokendh.com article, backbone section: a reference's time
coordinate sits a fixed positive constant before the target's; PaperDaily
review, section 1: aligned control frames and targets keep a stable positive
time offset, one-to-one in position but never at the same time). Readings:
x_ctrl [Tc, H, W, D] holds control frames on the video's spatial grid; control
frame k has coordinates (k, h, w) and rotates all three bands; with a
control offset c the video tokens use (t + c, h, w) and audio token j the
t-position j + c (every time position moves together, so the logits among
video and audio tokens do not change); control tokens are never compressed;
their block outputs are returned, and the sampler re-feeds the control frames
every evaluation, like text.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import compress as cmp
from .fp8 import quantize_act_fp8

KIND_TEXT, KIND_VIDEO, KIND_AUDIO = 0, 1, 2


@dataclass
class BlockWeights:
    """fp64 weights, [out, in]. With lowbit=True the projection weights are
    already the dequantised fp8 values (codes * scale) and every projection
    input is quantised per tensor before the product."""
    g1: np.ndarray
    wqkv: np.ndarray
    wo: np.ndarray
    g2: np.ndarray
    wgate: np.ndarray
    wup: np.ndarray
    wdown: np.ndarray
    lowbit: bool = False

    @classmethod
    def from_arrays(cls, w: dict, lowbit: bool = False) -> "BlockWeights":
        f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        return cls(f(w["g1"]), f(w["wqkv"]), f(w["wo"]), f(w["g2"]), f(w["wgate"]), f(w["wup"]),
                   f(w["wdown"]), lowbit)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


# Precision each low-bit projection input is held in when its e4m3 codes are
# decided (codes are integers decided by floating point, so the oracle decides
# them in the precision the kernels quantise from): the normalised rows in
# fp32, the attention output and the SwiGLU product in bf16 (the precision in
# which those steps hand them on).
LOWBIT_PRECISION = {"n1": "f32", "o": "bf16", "n2": "f32", "u": "bf16"}


def linear(a: np.ndarray, w: np.ndarray, lowbit: bool, precision: str = "f64") -> np.ndarray:
    """a @ w^T; with lowbit the input is first quantised to e4m3 with a
    per-tensor dynamic scale, its codes decided in `precision` (the weights
    are already dequantised fp8)."""
    if lowbit:
        a, s = quantize_act_fp8(a, precision)
        return (a @ w.T) * s
    return a @ w.T


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(n2: np.ndarray, wgate: np.ndarray, wup: np.ndarray, lowbit: bool = False,
           precision: str = "f64") -> np.ndarray:
    if lowbit:  # one quantised input feeds both projections
        a, s = quantize_act_fp8(n2, precision)
        return silu((a @ wgate.T) * s) * ((a @ wup.T) * s)
    return silu(n2 @ wgate.T) * (n2 @ wup.T)


def grid_coords(T: int, H: int, W: int) -> np.ndarray:
    """(t, h, w) of every position of a [T, H, W] grid in raster order."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.int64)


def token_coords(d, compressed: bool, stride: int = None, t_shift: int = 0, ctrl_idx=None):
    """Per token of the joint sequence: coordinates [S, 3] and kind [S].
    t_shift moves every time position (video, control, audio) by a constant;
    ctrl_idx selects control tokens by flat position in the control grid."""
    s = d.stride if stride is None else stride
    nc, c = getattr(d, "n_ctrl", 0), getattr(d, "ctrl_offset", 0)
    text = np.zeros((d.n_text, 3), dtype=np.int64)
    video = cmp.kept_coords(d.T, d.H, d.W, s) if compressed else grid_coords(d.T, d.H, d.W)
    video = video.copy()
    video[:, 0] += c + t_shift
    ctrl = grid_coords(nc, d.H, d.W)
    if ctrl_idx is not None:
        ctrl = ctrl[np.asarray(ctrl_idx, dtype=np.int64)]
    ctrl[:, 0] += t_shift
    audio = np.zeros((d.n_audio, 3), dtype=np.int64)
    audio[:, 0] = np.arange(d.n_audio) + c + t_shift
    coords = np.concatenate([text, video, ctrl, audio], axis=0)
    kinds = np.concatenate([np.full(d.n_text, KIND_TEXT), np.full(len(video) + len(ctrl), KIND_VIDEO),
                            np.full(d.n_audio, KIND_AUDIO)]).astype(np.int64)
    return coords, kinds


def rope_rotate(x: np.ndarray, coords: np.ndarray, kinds: np.ndarray, bands, base: float) -> np.ndarray:
    """x [S, heads, head_dim] -> rotated copy (see the module docstring)."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    off = 0
    for axis, width in enumerate(bands):
        if width % 2:
            raise ValueError("rotary band widths must be even")
        theta = base ** (-np.arange(0, width, 2, dtype=np.float64) / width)      # [width/2]
        applies = (kinds == KIND_VIDEO) | ((kinds == KIND_AUDIO) & (axis == 0))
        ang = coords[:, axis:axis + 1].astype(np.float64) * theta[None, :]        # [S, width/2]
        c = np.where(applies[:, None], np.cos(ang), 1.0)[:, None, :]
        s = np.where(applies[:, None], np.sin(ang), 0.0)[:, None, :]
        a = x[:, :, off:off + width:2]
        b = x[:, :, off + 1:off + width:2]
        out[:, :, off:off + width:2] = a * c - b * s
        out[:, :, off + 1:off + width:2] = a * s + b * c
        off += width
    if off != x.shape[-1]:
        raise ValueError("rotary bands must sum to head_dim")
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int = 1024, p_store=None) -> np.ndarray:
    """q [Sq, heads, dh], k and v [Sk, heads, dh] -> [Sq, heads, dh]:
    softmax(q k^T / sqrt(dh)) v per head, max-subtracted, unmasked.

    p_store (tests only, default none): applied to the unnormalised weights
    exp(logit - max) before they multiply v and enter the normaliser; a
    rounding model of an implementation that stores them."""
    sq, nh, dh = q.shape
    out = np.empty((sq, nh, v.shape[-1]), dtype=np.float64)
    scale = 1.0 / np.sqrt(dh)
    for h in range(nh):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, sq, chunk):
            logits = (q[r0:r0 + chunk, h, :] @ kh.T) * scale
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            if p_store is not None:
                p = p_store(p)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + chunk, h, :] = p @ vh
    return out


def block_core(X: np.ndarray, coords: np.ndarray, kinds: np.ndarray, w: BlockWeights, d,
               rows: np.ndarray = None, store=None) -> np.ndarray:
    """The block on an already assembled joint sequence X [S, D] -> y.
    With `rows`, only those output rows are evaluated (keys and values still
    come from every token); not available for the low-bit form, whose
    per-tensor activation scales need every row.

    store (tests only, default none): store(name, array) -> array is applied
    to the intermediates an implementation keeps in memory ("n1", "q", "k"
    after the rotary embedding, "v", "p" the attention weights, "o", "h",
    "n2", "u"), a rounding model used to measure how far two correct
    implementations that round differently can drift apart."""
    X = np.asarray(X, dtype=np.float64)
    S, D = X.shape
    nh, dh, I = d.n_heads, d.head_dim, d.n_heads * d.head_dim
    if rows is not None and w.lowbit:
        raise ValueError("row sampling needs the full tensor for low-bit scales")
    st = store if store is not None else (lambda name, a: a)
    lp = LOWBIT_PRECISION
    n1 = st("n1", rmsnorm(X, w.g1, d.eps))
    if w.lowbit:
        qkv = linear(n1, w.wqkv, True, lp["n1"])
        q, k, v = qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:]
    else:
        n1q = n1 if rows is None else n1[rows]
        q = n1q @ w.wqkv[:I].T
        k = n1 @ w.wqkv[I:2 * I].T
        v = n1 @ w.wqkv[2 * I:].T
    qrows = np.arange(S) if rows is None or w.lowbit else np.asarray(rows)
    q = st("q", rope_rotate(q.reshape(len(qrows), nh, dh), coords[qrows], kinds[qrows], d.rope, d.rope_base))
    k = st("k", rope_rotate(k.reshape(S, nh, dh), coords, kinds, d.rope, d.rope_base))
    v = st("v", v.reshape(S, nh, dh))
    p_store = None if store is None else (lambda p: store("p", p))
    o = st("o", attention(q, k, v, p_store=p_store).reshape(len(qrows), I))
    Xr = X[qrows]
    h = st("h", Xr + linear(o, w.wo, w.lowbit, lp["o"]))
    n2 = st("n2", rmsnorm(h, w.g2, d.eps))
    u = st("u", swiglu(n2, w.wgate, w.wup, w.lowbit, lp["n2"]))
    return h + linear(u, w.wdown, w.lowbit, lp["u"])


def block_forward(x_text, x_video, x_audio, w: BlockWeights, d, compress: bool, stride: int = None,
                  sample: dict = None, x_ctrl=None, t_shift: int = 0, ctrl_idx=None, store=None):
    """The full block on the three inputs (x_video [T, H, W, D]).

    Returns (y_text [Nt, D], y_video [T, H, W, D], y_audio [Na, D]), and
    y_ctrl [Tc, H, W, D] as a fourth element when x_ctrl is given. With
    ctrl_idx (flat positions in the [Tc, H, W] control grid, e.g. a bounded
    long-video history) only those control tokens join the sequence, with
    their own coordinates, and y_ctrl is [len(ctrl_idx), D] in that order.
    With compress=True the joint sequence holds only the kept video tokens;
    text and audio outputs come from the block, and every video position gets
    x + (update of its nearest kept slot).

    sample = {"text": idx, "video": flat positions, "audio": idx} evaluates only
    those outputs (returned flat, in the same three-tuple form; no control
    frames). store: the rounding model of block_core (tests only), also
    applied to the outputs as "out"."""
    s = d.stride if stride is None else stride
    D = d.d_model
    nc = getattr(d, "n_ctrl", 0)
    if (x_ctrl is None) != (nc == 0):
        raise ValueError("x_ctrl must be given exactly when the configuration has control frames")
    if nc and getattr(d, "ctrl_offset", 0) < 1:
        raise ValueError("control frames need a positive time offset")
    xt = np.asarray(x_text, dtype=np.float64).reshape(d.n_text, D)
    xv = np.asarray(x_video, dtype=np.float64).reshape(d.n_video, D)
    xa = np.asarray(x_audio, dtype=np.float64).reshape(d.n_audio, D)
    xc = np.asarray(x_ctrl, dtype=np.float64).reshape(nc * d.H * d.W, D) if nc else np.zeros((0, D))
    if ctrl_idx is not None:
        xc = xc[np.asarray(ctrl_idx, dtype=np.int64)]
    coords, kinds = token_coords(d, compress, s, t_shift, ctrl_idx)
    if compress:
        keep = cmp.keep_index(d.T, d.H, d.W, s)
        nk = cmp.nearest_kept_map(d.T, d.H, d.W, s)
        xv_seq = xv[keep]
    else:
        xv_seq = xv
    nvs, ncs = len(xv_seq), len(xc)
    X = np.concatenate([xt, xv_seq, xc, xa], axis=0)

    if sample is None:
        y = block_core(X, coords, kinds, w, d, store=store)
        yt, yv_seq = y[:d.n_text], y[d.n_text:d.n_text + nvs]
        yc, ya = y[d.n_text + nvs:d.n_text + nvs + ncs], y[d.n_text + nvs + ncs:]
        if compress:
            delta = yv_seq - xv_seq
            yv = xv + delta[nk]
        else:
            yv = yv_seq
        if store is not None:
            yt, yv, yc, ya = (store("out", a) for a in (yt, yv, yc, ya))
        out = (yt, yv.reshape(d.T, d.H, d.W, D), ya)
        if not nc:
            return out
        return out + ((yc if ctrl_idx is not None else yc.reshape(nc, d.H, d.W, D)),)
    if nc or store is not None:
        raise ValueError("row sampling is not available with control frames or a rounding model")

    st = np.asarray(sample.get("text", []), dtype=np.int64)
    sv = np.asarray(sample.get("video", []), dtype=np.int64)
    sa = np.asarray(sample.get("audio", []), dtype=np.int64)
    vslots = nk[sv] if compress else sv
    rows = np.concatenate([st, d.n_text + vslots, d.n_text + nvs + ncs + sa]).astype(np.int64)
    y = block_core(X, coords, kinds, w, d, rows=rows)
    yt, yv_rows, ya = y[:len(st)], y[len(st):len(st) + len(sv)], y[len(st) + len(sv):]
    if compress:
        yv = xv[sv] + (yv_rows - xv_seq[vslots])
    else:
        yv = yv_rows
    return yt, yv, ya
