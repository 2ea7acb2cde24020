"""Shared test plumbing: seeded inputs to torch / oracle form, error metric."""
from __future__ import annotations

import numpy as np

import oracle as O
from dit_synth import WEIGHT_NAMES, activations, weights

PROJ = ("wqkv", "wo", "wgate", "wup", "wdown")


def rel_err(got: list, ref: list) -> float:
    """max |got - ref| over every output element / RMS of the reference outputs."""
    g = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in got])
    r = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in ref])
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r)) / rms)


def rms_err(got: list, ref: list) -> float:
    """RMS of (got - ref) over every output element / RMS of the reference."""
    g = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in got])
    r = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in ref])
    return float(np.sqrt(np.mean((g - r) ** 2)) / np.sqrt(np.mean(r * r)))


# fp8 parity. Per-tensor e4m3 activation codes are a discontinuous function of
# the values they quantise: a difference of 1e-7 (relative) in a value that sits
# on a rounding boundary moves its code by one e4m3 step (up to 2^-3 of the
# value), and one such step in a large element of a norm output moves every
# projection output of that token by step * max|w|, about 3 % of the output RMS
# at width 5376. Two correct implementations that differ only by fp32 rounding
# order therefore differ by several percent in max|err|/RMS (the oracle moves by
# 4.4e-2 against itself under a 1e-7 perturbation of its quantiser inputs, and
# by 1.2e-1 under the 2^-9 of bf16 attention; see test_oracle_fp8_flips.py).
# The fp8 bar of 6e-2 is therefore applied to the RMS error, and the max error
# is held to the flip bound FP8_MAX_BOUND.
FP8_MAX_BOUND = 0.3


def torch_act(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype in ("bf16", "fp8") else t
    return t.cuda()


def to_numpy(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_weights(w: dict, dtype: str):
    """Weights on the device. For fp8 the library quantiser writes the codes;
    returns (device dict, host codes dict or None)."""
    import torch
    import video_diffusion_transformer_flash_amd as V
    out, codes = {}, {}
    for k in WEIGHT_NAMES:
        if dtype == "fp8" and k in PROJ:
            src = torch.from_numpy(np.ascontiguousarray(w[k], dtype=np.float32)).cuda()
            c, s = V.quantize_fp8(src)
            out[k], out["s_" + k] = c, s
            codes[k] = (c, s)
        else:
            out[k] = torch_act(w[k], "f32" if dtype == "f32" else "bf16")
    return out, (codes if dtype == "fp8" else None)


def oracle_weights(w: dict, dtype: str) -> O.BlockWeights:
    if dtype != "fp8":
        return O.BlockWeights.from_arrays(w)
    q = dict(w)
    for k in PROJ:
        c, s = O.quantize_weight_fp8(w[k])
        q[k] = O.e4m3_decode(c).reshape(w[k].shape) * float(s)
    return O.BlockWeights.from_arrays(q, lowbit=True)


def inputs(d, seed=None, dtype=None, layer=None):
    seed = d.seed if seed is None else seed
    dtype = dtype or d.dtype
    x = activations(d, seed, dtype)
    w = weights(d, seed, dtype, layer=layer)
    return x, w
