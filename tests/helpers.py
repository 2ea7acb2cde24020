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


# Parity bars. fp32 and bf16 blocks: max|err|/RMS <= 1e-4 / 2e-2 (fixed).
# Low-bit (fp8) blocks and every stack: FLOOR_MARGIN x the case's noise floor,
# on max|err|/RMS and on the RMS error (tests/floors.py: the oracle against
# itself with the GPU's storage rounding; e4m3 code flips put that floor
# above the fixed bars).
BLOCK_TOL = {"f32": 1e-4, "bf16": 2e-2}


def check_parity(got: list, ref: list, dtype: str, case: str = None) -> tuple:
    """Assert the bar of `dtype` (fixed), or of floor case `case`; returns (max, rms)."""
    import floors
    err, rerr = rel_err(got, ref), rms_err(got, ref)
    assert all(np.all(np.isfinite(np.asarray(g))) for g in got)
    if case is None:
        print(f"  max|err|/rms = {err:.3e}, rms err = {rerr:.3e} (bar {BLOCK_TOL[dtype]})")
        assert err <= BLOCK_TOL[dtype]
    else:
        fl = floors.load()[case]
        mb, rb = floors.bar(case)
        print(f"  max|err|/rms = {err:.3e} ({err / fl['max']:.2f} x floor {fl['max']:.3e}, bar {mb:.3e}); "
              f"rms err = {rerr:.3e} ({rerr / fl['rms']:.2f} x floor {fl['rms']:.3e}, bar {rb:.3e})")
        assert err <= mb and rerr <= rb
    return err, rerr


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
