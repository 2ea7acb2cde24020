"""Seeded synthetic inputs for the Flash DiT block.

This module is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and formats them for storage (bf16 rounding, raw bit
patterns). It holds none of the block's arithmetic: no normalisation, rotary
embedding, attention, projection, compression or quantisation.

Value recipe (the workload description of the block configurations):
  * activations (text, video, audio rows)  ~ N(0, 1)
  * projection weights W[out, in]          ~ N(0, 1/fan_in)   (second argument
    read as the variance, so std = 1/sqrt(fan_in))
  * RMSNorm gains                          ~ 1 + N(0, 0.1)    (variance 0.1)
Every tensor has its own streams: the flattened tensor is cut into chunks of
2**22 values and chunk c is drawn from numpy PCG64 seeded by
SeedSequence([seed, tensor_id, c]), so any tensor (or chunk) can be
regenerated on its own, and chunks are drawn in parallel threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import (BlockDims, CONFIGS, DECODER_LAYERS, FLASH_EVALS, FLASH_LAYERS, SWEEP_FRAMES,  # noqa: F401
                      get_config)

# tensor ids inside one seed
TID_X_TEXT, TID_X_VIDEO, TID_X_AUDIO, TID_X_CTRL = 0, 1, 2, 3
TID_G1, TID_WQKV, TID_WO, TID_G2, TID_WGATE, TID_WUP, TID_WDOWN = 10, 11, 12, 13, 14, 15, 16
WEIGHT_NAMES = ("g1", "wqkv", "wo", "g2", "wgate", "wup", "wdown")


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


CHUNK = 1 << 22
_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def round_bf16(a: np.ndarray, inplace: bool = False) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32 (storage
    format). Finite inputs only."""
    a = np.array(a, dtype=np.float32, copy=not inplace, order="C")
    u = a.reshape(-1).view(np.uint32)

    def work(lo):
        b = u[lo:lo + CHUNK]
        lsb = (b >> 16) & 1
        b += np.uint32(0x7FFF)
        b += lsb
        b &= np.uint32(0xFFFF0000)

    list(_POOL.map(work, range(0, u.size, CHUNK)))
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of an fp32 array whose values are bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(seed, tid, shape, std=1.0, mean=0.0):
    n = int(np.prod(shape))
    x = np.empty(n, dtype=np.float32)

    def work(c):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tid), c])))
        part = x[c * CHUNK:(c + 1) * CHUNK]
        g.standard_normal(out=part, dtype=np.float32)
        if std != 1.0:
            part *= np.float32(std)
        if mean != 0.0:
            part += np.float32(mean)

    list(_POOL.map(work, range((n + CHUNK - 1) // CHUNK)))
    return x.reshape(shape)


def _fmt(x, dtype):
    return round_bf16(x, inplace=True) if dtype in ("bf16", "fp8") else x


def activations(d: BlockDims, seed: int, dtype: str = None) -> dict:
    """x_text [Nt, D], x_video [T, H, W, D], x_audio [Na, D] (and x_ctrl
    [n_ctrl, H, W, D] when the configuration has control frames) as fp32
    arrays (bf16-exact values when the configuration is bf16 or fp8)."""
    dtype = dtype or d.dtype
    out = {
        "x_text": _fmt(_normal(seed, TID_X_TEXT, (d.n_text, d.d_model)), dtype),
        "x_video": _fmt(_normal(seed, TID_X_VIDEO, (d.T, d.H, d.W, d.d_model)), dtype),
        "x_audio": _fmt(_normal(seed, TID_X_AUDIO, (d.n_audio, d.d_model)), dtype),
    }
    if getattr(d, "n_ctrl", 0):
        out["x_ctrl"] = _fmt(_normal(seed, TID_X_CTRL, (d.n_ctrl, d.H, d.W, d.d_model)), dtype)
    return out


def weights(d: BlockDims, seed: int, dtype: str = None, layer: int = None) -> dict:
    """One block's weights, [out, in] row-major, fp32 arrays. For bf16 the
    values are bf16-exact; for fp8 they are the fp32 draws (each side
    quantises them itself)."""
    dtype = dtype or d.dtype
    base = 0 if layer is None else 1000 + 100 * int(layer)
    D, I, F = d.d_model, d.inner, d.d_ffn
    wq_dtype = "f32" if dtype == "fp8" else dtype
    out = {
        "g1": _fmt(_normal(seed, base + TID_G1, (D,), std=np.sqrt(0.1), mean=1.0), "f32" if dtype == "f32" else "bf16"),
        "wqkv": _fmt(_normal(seed, base + TID_WQKV, (3 * I, D), std=1.0 / np.sqrt(D)), wq_dtype),
        "wo": _fmt(_normal(seed, base + TID_WO, (D, I), std=1.0 / np.sqrt(I)), wq_dtype),
        "g2": _fmt(_normal(seed, base + TID_G2, (D,), std=np.sqrt(0.1), mean=1.0), "f32" if dtype == "f32" else "bf16"),
        "wgate": _fmt(_normal(seed, base + TID_WGATE, (F, D), std=1.0 / np.sqrt(D)), wq_dtype),
        "wup": _fmt(_normal(seed, base + TID_WUP, (F, D), std=1.0 / np.sqrt(D)), wq_dtype),
        "wdown": _fmt(_normal(seed, base + TID_WDOWN, (D, F), std=1.0 / np.sqrt(F)), wq_dtype),
    }
    return out


def block_inputs(d: BlockDims, seed: int, dtype: str = None) -> dict:
    out = activations(d, seed, dtype)
    out.update(weights(d, seed, dtype))
    return out
