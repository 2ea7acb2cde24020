"""Noise floors of the parity metric (test infrastructure, CPU only).

A block with low-bit projections quantises four activation tensors to e4m3
codes with per-tensor scales. A code is a discontinuous function of the value
it encodes, so two correct implementations whose intermediates differ by
rounding alone give codes that differ by one step wherever a value sits near a
rounding boundary; a changed code in the attention output or a norm output
moves whole token rows, and such changes cascade through the next norm. The
max |error| / RMS metric therefore has a floor that no implementation rounding
differently from the oracle can go below.

The floor of a case is measured with the oracle itself: the oracle against
the oracle with a rounding model of the GPU kernels' documented storage
points (GPU_STORE) applied through its `store` hook. The parity bar of a
low-bit case is FLOOR_MARGIN times that floor (max and RMS). The floors of
the cases the GPU tests use are written to tests/golden/parity_floors.json by
tests/golden/make_floors.py, which calls only the oracle and the seeded input
generator; test_floors.py recomputes the small ones.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle as O
from oracle.fp8 import round_to

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "parity_floors.json")
FLOOR_MARGIN = 1.5

# Precision in which the GPU kernels store each intermediate (None: not
# stored; the value goes on in registers or straight into its quantiser).
#   bf16 block: normalised rows, q / k / v, the attention weights P, the
#     attention output, the SwiGLU product and the outputs in bf16; h in fp32.
#   fp8 projections: the normalised rows go to the e4m3 quantiser from fp32;
#     the rest as for bf16.
#   stacks: the state between layers and evaluations in the activation dtype.
GPU_STORE = {
    "bf16": {"n1": "bf16", "q": "bf16", "k": "bf16", "v": "bf16", "p": "bf16", "o": "bf16", "h": "f32",
             "n2": "bf16", "u": "bf16", "out": "bf16", "state": "bf16"},
    "fp8": {"n1": None, "q": "bf16", "k": "bf16", "v": "bf16", "p": "bf16", "o": "bf16", "h": "f32", "n2": None,
            "u": "bf16", "out": "bf16", "state": "bf16"},
    "f32": {k: "f32" for k in ("n1", "q", "k", "v", "p", "o", "h", "n2", "u", "out", "state")},
}


def gpu_store(dtype: str):
    table = GPU_STORE[dtype]

    def store(name, a):
        prec = table.get(name)
        return a if prec is None else round_to(a, prec)
    return store


def errors(got, ref):
    g = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in got])
    r = np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in ref])
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r)) / rms), float(np.sqrt(np.mean((g - r) ** 2)) / rms)


def block_floor(d, x, ow, compress: bool):
    """(max, rms) of oracle vs the oracle under GPU_STORE, over every output."""
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress)
    mod = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, store=gpu_store(d.dtype))
    return errors(mod, ref)


def stack_floor(d, x, layers, flags, tv, ta):
    ref = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], layers, flags, tv, ta, d)
    mod = O.stack_sample(x["x_text"], x["x_video"], x["x_audio"], layers, flags, tv, ta, d,
                         store=gpu_store(d.dtype))
    return errors(mod, ref)


# how close (relative) to a code boundary a quantiser input must lie for the
# other code to be admissible: one bf16 unit for inputs held in bf16 (one
# rounding of a value whose accumulation differed can move it by that much),
# 2^-12 for inputs held in fp32 (accumulation-order differences of the
# projections and norms feeding them, fp8 products included)
FLIP_REACH = {"bf16": 2.0 ** -8, "f32": 2.0 ** -12}


def admissible_flips(d, x, ow, compress: bool):
    """Oracle outputs under each admissible single code decision: an e4m3
    code is an integer decided by floating point, and where the value at a
    quantiser input (n1, o, n2, u; in the precision the codes are decided in)
    lies within FLIP_REACH (relative) of the rounding boundary between two codes,
    an implementation whose accumulation differs from the oracle's by rounding
    may take the other code, which is as correct. Yields the oracle's outputs
    with one such element moved to the code across its boundary (the tensor's
    amax kept). For small cases: one oracle block per candidate."""
    from oracle.fp8 import e4m3_decode, e4m3_encode

    grid = np.sort(np.unique(np.abs(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))))
    mids = (grid[1:] + grid[:-1]) / 2
    args = (x["x_text"], x["x_video"], x["x_audio"], ow, d, compress)
    vals = {}

    def probe(name, a):
        if name in O.block.LOWBIT_PRECISION:
            vals[name] = np.array(a, dtype=np.float64).reshape(-1)
        return a
    O.block_forward(*args, store=probe)
    for site, v in vals.items():
        prec = O.block.LOWBIT_PRECISION[site]
        rel = FLIP_REACH[prec]
        r = round_to(v, prec)
        amax = float(np.max(np.abs(r)))
        if amax == 0.0:
            continue
        z = np.abs(r) / (amax / 448.0)
        j = np.clip(np.searchsorted(mids, z), 1, len(mids) - 1)
        for jj in (j - 1, j):
            near = np.abs(z - mids[jj]) <= rel * z
            for i in np.nonzero(near & (np.abs(r) < amax))[0]:
                lo, hi = grid[jj[i]], grid[jj[i] + 1]
                c = int(e4m3_encode(np.array([r[i] / (amax / 448.0)]))[0])
                other = hi if float(e4m3_decode(np.array([c], dtype=np.uint8))[0]) == np.copysign(lo, r[i]) else lo
                target = np.copysign(other, r[i]) * (amax / 448.0)

                def flip(name, a, site=site, i=i, target=target):
                    if name != site:
                        return a
                    flat = np.array(a, dtype=np.float64).reshape(-1)
                    flat[i] = target
                    return flat.reshape(np.shape(a))
                yield (site, int(i)), O.block_forward(*args, store=flip)


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def bar(case: str):
    """(max bar, rms bar) of a low-bit or stack case: FLOOR_MARGIN x its floor."""
    fl = load()[case]
    return FLOOR_MARGIN * fl["max"], FLOOR_MARGIN * fl["rms"]
