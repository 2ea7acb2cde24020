"""Write tests/golden/parity_floors.json: the noise floor of every low-bit
block case and every stack case of the GPU parity tests.

A floor is max |a - b| / RMS(b) and RMS(a - b) / RMS(b) over every output,
where b is the oracle and a the oracle with the GPU kernels' storage rounding
applied (tests/floors.py, GPU_STORE). The inputs, layer weights, flags and
schedules are those of the GPU tests (tests/cases.py). This script calls only
the oracle and the seeded input generator.

    python tests/golden/make_floors.py            # every case
    python tests/golden/make_floors.py NAME ...   # recompute these, keep the rest
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import cases as C  # noqa: E402
import floors as FL  # noqa: E402
from helpers import inputs, oracle_weights  # noqa: E402


def block_case(d, compress, hist=False):
    def run():
        x, w = inputs(d)
        kw = {}
        if d.n_ctrl:
            kw["x_ctrl"] = x["x_ctrl"]
            if hist:
                kw["ctrl_idx"] = O.history_index(d.n_ctrl, d.H, d.W)
        ow = oracle_weights(w, d.dtype)
        ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, **kw)
        mod = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, compress, store=FL.gpu_store(d.dtype),
                              **kw)
        return FL.errors(mod, ref)
    return run


def layers_of(d, n):
    return [oracle_weights(inputs(d, layer=l)[1], d.dtype) for l in range(n)]


def stack_case(d, flags, tv, ta, hist=False):
    def run():
        x, _ = inputs(d)
        layers = layers_of(d, len(flags))
        kw = {}
        if d.n_ctrl:
            kw["x_ctrl"] = x["x_ctrl"]
            if hist:
                kw["ctrl_idx"] = O.history_index(d.n_ctrl, d.H, d.W)
        args = (x["x_text"], x["x_video"], x["x_audio"], layers, flags, tv, ta, d)
        ref = O.stack_sample(*args, **kw)
        mod = O.stack_sample(*args, store=FL.gpu_store(d.dtype), **kw)
        return FL.errors(mod, ref)
    return run


def long_video_case():
    d = C.LONG_VIDEO
    flags = [0, 1, 1, 0]
    tv, ta = O.flow_schedule(3, 12.0).astype(np.float32), O.flow_schedule(3, 3.0).astype(np.float32)

    def run():
        from dit_synth import round_bf16
        x, _ = inputs(d)
        layers = layers_of(d, len(flags))
        g = np.random.default_rng(99)
        new = [round_bf16(g.standard_normal((d.T - 1, d.H, d.W, d.d_model)).astype(np.float32)) for _ in range(4)]
        audio = [x["x_audio"]] + [round_bf16(g.standard_normal((d.n_audio, d.d_model)).astype(np.float32))
                                  for _ in range(4)]
        args = (x["x_text"], x["x_video"], new, audio, layers, flags, tv, ta, d)
        rf, ra = O.long_video_sample(*args)
        mf, ma = O.long_video_sample(*args, store=FL.gpu_store(d.dtype))
        return FL.errors([mf] + list(ma), [rf] + list(ra))
    return run


def all_cases():
    tv = O.flow_schedule(3, 12.0).astype(np.float32)
    ta = O.flow_schedule(3, 3.0).astype(np.float32)
    cs = {}
    for d in (C.SMALL_FP8, C.WIDE_FP8, C.SPLIT_FP8, C.CTRL_FP8):
        for on in (False, True):
            cs[f"{d.name}_{'on' if on else 'off'}"] = block_case(d, on)
    cs["long_fp8_off"] = block_case(C.LONG_FP8, False)
    for d in C.DEG_FP8:
        for on in (False, True):
            cs[f"{d.name}_{'on' if on else 'off'}"] = block_case(d, on)
    for on in (False, True):
        cs[f"hist_fp8_{'on' if on else 'off'}"] = block_case(C.HIST.with_(name="hist_fp8", dtype="fp8"), on, hist=True)
    cs["c5_block_on"] = block_case(C.C5_BLOCK, True)
    cs["c5_block_off"] = block_case(C.C5_BLOCK, False)
    # bf16 blocks at the 540p configurations (their bar is the fixed 2e-2;
    # the floor says how much of it the storage rounding alone takes)
    from dit_synth import CONFIGS
    cs["c3_bf16_on"] = block_case(CONFIGS["540p_on"], True)
    cs["c2_bf16_off"] = block_case(CONFIGS["540p_off"], False)
    cs["c4_bf16_on"] = block_case(CONFIGS["768p"], True)
    for T, on in ((2, True), (2, False), (8, True)):
        cs[f"t{T}_bf16_{'on' if on else 'off'}"] = block_case(CONFIGS["768p"].with_(name=f"768p_T{T}", T=T), on)
    for dt in ("fp8", "bf16"):
        cs[f"stack_small_{dt}"] = stack_case(C.STACK_SMALL.with_(dtype=dt), C.STACK_FLAGS, tv, ta)
    cs["stack_wide_fp8"] = stack_case(C.STACK_WIDE, C.STACK_WIDE_FLAGS, tv, None)
    cs["flash42_fp8"] = stack_case(C.FLASH42, list(O.flash_layer_flags()), tv, None)
    cs["ctrl_stack_bf16"] = stack_case(C.CTRL_STACK, [0, 1, 1, 0], tv, ta)
    cs["hist_stack_bf16"] = stack_case(C.HIST_STACK, [0, 1, 0], tv, None, hist=True)
    cs["long_video_bf16"] = long_video_case()
    return cs


def main(names):
    cs = all_cases()
    out = {}
    if os.path.exists(FL.GOLDEN):
        with open(FL.GOLDEN) as f:
            out = json.load(f)
    for name in (names or list(cs)):
        t0 = time.time()
        mx, rm = cs[name]()
        out[name] = {"max": round(mx, 6), "rms": round(rm, 6)}
        print(f"{name}: max {mx:.4e} rms {rm:.4e} ({time.time() - t0:.0f} s)", flush=True)
        with open(FL.GOLDEN, "w") as f:
            json.dump(dict(sorted(out.items())), f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
