"""The stored noise floors (tests/golden/parity_floors.json) against a fresh
computation of the cheap cases, and what the floors say (CPU only)."""
import os
import sys

import numpy as np
import pytest

import floors as FL
import oracle as O
from cases import SMALL_BF16
from helpers import inputs, oracle_weights

pytestmark = pytest.mark.cpu

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_floors  # noqa: E402

CHEAP = ["small_fp8_off", "small_fp8_on", "split_fp8_on", "ctrl_fp8_on", "hist_fp8_on", "stack_small_fp8",
         "stack_small_bf16", "ctrl_stack_bf16", "hist_stack_bf16", "long_video_bf16"]


@pytest.mark.parametrize("case", CHEAP)
def test_stored_floor_reproduces(case):
    stored = FL.load()[case]
    mx, rm = make_floors.all_cases()[case]()
    assert abs(mx - stored["max"]) <= 1e-4 * stored["max"] + 1e-6
    assert abs(rm - stored["rms"]) <= 1e-4 * stored["rms"] + 1e-6


def test_every_gpu_case_has_a_floor():
    assert set(make_floors.all_cases()) <= set(FL.load())


def test_lowbit_floors_sit_above_the_fixed_bar():
    """The e4m3 code flips put every low-bit block's floor above 6e-2 on
    max|err|/RMS, while its RMS floor stays near 1-2 %. (Degenerate grids
    aside: a single token has no flip in the rounding model and nothing to
    spread one to.)"""
    fl = FL.load()
    blocks = [k for k in fl if k.endswith(("_on", "_off")) and ("fp8" in k or k.startswith("c5_block"))
              and not k.startswith("deg_")]
    assert len(blocks) >= 11
    for k in blocks:
        assert fl[k]["max"] > 6e-2 and fl[k]["rms"] < 3e-2, (k, fl[k])


def test_fp32_storage_gives_a_negligible_floor():
    """Sanity of the rounding model: with fp32 storage everywhere a bf16-exact
    block moves by fp32 rounding only."""
    d = SMALL_BF16
    x, w = inputs(d)
    ow = oracle_weights(w, "bf16")
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, True)
    mod = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, True, store=FL.gpu_store("f32"))
    mx, rm = FL.errors(mod, ref)
    assert mx < 1e-5 and rm < 1e-6


def test_bf16_storage_floor_within_the_bf16_bar():
    d = SMALL_BF16
    x, w = inputs(d)
    ow = oracle_weights(w, "bf16")
    mx, rm = FL.block_floor(d, x, ow, True)
    assert 1e-3 < mx < 2e-2 and np.isfinite(rm)


def test_admissible_flips_sit_at_code_boundaries():
    """Each admissible single decision moves exactly one element of one
    quantiser input to the neighbouring code, and only elements within the
    reach of a boundary qualify: on the single-token case there are some, and
    each changes the oracle's outputs."""
    from cases import DEG_FP8
    from oracle.fp8 import e4m3_encode
    d = DEG_FP8[0]
    x, w = inputs(d)
    ow = oracle_weights(w, d.dtype)
    ref = O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, False)
    vals = {}

    def probe(name, a):
        vals[name] = np.array(a, dtype=np.float64).reshape(-1)
        return a
    O.block_forward(x["x_text"], x["x_video"], x["x_audio"], ow, d, False, store=probe)
    n = 0
    for (site, i), out in FL.admissible_flips(d, x, ow, False):
        n += 1
        prec = O.block.LOWBIT_PRECISION[site]
        r = FL.round_to(vals[site], prec)
        s = np.max(np.abs(r)) / 448.0
        z = r[i] / s
        zs = z * (1 + FL.FLIP_REACH[prec] * np.array([-1.0, 1.0]))
        codes = e4m3_encode(zs)
        assert codes[0] != codes[1], (site, i)        # a boundary lies within reach
        mx, _ = FL.errors(out, ref)
        assert mx > 0
    assert 0 < n < 0.1 * sum(v.size for k, v in vals.items() if k in O.block.LOWBIT_PRECISION)
