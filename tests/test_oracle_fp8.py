"""Pins of the oracle's e4m3 encoder (CPU only).

The encoder is checked against an independent library routine (torch's
float8_e4m3fn cast, which rounds to nearest-even) on every bf16 bit pattern
after clamping to +-448, and against hand-derived special values of the OCP
e4m3 format (largest finite 448, subnormal step 2**-9, ties to even code).
"""
import numpy as np
import pytest
import torch

import oracle as O
from dit_synth import round_bf16

pytestmark = pytest.mark.cpu


def _torch_codes(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_all_bf16_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(x), _torch_codes(x))
    # and the brute-force nearest-table map agrees, including every exact tie
    assert np.array_equal(O.fp8.e4m3_encode_nearest(x), O.e4m3_encode(x))
    ties = (O.fp8._POS[1:] + O.fp8._POS[:-1]) / 2
    assert np.array_equal(O.fp8.e4m3_encode_nearest(ties), O.e4m3_encode(ties))


def test_dense_fp32_sample_matches_torch():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = np.clip(x.astype(np.float32), -448, 448)
    assert np.array_equal(O.e4m3_encode(x), _torch_codes(x))


def test_roundtrip_every_code():
    codes = np.asarray([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    back = O.e4m3_encode(vals)
    # +0 and -0 both decode to 0; the sign is kept
    assert np.array_equal(back, codes)


def test_special_values():
    enc = lambda v: int(O.e4m3_encode(np.asarray([v]))[0])  # noqa: E731
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(1000.0) == 0x7E and enc(-1e6) == 0xFE           # saturation
    assert enc(2.0 ** -9) == 0x01                              # smallest subnormal
    assert enc(2.0 ** -10) == 0x00                             # tie between 0 and 2^-9 -> even code 0
    assert enc(3 * 2.0 ** -10) == 0x02                         # tie between codes 1 and 2 -> 2
    assert enc(1.0) == 0x38 and enc(1.0625) == 0x38            # 1.0625 is a tie (1, 1.125) -> even 0x38
    assert enc(1.1875) == 0x3A                                 # tie (1.125, 1.25) -> even 0x3A
    assert enc(-0.0) == 0x80
    assert O.e4m3_decode(np.asarray([0x7E]))[0] == 448.0
    assert np.isnan(O.e4m3_decode(np.asarray([0x7F]))[0])


def test_weight_quantiser_scale_rule():
    g = np.random.default_rng(3)
    w = round_bf16(g.standard_normal((64, 48)).astype(np.float32) * 0.1)
    codes, scale = O.quantize_weight_fp8(w)
    amax = np.float32(np.abs(w).max())
    assert scale == np.float32(amax / np.float32(448))
    assert codes.reshape(-1)[np.argmax(np.abs(w))] & 0x7F == 0x7E   # amax lands on 448
    deq = O.e4m3_decode(codes).reshape(w.shape) * float(scale)
    # relative error of e4m3 is at most 2^-4 for normals; subnormals are absolute 2^-10 * scale
    err = np.abs(deq - w)
    assert np.all(err <= np.maximum(np.abs(w) * 2 ** -4, 2 ** -10 * float(scale)) + 1e-12)
    z, zs = O.quantize_weight_fp8(np.zeros((4, 4), np.float32))
    assert zs == 1.0 and not z.any()


def test_activation_quantiser():
    g = np.random.default_rng(5)
    a = g.standard_normal((33, 17))
    vals, s = O.fp8.quantize_act_fp8(a)
    assert s == np.abs(a).max() / 448.0
    assert np.max(np.abs(vals)) == 448.0                      # the amax element maps to the top code
    deq = vals * s
    assert np.all(np.abs(deq - a) <= np.maximum(np.abs(a) * 2 ** -4, 2 ** -10 * s) + 1e-15)
