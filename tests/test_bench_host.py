"""CPU checks of bench.py's host side: the one-GPU guard and the algorithmic
FLOP / byte counts its roofline figures divide by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from dit_synth import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _tokens(d, compress):
    hk = (d.H + 1) // 2 + (1 - d.H % 2)
    wk = (d.W + 1) // 2 + (1 - d.W % 2)
    nv = d.T * hk * wk if compress else d.n_video
    return d.n_text + d.n_audio + nv, nv


@pytest.mark.parametrize("name,compress,tflop", [
    ("540p_on", True, 3.280),     # 2 S D 3I + 4 S^2 I + 2 S I D + 4 S D F + 2 S F D at S = 3736
    ("540p_off", False, 14.305),  # the same at S = 12628
])
def test_block_flops(name, compress, tflop):
    d = CONFIGS[name]
    S, _ = _tokens(d, compress)
    fl = bench.block_flops(d, S)
    assert set(fl) == {"gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down"}
    assert sum(fl.values()) / 1e12 == pytest.approx(tflop, abs=5e-4)
    # the attention share at the two sequence lengths (12 % and 32 %)
    assert fl["attention"] / sum(fl.values()) == pytest.approx(0.12 if compress else 0.32, abs=0.005)


def test_broadcast_bytes():
    """Broadcast + residual at 540p compressed: algorithmic bytes read x_video
    and the 3348 kept update rows once and write 12240 rows, all at 2 bytes
    (299.2 MB); the standalone kernel's fp32 update rows make it move 335.2 MB."""
    d = CONFIGS["540p_on"]
    S, nk = _tokens(d, True)
    assert (S, nk) == (3736, 3348)
    b = bench.hbm_bytes(d, S, d.n_video, nk)
    assert b["broadcast_residual"] == (2 * 12240 + 3348) * 5376 * 2 == 299206656
    assert bench.broadcast_bytes_moved(12240, 3348, 5376) == (2 * 12240 * 2 + 3348 * 4) * 5376 == 335204352
    assert b["rmsnorm1"] == 2 * 3736 * 5376 * 2
