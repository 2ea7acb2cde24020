"""Pins of the oracle's keep sets and nearest-kept maps (CPU only).

What fixes them: the pages (PaperDaily review, section 2; tokendh.com article,
training section) keep every other row and column of each frame plus the edge
rows and columns, about a quarter of the positions, and give every dropped
position the update of the nearest kept position of the same frame. The
configuration sizes 18 x 31 per frame (540p grid 34 x 60) and 25 x 43 (768p
grid 48 x 84) and the count formula ceil(n/2) + [n even] are checked against
the oracle, and the maps against brute force.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("n", range(1, 65))
def test_count_formula_stride2(n):
    assert len(O.keep_axis(n, 2)) == math.ceil(n / 2) + (1 if n % 2 == 0 else 0)


@pytest.mark.parametrize("s", [1, 2, 3, 4, 5])
def test_count_formula_general_stride(s):
    for n in range(1, 70):
        expect = math.ceil(n / s) + (1 if (n - 1) % s != 0 else 0)
        assert len(O.keep_axis(n, s)) == expect


def test_config_sizes():
    assert O.keep_dims(34, 60) == (18, 31)          # 540p grid
    assert O.keep_dims(48, 84) == (25, 43)          # 768p grid
    assert 6 * 18 * 31 == 3348 and 6 * 25 * 43 == 6450
    # Tiny grid 9 x 15: the stated rule (even indices plus the last) gives
    # 5 x 8 = 40 per frame, i.e. 80 for two frames. The tiny configuration's
    # text states 6 x 9 per frame, which corresponds to ceil(n/2) + 1 for odd
    # n and contradicts the count formula; the formula is followed here.
    assert O.keep_dims(9, 15) == (5, 8)
    assert len(O.keep_index(2, 9, 15)) == 80


def test_about_a_quarter_kept():
    for H, W in [(34, 60), (48, 84)]:
        Hk, Wk = O.keep_dims(H, W)
        frac = Hk * Wk / (H * W)
        assert 0.24 < frac < 0.30


@pytest.mark.parametrize("n", range(1, 40))
@pytest.mark.parametrize("s", [2, 3, 4])
def test_edges_always_kept(n, s):
    k = O.keep_axis(n, s)
    assert k[0] == 0 and k[-1] == n - 1
    assert k == sorted(set(k))
    assert all(r in k for r in range(0, n, s))


def test_stride2_closed_form():
    for n in range(1, 50):
        nk = O.nearest_axis(n, 2)
        assert nk == [r - (1 if (r % 2 == 1 and r != n - 1) else 0) for r in range(n)]


def _brute_nearest_slot(T, H, W, s, metric):
    kh, kw = O.keep_axis(H, s), O.keep_axis(W, s)
    kept = [(a, b) for a in kh for b in kw]           # raster order within a frame
    out = []
    for t in range(T):
        for h in range(H):
            for w in range(W):
                best = None
                for j, (a, b) in enumerate(kept):
                    if metric == "l2":
                        dist = (h - a) ** 2 + (w - b) ** 2
                    else:
                        dist = abs(h - a) + abs(w - b)
                    key = (dist, a, b)              # lexicographic tie: lower row, then lower column
                    if best is None or key < best[0]:
                        best = (key, j)
                out.append(t * len(kept) + best[1])
    return np.asarray(out, dtype=np.int32)


@pytest.mark.parametrize("s", [2, 3, 4])
@pytest.mark.parametrize("metric", ["l2", "l1"])
def test_nearest_map_brute_force(s, metric):
    for H, W in itertools.product(range(1, 17), range(1, 17)):
        if (H * W) % 3 and H > 4 and W > 4 and (H + W) % 2:   # thin the sweep, keep every small grid
            continue
        got = O.nearest_kept_map(2, H, W, s)
        ref = _brute_nearest_slot(2, H, W, s, metric)
        assert np.array_equal(got, ref), (H, W, s, metric)


def test_keep_index_brute_force():
    for T, H, W, s in [(1, 1, 1, 2), (2, 9, 15, 2), (3, 4, 5, 2), (2, 16, 7, 4), (1, 5, 5, 1)]:
        kh, kw = O.keep_axis(H, s), O.keep_axis(W, s)
        ref = []
        for p in range(T * H * W):
            t, r = divmod(p, H * W)
            h, w = divmod(r, W)
            if h in kh and w in kw:
                ref.append(p)
        assert np.array_equal(O.keep_index(T, H, W, s), np.asarray(ref, dtype=np.int32))


def test_kept_positions_map_to_themselves_and_same_frame():
    T, H, W = 3, 34, 60
    keep = O.keep_index(T, H, W)
    nk = O.nearest_kept_map(T, H, W)
    assert np.array_equal(nk[keep], np.arange(len(keep)))
    frame_of_pos = np.arange(T * H * W) // (H * W)
    frame_of_slot = keep[nk] // (H * W)
    assert np.array_equal(frame_of_pos, frame_of_slot)
    coords = O.kept_coords(T, H, W)
    assert np.array_equal(coords[:, 0] * H * W + coords[:, 1] * W + coords[:, 2], keep)


def test_stride1_is_identity():
    T, H, W = 2, 7, 5
    assert np.array_equal(O.keep_index(T, H, W, 1), np.arange(T * H * W))
    assert np.array_equal(O.nearest_kept_map(T, H, W, 1), np.arange(T * H * W))


def test_degenerate_axes_not_compressed():
    # H or W in {1, 2}: every index is an edge, so nothing is dropped on that axis.
    for n in (1, 2):
        assert O.keep_axis(n, 2) == list(range(n))
    assert len(O.keep_index(1, 2, 2)) == 4
