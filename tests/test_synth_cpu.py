"""Seeded input generators (no method arithmetic): the relations the GPU property tests rely on."""
import numpy as np

import synth


def test_large_shift_pair_is_an_exact_shift():
    H, W, dx, dy = 40, 56, 7, -5
    p = synth.large_shift_pair(H, W, 8, synth.F16, 3, (dx, dy))
    assert p.D1.dtype == np.float16 and p.D1.shape == (H, W, 8) and p.D2.shape == (H, W, 8)
    ys, xs = np.mgrid[0:H, 0:W]
    inside = (xs + dx >= 0) & (xs + dx < W) & (ys + dy >= 0) & (ys + dy < H)
    src = p.D1[np.clip(ys + dy, 0, H - 1), np.clip(xs + dx, 0, W - 1)]
    assert np.array_equal(p.D2[inside], src[inside])
    # fresh rows elsewhere, and every row near unit norm
    assert not np.array_equal(p.D2[~inside], src[~inside])
    n = np.linalg.norm(p.D2.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 2e-3
    again = synth.large_shift_pair(H, W, 8, synth.F16, 3, (dx, dy))
    assert np.array_equal(again.D1, p.D1) and np.array_equal(again.D2, p.D2)
