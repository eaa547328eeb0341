"""Large maps, checked through properties that hold at any size.

A 4096 x 4096 pair (16.8 M pixels per map, 805 MB each in fp16; 5,462 reference
chunks per sweep) in which image 2 is image 1 shifted without noise: every seed
whose shifted pixel lies inside image 2 must end on (s, s - dx - dy * W) in its
first iteration (the true counterpart is the only score near 1; random unit
rows stay far below). Exercises pixel indices up to 2^24 and the chunk and
partial bookkeeping of maps far larger than the oracle can sweep.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def test_frm_4096x4096_pure_shift(ddm):
    import torch
    from synth.torchio import to_device
    H = W = 4096
    dx, dy = 7, -5
    p = synth.large_shift_pair(H, W, 24, synth.F16, 77, (dx, dy))
    print(f"4096x4096x24 f16 pure shift {dx},{dy}: maps built", flush=True)
    D1, D2 = to_device(p.D1, p.dtype, "cuda"), to_device(p.D2, p.dtype, "cuda")
    del p
    S = 128
    i, j, s, st = ddm.frm_match(D1, D2, S, 10, return_state=True)
    state = st["state"].cpu().numpy()
    seeds = oracle.seed_grid(H, W, S)
    assert len(seeds) == 32 * 32 and state.shape[0] == len(seeds)
    x, y = seeds % W, seeds // W
    inside = (x - dx >= 0) & (x - dx < W) & (y - dy >= 0) & (y - dy < H)
    assert inside.sum() == len(seeds)             # the stride-128 grid stays clear of the borders
    assert np.array_equal(state[:, 0], seeds)
    assert np.array_equal(state[:, 1], seeds - dx - dy * W)
    assert (state[:, 2] == 1).all()
    assert np.array_equal(i.cpu().numpy(), seeds) and np.array_equal(j.cpu().numpy(), seeds - dx - dy * W)
    # the score of each pair is its own squared norm in fp32 (within fp16 rounding of unit rows)
    assert np.abs(s.cpu().numpy() - 1.0).max() < 5e-3
    qc = st["query_counts"].cpu().numpy()
    assert qc[0] == len(seeds) and qc[1] == len(seeds) and (qc[2:] == 0).all()
    del D1, D2
    torch.cuda.empty_cache()


def test_frm_at_the_pixel_limit_pure_shift(ddm):
    """Maps of 8192 x 16384 = 2^27 pixels, the per-map limit (6.4 GB each in fp16; 43,691
    reference chunks), drawn on the device: every seed of a stride-512 grid ends on its
    shifted counterpart in iteration 1."""
    import torch
    H, W = 8192, 16384
    dx, dy = 5, -3
    D1, D2 = synth.large_shift_pair_device(H, W, 24, synth.F16, 91, (dx, dy), "cuda")
    print(f"{H}x{W}x24 f16 pure shift {dx},{dy}: maps drawn on the device", flush=True)
    S = 512
    i, j, s, st = ddm.frm_match(D1, D2, S, 4, return_state=True)
    state = st["state"].cpu().numpy()
    seeds = oracle.seed_grid(H, W, S)
    assert len(seeds) == 16 * 32 and state.shape[0] == len(seeds)
    assert seeds.max() > (1 << 26)
    assert np.array_equal(state[:, 0], seeds)
    assert np.array_equal(state[:, 1], seeds - dx - dy * W)
    assert (state[:, 2] == 1).all()
    assert np.array_equal(i.cpu().numpy(), seeds) and np.array_equal(j.cpu().numpy(), seeds - dx - dy * W)
    assert np.abs(s.cpu().numpy() - 1.0).max() < 5e-3
    del D1, D2
    torch.cuda.empty_cache()
