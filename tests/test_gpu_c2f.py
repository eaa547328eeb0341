"""GPU parity of coarse-to-fine crop matching (ddm_c2f_match) against the
oracle's reading: crop windows, and the merged full-resolution pairs.

When no coarse or fine seed met a margin below tau, the crop windows and the
pairs must be identical; otherwise the crop windows of tiles whose coarse pairs
all stayed sharp must agree, and every GPU pair must be reciprocal inside its
crop pair within tau.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import TAU, exact_scores, near_reciprocal_many

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def dev(a, dtype):
    from synth.torchio import to_device
    return to_device(a, dtype, "cuda")


CASES = [
    # (H, W, d, dtype, seed, shift, sigma, factor, coarse stride, crop (h, w), fine stride)
    (256, 192, 24, synth.F16, 301, (12, -8), 0.1, 2, 4, (128, 96), 4),
    (300, 200, 24, synth.F16, 302, (-10, 6), 0.1, 2, 4, (128, 96), 4),       # overlapping tiles
    (192, 160, 16, synth.BF16, 303, (8, 8), 0.05, 4, 2, (96, 64), 4),
    (160, 128, 8, synth.F32, 304, (0, 0), 0.0, 2, 4, (160, 128), 4),         # one crop = the whole map
    (1024, 768, 24, synth.F16, 305, (34, -18), 0.1, 2, 8, (512, 384), 8),    # 4 crops of the benchmark size
]


@pytest.mark.parametrize("H,W,d,dt,seed,shift,sigma,factor,cs,crop,fs", CASES)
def test_c2f_against_oracle(ddm, H, W, d, dt, seed, shift, sigma, factor, cs, crop, fs):
    p = synth.make_pair(H, W, d, dt, seed, sigma=sigma, shift=shift)
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    ref = oracle.coarse_to_fine(A, B, factor=factor, coarse_stride=cs, coarse_iter=10, crop_h=crop[0],
                                crop_w=crop[1], fine_stride=fs, fine_iter=10)
    gi, gj, gs, crops = ddm.c2f_match(dev(p.D1, p.dtype), dev(p.D2, p.dtype), factor=factor, coarse_stride=cs,
                                      coarse_iter=10, crop=crop, fine_stride=fs, fine_iter=10, return_crops=True)
    gi, gj, gs, crops = (t.cpu().numpy() for t in (gi, gj, gs, crops))
    # ambiguity of the coarse stage: the oracle's coarse FRM on the subsampled maps
    C1 = A[::factor, ::factor]; C2 = B[::factor, ::factor]
    cr = oracle.frm(np.ascontiguousarray(C1), np.ascontiguousarray(C2),
                    oracle.seed_grid(C1.shape[0], C1.shape[1], cs), 10)
    coarse_sharp = not cr["ambiguous"].any()
    fine_sharp = all(f is None or not f["ambiguous"].any() for f in ref["fine"])
    if coarse_sharp:
        assert [tuple(c) for c in crops.tolist()] == ref["crops"]
    assert np.all(np.diff(gi) > 0)
    np.testing.assert_allclose(gs, exact_scores(A, B, gi, gj), atol=TAU, rtol=0)
    if coarse_sharp and fine_sharp:
        assert gi.tolist() == ref["i"].tolist() and gj.tolist() == ref["j"].tolist()
    else:
        # every GPU pair is reciprocal (within tau) inside a tile of its image-1 pixel whose image-2
        # window holds its image-2 pixel; all pairs are checked, one batch of oracle queries per tile
        Wi, Wj = A.shape[1], B.shape[1]
        xi, yi, xj, yj = gi % Wi, gi // Wi, gj % Wj, gj // Wj
        ok = np.zeros(len(gi), bool)
        for (x01, y01, x02, y02, n) in crops.tolist():
            if not n:
                continue
            inside = (~ok & (xi >= x01) & (xi < x01 + crop[1]) & (yi >= y01) & (yi < y01 + crop[0])
                      & (xj >= x02) & (xj < x02 + crop[1]) & (yj >= y02) & (yj < y02 + crop[0]))
            sel = np.nonzero(inside)[0]
            if sel.size == 0:
                continue
            ca = np.ascontiguousarray(A[y01:y01 + crop[0], x01:x01 + crop[1]]).reshape(-1, d)
            cb = np.ascontiguousarray(B[y02:y02 + crop[0], x02:x02 + crop[1]]).reshape(-1, d)
            li = ((yi[sel] - y01) * crop[1] + (xi[sel] - x01)).astype(np.int32)
            lj = ((yj[sel] - y02) * crop[1] + (xj[sel] - x02)).astype(np.int32)
            ok[sel] = near_reciprocal_many(ca, cb, li, lj)
        bad = np.nonzero(~ok)[0]
        assert bad.size == 0, f"{bad.size} GPU pairs not reciprocal in any covering crop, e.g. {list(zip(gi[bad[:5]], gj[bad[:5]]))}"
    print(f"{H}x{W}: tiles {len(crops)} pairs gpu {len(gi)} oracle {len(ref['i'])} "
          f"coarse sharp {coarse_sharp} fine sharp {fine_sharp}")


def test_c2f_rejects_bad_sizes(ddm):
    import torch
    x = torch.zeros(64, 48, 24, dtype=torch.float16, device="cuda")
    with pytest.raises(ddm.DDMError):
        ddm.c2f_match(x, x, crop=(65, 48))
    y = torch.zeros(64, 48, 23, dtype=torch.float16, device="cuda")
    with pytest.raises(ddm.DDMError):
        ddm.c2f_match(y, y, crop=(32, 24))


@pytest.mark.parametrize("case", [0, 2, 4])
def test_c2f_output_paths_agree(ddm, case):
    """The coarse and the fine FRM inside coarse-to-fine through the one-workgroup bitmap output
    and through the multi-workgroup compaction: identical pairs, scores and crop windows."""
    H, W, d, dt, seed, shift, sigma, factor, cs, crop, fs = CASES[case]
    p = synth.make_pair(H, W, d, dt, seed, sigma=sigma, shift=shift)
    F1, F2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    runs = []
    try:
        for limit in (-1, 0):
            ddm.debug_set_output_bitmap_limit(limit)
            runs.append([t.cpu().numpy() for t in ddm.c2f_match(F1, F2, factor=factor, coarse_stride=cs,
                                                                coarse_iter=10, crop=crop, fine_stride=fs,
                                                                fine_iter=10, return_crops=True)])
    finally:
        ddm.debug_set_output_bitmap_limit(-1)
    assert runs[0][0].size > 100
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
