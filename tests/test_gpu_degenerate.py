"""Degenerate inputs on the GPU against the oracle.

Constant and all-zero maps make every score tie. Equal stored rows give
bit-identical dot products on the matrix cores (fp32) and in the oracle
(fp64), so both sides must break every tie the same way, at the lowest index,
across chunks, index groups and slots: the results are compared exactly.
Single-row and single-column maps and a one-pixel image 2 go through the usual
parity rules.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_frm, check_mutual, check_nn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def dev(a, dtype):
    from synth.torchio import to_device
    return to_device(a, dtype, "cuda")


def constant_map(H, W, d, dtype, value_seed):
    """Every pixel holds the same unit descriptor (all zero when value_seed is None)."""
    if value_seed is None:
        return synth.cast_stored(np.zeros((H, W, d)), dtype)
    row = synth.gaussian_rows(1, d, synth.F32, value_seed)[0].astype(np.float64)
    return synth.cast_stored(np.broadcast_to(row, (H, W, d)).copy(), dtype)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16, synth.F32])
@pytest.mark.parametrize("value_seed", [7, None], ids=["constant", "zero"])
def test_all_ties(ddm, dtype, value_seed):
    H, W, d = 96, 80, 24            # 7680 pixels: several reference chunks of the sweep
    D = constant_map(H, W, d, dtype, value_seed)
    A = oracle.decode(D, dtype)
    # NN: every query ties over all references -> reference 0
    idx, s = ddm.nn(dev(D.reshape(H * W, d), dtype), dev(D.reshape(H * W, d), dtype))
    o_idx, o_s, _ = oracle.nn(A, A)
    assert (o_idx == 0).all()
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(s.cpu().numpy(), o_s, rtol=0, atol=1e-6)
    # FRM: every seed goes to (0, 0) in its second iteration
    i, j, sc, st = ddm.frm_match(dev(D, dtype), dev(D, dtype), 8, 10, return_state=True)
    seeds = oracle.seed_grid(H, W, 8)
    r = oracle.frm(A, A, seeds, 10)
    state = st["state"].cpu().numpy()
    assert np.array_equal(state[:, 0], r["u"]) and np.array_equal(state[:, 1], r["v"])
    assert np.array_equal(state[:, 2], r["conv_iter"])
    assert i.cpu().numpy().tolist() == r["i"].tolist() == [0]
    assert j.cpu().numpy().tolist() == r["j"].tolist() == [0]
    # mutual: only (0, 0)
    mi, mj, ms, nn12, _ = ddm.mutual_nn(dev(D, dtype), dev(D, dtype), return_nn=True)
    m = oracle.mutual(A, A)
    assert np.array_equal(nn12.cpu().numpy(), m["nn12"])
    assert mi.cpu().numpy().tolist() == m["i"].tolist() == [0]
    assert mj.cpu().numpy().tolist() == m["j"].tolist() == [0]


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_constant_references_random_queries(ddm, dtype):
    """Image 2 constant: every image-1 pixel's NN is reference 0; the reverse NN
    of reference 0 is the best image-1 pixel, which every seed reaches."""
    D1 = synth.random_map(64, 96, 24, dtype, 21)
    D2 = constant_map(64, 96, 24, dtype, 22)
    A, B = oracle.decode(D1, dtype), oracle.decode(D2, dtype)
    seeds = oracle.seed_grid(64, 96, 4)
    r = oracle.frm(A, B, seeds, 10)
    i, j, s, st = ddm.frm_match(dev(D1, dtype), dev(D2, dtype), 4, 10, return_state=True)
    state = st["state"].cpu().numpy()
    assert np.array_equal(state[:, 1], r["v"]) and (r["v"] == 0).all()
    best = int(np.argmax(A.reshape(-1, 24) @ B.reshape(-1, 24)[0]))
    assert i.cpu().numpy().tolist() == [best] and j.cpu().numpy().tolist() == [0]
    mi, mj, ms = ddm.mutual_nn(dev(D1, dtype), dev(D2, dtype))
    assert mi.cpu().numpy().tolist() == [best] and mj.cpu().numpy().tolist() == [0]


@pytest.mark.parametrize("shape1,shape2", [((1, 700), (1, 650)), ((700, 1), (640, 1)), ((40, 30), (1, 1)),
                                           ((1, 1), (33, 47))])
def test_thin_and_single_pixel_maps(ddm, shape1, shape2):
    dt = synth.F16
    D1 = synth.random_map(*shape1, 24, dt, 31)
    D2 = synth.random_map(*shape2, 24, dt, 32)
    A, B = oracle.decode(D1, dt), oracle.decode(D2, dt)
    S = 1 if min(shape1) == 1 else 3          # a one-pixel-wide map has grid seeds only at stride 1
    seeds = oracle.seed_grid(*shape1, S)
    i, j, s, st = ddm.frm_match(dev(D1, dt), dev(D2, dt), S, 10, return_state=True)
    assert st["state"].shape[0] == len(seeds)
    if len(seeds):
        check_frm(A, B, st["state"].cpu().numpy(), i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy(), seeds, 10)
    else:
        assert i.numel() == 0
    mi, mj, ms, nn12, s12 = ddm.mutual_nn(dev(D1, dt), dev(D2, dt), return_nn=True)
    check_nn(A, B, None, nn12.cpu().numpy(), s12.cpu().numpy())
    check_mutual(A, B, mi.cpu().numpy(), mj.cpu().numpy(), ms.cpu().numpy())
