"""GPU parity of the Euclidean metric (3D points) against the oracle: NN, mutual
and FRM, called through ddm_nn_ex / ddm_mutual_nn_ex / ddm_frm_match_ex.

Rule (tau = 1e-4, in squared-distance units): where the oracle's margin
(second-nearest minus nearest squared distance) is >= tau the GPU index equals
the oracle's; otherwise the GPU point must be within tau of the nearest squared
distance. Reported scores are squared distances within tau of the exact ones.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import TAU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def sqd(A, B, ii, jj):
    A = A.reshape(-1, 3).astype(np.float64); B = B.reshape(-1, 3).astype(np.float64)
    return ((A[np.asarray(ii)] - B[np.asarray(jj)]) ** 2).sum(-1)


def check_nn_l2(A, B, qrows, g_idx, g_d2):
    o_idx, s1, m = oracle.nn(A.reshape(-1, 3).astype(np.float64), B.reshape(-1, 3).astype(np.float64),
                             qrows=qrows, metric="l2")
    rows = np.arange(len(g_idx)) if qrows is None else qrows
    sharp = m >= TAU
    assert np.array_equal(g_idx[sharp], o_idx[sharp]), np.nonzero(g_idx[sharp] != o_idx[sharp])[0][:5]
    d2 = sqd(A, B, rows, g_idx)
    assert np.all(d2 <= -s1 + TAU)
    assert np.abs(g_d2 - d2).max() <= TAU
    return int((~sharp).sum())


def test_nn_l2_random_points_and_ties(ddm):
    rng = np.random.default_rng(91)
    B = rng.standard_normal((5000, 3)).astype(np.float32)
    B[4000] = B[17]; B[4500] = B[17]                  # duplicates: the lowest index wins
    A = np.concatenate([B[[17, 4000, 9]], rng.standard_normal((2997, 3)).astype(np.float32)])
    idx, d2 = ddm.nn(cuda(A), cuda(B), metric="l2")
    idx, d2 = idx.cpu().numpy(), d2.cpu().numpy()
    assert idx[0] == 17 and idx[1] == 17 and idx[2] == 9 and d2[0] <= TAU
    amb = check_nn_l2(A, B, None, idx, d2)
    rows = rng.choice(3000, 500, replace=False).astype(np.int32)
    import torch
    gi, gd = ddm.nn(cuda(A), cuda(B), q_rows=torch.from_numpy(rows).cuda(), metric="l2")
    check_nn_l2(A, B, rows, gi.cpu().numpy(), gd.cpu().numpy())
    print(f"ambiguous queries: {amb}")


@pytest.mark.parametrize("shape,shift,sigma", [((64, 48), (3, -2), 0.002), ((96, 80), (-5, 4), 0.0),
                                               ((40, 56), (0, 0), 0.004)])
def test_mutual_l2_pointmaps(ddm, shape, shift, sigma):
    H, W = shape
    P1, P2 = synth.pointmap_pair(H, W, 92 + H, shift=shift, sigma=sigma)
    gi, gj, gs, nn12, s12 = ddm.mutual_nn(cuda(P1), cuda(P2), return_nn=True, metric="l2")
    gi, gj, gs = gi.cpu().numpy(), gj.cpu().numpy(), gs.cpu().numpy()
    A = P1.astype(np.float64).reshape(-1, 3); B = P2.astype(np.float64).reshape(-1, 3)
    ref = oracle.mutual(A, B, metric="l2")
    check_nn_l2(P1, P2, None, nn12.cpu().numpy(), s12.cpu().numpy())
    gpu = set(zip(gi.tolist(), gj.tolist()))
    ref_set = set(zip(ref["i"].tolist(), ref["j"].tolist()))
    sharp = {(i, j) for i, j in ref_set if ref["m12"][i] >= TAU and ref["m21"][j] >= TAU}
    assert sharp <= gpu
    for i, j in gpu - ref_set:
        d2 = sqd(P1, P2, [i], [j])[0]
        assert d2 <= -ref["s12"][i] + TAU and d2 <= -ref["s21"][j] + TAU
    assert np.abs(gs - sqd(P1, P2, gi, gj)).max() <= TAU
    assert len(gpu) > H * W // 3
    print(f"{shape}: pairs gpu {len(gpu)} oracle {len(ref_set)} sharp {len(sharp)}")


@pytest.mark.parametrize("it,tol,basin", [(1, 0.0, False), (1, 1.5, True), (5, 0.0, False)])
def test_frm_l2_explicit_starts(ddm, it, tol, basin):
    import torch
    H, W = 96, 72
    P1, P2 = synth.pointmap_pair(H, W, 93, shift=(4, 3), sigma=0.003)
    starts = np.random.default_rng(it).integers(0, H * W, 1500)
    A = P1.astype(np.float64).reshape(-1, 3); B = P2.astype(np.float64).reshape(-1, 3)
    ref = oracle.frm_ex(A, B, H, W, starts=starts, max_iter=it, pixel_tol=tol, ret_basin=basin, metric="l2")
    out = ddm.frm_match_ex(cuda(P1), cuda(P2), starts=torch.from_numpy(starts).cuda(), max_iter=it,
                           pixel_tol=tol, ret_basin=basin, return_state=True, metric="l2")
    st = out[-1]["state"].cpu().numpy()
    ok = ~ref["ambiguous"]
    for col, key in ((0, "u"), (1, "v"), (2, "conv_iter"), (3, "u_old")):
        assert np.array_equal(st[ok, col], ref[key][ok]), key
    gi, gj, gs = (t.cpu().numpy() for t in out[:3])
    if not ref["ambiguous"].any():
        assert gi.tolist() == ref["i"].tolist() and gj.tolist() == ref["j"].tolist()
        if basin:
            assert np.array_equal(out[3].cpu().numpy(), ref["basin"])
    assert np.abs(gs - sqd(P1, P2, gi, gj)).max() <= TAU
    print(f"it={it} tol={tol}: seeds {ref['seeds'].size} pairs {len(gi)} ambiguous {int(ref['ambiguous'].sum())}")


def test_frm_l2_grid_pure_shift(ddm):
    dx, dy, H, W = 3, -2, 64, 48
    P1, P2 = synth.pointmap_pair(H, W, 94, shift=(dx, dy))
    i, j, s = ddm.frm_match_ex(cuda(P1), cuda(P2), grid_stride=4, max_iter=10, metric="l2")
    seeds = oracle.seed_grid(H, W, 4)
    inside = [q for q in seeds.tolist() if 0 <= q % W - dx < W and 0 <= q // W - dy < H]
    got = dict(zip(i.cpu().tolist(), j.cpu().tolist()))
    for q in inside:
        assert got.get(q) == q - dx - dy * W
    assert float(s.max()) <= TAU
