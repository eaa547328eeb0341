"""GPU parity of FRM with the routine's options (explicit starts, pixel_tol,
basin map), called through ddm_frm_match_ex, against the oracle's frm_ex.

When no seed of a case met a top-1/top-2 margin below tau on its path, every
output must be identical (pairs, scores within tau, per-seed state including
u_old, query counts, basin map). Otherwise the seeds whose path stayed sharp
must agree and the pair set must follow from the GPU's own seed states by the
selection rule.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from parity import TAU, exact_scores

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def dev(a, dtype):
    from synth.torchio import to_device
    return to_device(a, dtype, "cuda")


def _angle_map(deg):
    a = np.radians(np.asarray(deg, dtype=np.float64))
    return np.stack([np.cos(a), np.sin(a)], axis=-1).astype(np.float32)


@pytest.mark.parametrize("case", range(8))
def test_handworked_fixture_on_gpu(ddm, case):
    import torch
    g = json.load(open(os.path.join(GOLD, "frm_starts_tol_basin.json")))
    c = g["cases"][case]
    D1 = torch.from_numpy(_angle_map(g["D1_degrees"]).reshape(g["H1"], g["W1"], 2)).cuda()
    D2 = torch.from_numpy(_angle_map(g["D2_degrees"]).reshape(g["H2"], g["W2"], 2)).cuda()
    starts = torch.tensor(g["starts"], dtype=torch.int32, device="cuda")
    out = ddm.frm_match_ex(D1, D2, starts=starts, max_iter=c["max_iter"], pixel_tol=c["pixel_tol"],
                           ret_basin=c["ret_basin"], return_state=True)
    i, j = out[0].cpu().tolist(), out[1].cpu().tolist()
    st = out[-1]["state"].cpu().numpy()
    assert [list(p) for p in zip(i, j)] == c["pairs"], c["name"]
    assert st[:, 0].tolist() == c["u"] and st[:, 1].tolist() == c["v"], c["name"]
    assert st[:, 2].tolist() == c["conv_iter"] and st[:, 3].tolist() == c["u_old"], c["name"]
    qc = out[-1]["query_counts"].cpu().numpy()
    assert qc[0::2].tolist() == c["n_fwd"] and qc[1::2].tolist() == c["n_bwd"], c["name"]
    if c["ret_basin"]:
        assert out[3].cpu().tolist() == c["basin"], c["name"]


def _compare(A, B, H1, W1, out, ref, tol, basin):
    gi, gj, gs = (t.cpu().numpy() for t in out[:3])
    st = out[-1]["state"].cpu().numpy()
    k = ref["seeds"].size
    st = st[:k]
    amb = ref["ambiguous"]
    ok = ~amb
    for col, key in ((0, "u"), (1, "v"), (2, "conv_iter"), (3, "u_old")):
        bad = np.nonzero(ok & (st[:, col] != ref[key]))[0]
        assert bad.size == 0, (key, bad[:5], st[bad[:5]], ref[key][bad[:5]])
    np.testing.assert_allclose(gs, exact_scores(A, B, gi, gj), atol=TAU, rtol=0)
    assert np.all(np.diff(gi) > 0)
    # the GPU pairs are its own seed states through the selection rule
    u, v, it, uold = st[:, 0], st[:, 1], st[:, 2], st[:, 3]
    if tol > 0:
        dist = np.hypot(uold // W1 - u // W1, uold % W1 - u % W1)
        keep, rep = dist < tol, uold
    else:
        keep, rep = it >= 0, u
    assert sorted(set(zip(rep[keep].tolist(), v[keep].tolist()))) == list(zip(gi.tolist(), gj.tolist()))
    if not amb.any():
        assert gi.tolist() == ref["i"].tolist() and gj.tolist() == ref["j"].tolist()
        qc = out[-1]["query_counts"].cpu().numpy()
        assert qc[0::2].tolist() == ref["n_fwd"].tolist() and qc[1::2].tolist() == ref["n_bwd"].tolist()
        if basin:
            assert np.array_equal(out[3].cpu().numpy(), ref["basin"])
    elif basin:
        gb = out[3].cpu().numpy()
        both = (gb >= 0) & (ref["basin"] >= 0)
        p = np.nonzero(both)[0]
        # a basin entry is f(p) = NN1(NN2(p)); compare where both queries are sharp
        j2, _, m2 = oracle.nn(A, B, qrows=p.astype(np.int32))
        i1, _, m1 = oracle.nn(B, A, qrows=j2.astype(np.int32))
        sharp = (m2 >= TAU) & (m1 >= TAU)
        assert np.array_equal(gb[p][sharp], ref["basin"][p][sharp])
    return int(amb.sum())


CASES = [
    # (config, max_iter, pixel_tol, basin, n_starts)
    ("tiny_frm_64x48x24_f32", 1, 0.0, False, 400),
    ("tiny_frm_64x48x24_f32", 1, 1.5, True, 400),
    ("tiny_frm_64x48x24_f32", 3, 2.5, False, 3000),
    ("tiny_frm_64x48x24_f32", 10, 0.0, True, 1000),
    ("frm_512x384x24_f16", 1, 0.0, False, 5000),
    ("frm_512x384x24_f16", 1, 2.0, False, 5000),
    ("frm_512x384x24_f16", 4, 3.0, True, 3000),
    ("hard_frm_512x512x64_bf16", 1, 4.0, True, 2000),
]


@pytest.mark.parametrize("name,it,tol,basin,n", CASES)
def test_explicit_starts_against_oracle(ddm, name, it, tol, basin, n):
    (p,) = synth.make_config(name)
    N1 = p.H1 * p.W1
    rng = np.random.default_rng(n + it)
    starts = rng.integers(0, N1, size=n)
    starts[:7] = starts[7:14]                      # duplicates
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    ref = oracle.frm_ex(A, B, p.H1, p.W1, starts=starts, max_iter=it, pixel_tol=tol, ret_basin=basin)
    import torch
    out = ddm.frm_match_ex(dev(p.D1, p.dtype), dev(p.D2, p.dtype), starts=torch.tensor(starts, device="cuda"),
                           max_iter=it, pixel_tol=tol, ret_basin=basin, return_state=True)
    amb = _compare(A, B, p.H1, p.W1, out, ref, tol, basin)
    print(f"{name} it={it} tol={tol} basin={basin}: seeds={ref['seeds'].size} pairs={len(out[0])} ambiguous={amb}")


def test_grid_basin_against_oracle(ddm):
    (p,) = synth.make_config("frm_512x384x24_f16")
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    ref = oracle.frm_ex(A, B, p.H1, p.W1, grid_stride=8, max_iter=10, ret_basin=True)
    out = ddm.frm_match_ex(dev(p.D1, p.dtype), dev(p.D2, p.dtype), grid_stride=8, max_iter=10, ret_basin=True,
                           return_state=True)
    _compare(A, B, p.H1, p.W1, out, ref, 0.0, True)


def test_invalid_starts_are_ignored_and_empty_lists(ddm):
    import torch
    (p,) = synth.make_config("tiny_frm_64x48x24_f32")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    N1 = p.H1 * p.W1
    good = torch.tensor([5, 700, 3071, 12, 700], dtype=torch.int32, device="cuda")
    noisy = torch.tensor([-1, 5, N1, 700, 3071, -70000, 12, N1 + 9, 700], dtype=torch.int32, device="cuda")
    a = ddm.frm_match_ex(D1, D2, starts=good, max_iter=2, pixel_tol=1.0, return_state=True)
    b = ddm.frm_match_ex(D1, D2, starts=noisy, max_iter=2, pixel_tol=1.0, return_state=True)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    sa, sb = a[-1]["state"], b[-1]["state"]
    assert sa.shape[0] == 4 and torch.equal(sa, sb)
    e = ddm.frm_match_ex(D1, D2, starts=torch.zeros(0, dtype=torch.int32, device="cuda"), max_iter=1)
    assert all(t.numel() == 0 for t in e[:3])
    xy = ddm.frm_match_ex(D1, D2, starts=(good % p.W1, good // p.W1), max_iter=2, pixel_tol=1.0)
    for x, y in zip(a[:3], xy[:3]):
        assert torch.equal(x, y)


def test_options_in_loop_and_tail_modes_equal_per_half_step(ddm):
    import torch
    (p,) = synth.make_config("frm_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    starts = torch.tensor(np.random.default_rng(5).integers(0, p.H1 * p.W1, 2500), device="cuda")
    runs = []
    try:
        for mode, after in ((ddm.FRM_PER_HALF_STEP, 2), (ddm.FRM_LOOP, 2), (ddm.FRM_TAIL, 2), (ddm.FRM_TAIL, 0)):
            ddm.frm_set_mode(mode)
            ddm.frm_set_tail_after(after)
            runs.append(ddm.frm_match_ex(D1, D2, starts=starts, max_iter=5, pixel_tol=2.0, ret_basin=True,
                                         return_state=True))
    finally:
        ddm.frm_set_mode(ddm.FRM_DEFAULT)
        ddm.frm_set_tail_after(-1)
    a = runs[0]
    for b in runs[1:]:
        for x, y in zip(a[:4], b[:4]):
            assert torch.equal(x, y)
        assert torch.equal(a[-1]["state"], b[-1]["state"])
        assert torch.equal(a[-1]["query_counts"], b[-1]["query_counts"])
