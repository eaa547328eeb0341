"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against something other than itself: a library
routine (numpy argmax / sort over the full float64 score matrix, numpy's and
torch's float16 / bfloat16 decoders), a closed form, a hand-worked fixture under
tests/golden/, or an invariant the method guarantees. The set is chosen so that
a dropped term, a flipped comparison, a wrong index or a swapped operand in the
oracle fails at least one of them (tests/test_oracle_mutations.py plants such
mistakes and checks exactly that).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _scores(A, B):
    A = A.reshape(-1, A.shape[-1]); B = B.reshape(-1, B.shape[-1])
    return A @ B.T


def _np_nn(A, B):
    """Library pin: numpy argmax returns the first (lowest) index of the maximum."""
    S = _scores(A, B)
    idx = S.argmax(axis=1)
    srt = np.sort(S, axis=1)
    second = srt[:, -2] if S.shape[1] > 1 else np.full(S.shape[0], -np.inf)
    return idx, srt[:, -1], srt[:, -1] - second


# --------------------------------------------------------------------- decode
def test_decode_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.decode(h, oracle.F16)
    ref = h.astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_decode_bf16_all_patterns():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_decode_f32_exact():
    x = synth.gaussian_rows(1000, 7, synth.F32, 5, unit=False)
    assert np.array_equal(oracle.decode(x, oracle.F32), x.astype(np.float64))


# --------------------------------------------------------------------- NN
@pytest.mark.parametrize("nq,nr,d,seed", [(37, 53, 24, 1), (64, 200, 3, 2), (5, 9, 1, 3), (128, 96, 64, 4),
                                          (1, 1, 8, 5), (33, 1, 24, 6)])
def test_nn_matches_numpy_argmax(nq, nr, d, seed):
    Q = synth.gaussian_rows(nq, d, synth.F16, seed).astype(np.float64)
    R = synth.gaussian_rows(nr, d, synth.F16, seed + 100).astype(np.float64)
    idx, s1, m = oracle.nn(Q, R)
    ridx, rs1, rm = _np_nn(Q, R)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(s1, rs1, atol=1e-12, rtol=0)
    if nr > 1:
        np.testing.assert_allclose(m, rm, atol=1e-12, rtol=0)
    else:
        assert np.all(np.isinf(m))


def test_nn_ties_take_lowest_index():
    R = synth.gaussian_rows(40, 24, synth.F16, 11).astype(np.float64)
    R[[7, 19, 33]] = R[25]              # duplicated reference rows
    Q = R[[25, 3, 25]].copy()
    idx, s1, m = oracle.nn(Q, R)
    ridx, _, _ = _np_nn(Q, R)
    assert np.array_equal(idx, ridx)
    assert idx[0] == 7 and idx[2] == 7  # lowest of {7, 19, 25, 33}
    assert m[0] == 0.0 and m[2] == 0.0


def test_nn_gathered_rows():
    Q = synth.gaussian_rows(50, 24, synth.F16, 12).astype(np.float64)
    R = synth.gaussian_rows(70, 24, synth.F16, 13).astype(np.float64)
    rows = np.array([49, 0, 7, 7, 31], np.int32)
    idx, s1, m = oracle.nn(Q, R, qrows=rows)
    ridx, rs1, _ = _np_nn(Q[rows], R)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(s1, rs1, atol=1e-12, rtol=0)


def test_nn_negative_scores_only():
    # every score negative: the maximum is still the least negative one
    R = -np.abs(synth.gaussian_rows(30, 4, synth.F32, 14).astype(np.float64))
    Q = np.abs(synth.gaussian_rows(6, 4, synth.F32, 15).astype(np.float64))
    idx, s1, _ = oracle.nn(Q, R)
    assert np.all(s1 < 0)
    assert np.array_equal(idx, _np_nn(Q, R)[0])


def test_nn_score_is_exact_for_f16_inputs():
    # f16 x f16 products are exact in double; 24 of them sum with error << 1e-12
    Q = synth.gaussian_rows(20, 24, synth.F16, 16)
    R = synth.gaussian_rows(30, 24, synth.F16, 17)
    idx, s1, _ = oracle.nn(oracle.decode(Q, oracle.F16), oracle.decode(R, oracle.F16))
    from fractions import Fraction
    for a in range(3):
        exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(Q[a], R[idx[a]]))
        assert abs(float(exact) - s1[a]) < 1e-15


# --------------------------------------------------------------------- seeds
def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_seed_grid_closed_forms():
    g = _gold("seed_grid.json")
    for c in g["cases"]:
        s = oracle.seed_grid(c["H"], c["W"], c["S"])
        assert s.size == c["k"], c
        if "first" in c:
            assert s[0] == c["first"] and s[-1] == c["last"], c
        if "all" in c:
            assert s.tolist() == c["all"], c
        if s.size:
            assert np.all(np.diff(s) > 0)


# --------------------------------------------------------------------- FRM
def _angle_map(deg):
    a = np.radians(np.asarray(deg, dtype=np.float64))
    return np.stack([np.cos(a), np.sin(a)], axis=-1).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("orient", ["row", "col"])
def test_frm_handworked_fixture(orient):
    g = _gold("frm_handworked.json")
    A = _angle_map(g["angles1_deg"]); B = _angle_map(g["angles2_deg"])
    if orient == "col":       # H x 1 instead of 1 x W: same linear indices
        A = A.reshape(-1, 1, 2); B = B.reshape(-1, 1, 2)
    seeds = np.array(g["seeds"], np.int32)
    for case in g["cases"]:
        r = oracle.frm(A, B, seeds, case["max_iter"])
        assert r["u"].tolist() == case["u"], case
        assert r["v"].tolist() == case["v"], case
        assert r["conv_iter"].tolist() == case["conv_iter"], case
        assert (~r["active"]).tolist() == case["converged"], case
        assert r["i"].tolist() == case["pairs_i"] and r["j"].tolist() == case["pairs_j"], case
        assert r["niter"] == case["niter"]
        assert r["n_fwd"].tolist() == case["n_fwd"] and r["n_bwd"].tolist() == case["n_bwd"], case
        np.testing.assert_allclose(r["s"], np.cos(np.radians(g["mutual"]["angle_diff_deg"])), atol=1e-6)
    m = oracle.mutual(A, B)
    assert m["i"].tolist() == g["mutual"]["i"] and m["j"].tolist() == g["mutual"]["j"]


def _orbit_expectation(A, B, seeds, max_iter):
    """Second, independent derivation of FRM from the full NN tables.

    With f = NN1 o NN2 and m the least depth with f^{m+1}(s) = f^m(s), the seed
    stops in iteration m + 1 (kept iff m + 1 <= max_iter) at (f^m(s), NN2(f^m(s))).
    NN tables come from numpy argmax (lowest index on ties)."""
    nn12 = _np_nn(A, B)[0]; nn21 = _np_nn(B, A)[0]
    out = []
    for s in seeds:
        x, m = int(s), 0
        while True:
            y = int(nn21[nn12[x]])
            if y == x:
                break
            x, m = y, m + 1
            if m > 10 * len(nn12):
                raise AssertionError("orbit without fixed point")
        out.append((x, int(nn12[x]), m + 1))
    return out


@pytest.mark.parametrize("shape1,shape2,d,seed", [((8, 8), (8, 8), 3, 21), ((6, 10), (9, 7), 2, 22),
                                                  ((12, 9), (12, 9), 24, 23), ((16, 16), (10, 20), 4, 24),
                                                  ((1, 40), (40, 1), 2, 25)])
@pytest.mark.parametrize("max_iter", [1, 2, 3, 10])
def test_frm_equals_orbit_derivation(shape1, shape2, d, seed, max_iter):
    A = synth.random_map(*shape1, d, synth.F16, seed).astype(np.float64)
    B = synth.random_map(*shape2, d, synth.F16, seed + 1).astype(np.float64)
    seeds = np.arange(A.shape[0] * A.shape[1], dtype=np.int32)      # every pixel is a seed
    r = oracle.frm(A, B, seeds, max_iter)
    exp = _orbit_expectation(A, B, seeds, max_iter)
    for a, (u_star, v_star, it) in enumerate(exp):
        if it <= max_iter:
            assert not r["active"][a]
            assert r["conv_iter"][a] == it
            assert (r["u"][a], r["v"][a]) == (u_star, v_star)
        else:
            assert r["active"][a] and r["conv_iter"][a] == -1
    # the merged output is exactly the converged states, unique and ascending in i
    conv = ~r["active"]
    pairs = sorted(set(zip(r["u"][conv].tolist(), r["v"][conv].tolist())))
    assert list(zip(r["i"].tolist(), r["j"].tolist())) == pairs


@pytest.mark.parametrize("seed", [31, 32, 33])
def test_frm_pairs_are_reciprocal_and_inside_mutual_set(seed):
    A = synth.random_map(20, 16, 8, synth.F16, seed).astype(np.float64)
    B = synth.random_map(18, 15, 8, synth.F16, seed + 50).astype(np.float64)
    seeds = oracle.seed_grid(20, 16, 2)
    r = oracle.frm(A, B, seeds, 10)
    nn12 = _np_nn(A, B)[0]; nn21 = _np_nn(B, A)[0]
    for i, j in zip(r["i"], r["j"]):
        assert nn12[i] == j and nn21[j] == i
    m = oracle.mutual(A, B)
    M = set(zip(m["i"].tolist(), m["j"].tolist()))
    assert set(zip(r["i"].tolist(), r["j"].tolist())) <= M
    # seeds already in M stop in the first iteration
    for a, s in enumerate(seeds):
        if nn21[nn12[s]] == s:
            assert r["conv_iter"][a] == 1 and r["u"][a] == s


def test_frm_identity_map():
    p = synth.make_pair(24, 16, 24, synth.F16, 41, sigma=0.0, shift=(0, 0))
    assert np.array_equal(p.D1.view(np.uint16), p.D2.view(np.uint16))
    A = oracle.decode(p.D1, oracle.F16); B = oracle.decode(p.D2, oracle.F16)
    seeds = oracle.seed_grid(24, 16, 4)
    r = oracle.frm(A, B, seeds, 10)
    assert np.all(r["conv_iter"] == 1)
    assert np.array_equal(r["u"], seeds) and np.array_equal(r["v"], seeds)
    norms = (A.reshape(-1, 24)[seeds] ** 2).sum(1)
    np.testing.assert_allclose(r["score"], norms, atol=1e-12, rtol=0)


@pytest.mark.parametrize("dx,dy", [(3, 2), (-5, 4), (0, -7)])
def test_frm_pure_shift_closed_form(dx, dy):
    H, W, d = 32, 24, 24
    p = synth.make_pair(H, W, d, synth.F16, 42, sigma=0.0, shift=(dx, dy))
    A = oracle.decode(p.D1, oracle.F16); B = oracle.decode(p.D2, oracle.F16)
    seeds = oracle.seed_grid(H, W, 4)
    r = oracle.frm(A, B, seeds, 10)
    n_checked = 0
    for a, s in enumerate(seeds):
        x, y = s % W, s // W
        if 0 <= x - dx < W and 0 <= y - dy < H:
            assert r["conv_iter"][a] == 1
            assert (r["u"][a], r["v"][a]) == (s, s - dx - dy * W)
            assert abs(r["score"][a] - (A.reshape(-1, d)[s] ** 2).sum()) < 1e-12
            n_checked += 1
    assert n_checked > len(seeds) // 2


def test_frm_no_seeds_and_empty_maps():
    A = synth.random_map(4, 4, 3, synth.F32, 1).astype(np.float64)
    r = oracle.frm(A, A, np.zeros(0, np.int32), 10)
    assert r["i"].size == 0 and r["niter"] == 0
    assert oracle.seed_grid(2, 2, 5).size == 0


# ------------------------------------------------- FRM options: starts, pixel_tol, basin
@pytest.mark.parametrize("case", range(8))
def test_frm_ex_handworked_fixture(case):
    g = _gold("frm_starts_tol_basin.json")
    c = g["cases"][case]
    A = _angle_map(g["D1_degrees"]).reshape(g["H1"], g["W1"], 2)
    B = _angle_map(g["D2_degrees"]).reshape(g["H2"], g["W2"], 2)
    r = oracle.frm_ex(A, B, g["H1"], g["W1"], starts=np.array(g["starts"]), max_iter=c["max_iter"],
                      pixel_tol=c["pixel_tol"], ret_basin=c["ret_basin"])
    assert r["seeds"].tolist() == sorted(set(g["starts"])), c["name"]
    for key in ("u", "v", "u_old", "conv_iter", "n_fwd", "n_bwd"):
        assert r[key].tolist() == c[key], (c["name"], key, r[key].tolist())
    assert [list(p) for p in zip(r["i"].tolist(), r["j"].tolist())] == c["pairs"], c["name"]
    if c["ret_basin"]:
        assert r["basin"].tolist() == c["basin"], c["name"]
    else:
        assert r["basin"] is None


def _orbit_ex_expectation(A, B, W1, seeds, max_iter, pixel_tol, explicit, basin_mode):
    """Independent derivation of the optioned routine from the NN tables (numpy argmax) and
    the orbit of f = NN1 o NN2: seed s sits at u_t = f^t(s) after t backward steps and
    stops in iteration m_s + 1 (m_s = first t with f(u_t) = u_t) whichever test is on;
    the loop runs iteration max_iter iff some seed is still active when it starts, and
    then u_old = u at its start, else u_old = final u; the basin records f(u_t) at u_t for
    every backward step taken."""
    nn12 = _np_nn(A, B)[0]; nn21 = _np_nn(B, A)[0]
    f = nn21[nn12]
    N1 = len(nn12)
    traj, stop = [], []
    for s in seeds:
        t = [int(s)]
        m = None
        for step in range(max_iter):
            nxt = int(f[t[-1]])
            if nxt == t[-1]:
                m = step
                break
            t.append(nxt)
        traj.append(t)
        stop.append(m + 1 if m is not None else None)      # iteration in which the seed stops
    reached_last = any(st is None or st >= max_iter for st in stop)
    out = dict(u=[], v=[], u_old=[], conv=[], basin=np.full(N1, -1, np.int64), pairs=set())
    for t, st in zip(traj, stop):
        final_u = t[-1]
        last_fwd_from = t[-1] if st is not None else t[-2]
        v = int(nn12[last_fwd_from])
        u_old = t[min(len(t) - 1, max_iter - 1)] if reached_last else final_u
        out["u"].append(final_u); out["v"].append(v); out["u_old"].append(u_old)
        out["conv"].append(st if st is not None else -1)
        n_bwd_steps = min(st if st is not None else max_iter, max_iter)
        if basin_mode:
            for q in range(n_bwd_steps):
                out["basin"][t[q]] = int(f[t[q]])
        if pixel_tol > 0:
            dy, dx = u_old // W1 - final_u // W1, u_old % W1 - final_u % W1
            if (dy * dy + dx * dx) ** 0.5 < pixel_tol:
                out["pairs"].add((u_old if explicit else final_u, v))
        elif st is not None:
            out["pairs"].add((final_u, v))
    return out


@pytest.mark.parametrize("shape,d,seed", [((8, 8), 3, 61), ((6, 10), 2, 62), ((12, 9), 24, 63), ((1, 40), 2, 64)])
@pytest.mark.parametrize("max_iter", [1, 2, 3, 10])
@pytest.mark.parametrize("pixel_tol,basin", [(0.0, False), (0.0, True), (1.0, False), (2.5, False), (1.5, True)])
def test_frm_ex_equals_orbit_derivation(shape, d, seed, max_iter, pixel_tol, basin):
    H1, W1 = shape
    A = synth.random_map(H1, W1, d, synth.F16, seed).astype(np.float64)
    B = synth.random_map(W1, H1, d, synth.F16, seed + 1).astype(np.float64)
    rng = np.random.default_rng(seed)
    starts = rng.integers(0, H1 * W1, size=H1 * W1 // 2 + 3)          # duplicates on purpose
    r = oracle.frm_ex(A, B, H1, W1, starts=starts, max_iter=max_iter, pixel_tol=pixel_tol, ret_basin=basin)
    seeds = np.unique(starts)
    assert np.array_equal(r["seeds"], seeds)
    exp = _orbit_ex_expectation(A, B, W1, seeds, max_iter, pixel_tol, True, basin)
    assert r["u"].tolist() == exp["u"] and r["v"].tolist() == exp["v"]
    assert r["u_old"].tolist() == exp["u_old"] and r["conv_iter"].tolist() == exp["conv"]
    assert list(zip(r["i"].tolist(), r["j"].tolist())) == sorted(exp["pairs"])
    if basin:
        assert r["basin"].tolist() == exp["basin"].tolist()


def test_frm_ex_grid_matches_plain_routine():
    A = synth.random_map(16, 12, 8, synth.F16, 71).astype(np.float64)
    B = synth.random_map(14, 12, 8, synth.F16, 72).astype(np.float64)
    for it in (1, 3, 10):
        a = oracle.frm_ex(A, B, 16, 12, grid_stride=3, max_iter=it)
        b = oracle.frm(A, B, oracle.seed_grid(16, 12, 3), it)
        for key in ("u", "v", "conv_iter", "i", "j", "n_fwd", "n_bwd"):
            assert np.array_equal(a[key], b[key]), key


def test_frm_ex_identity_and_shift_closed_forms():
    # identity: every start is its own reciprocal pair, its basin entry is itself
    p = synth.make_pair(12, 10, 24, synth.F16, 73, sigma=0.0, shift=(0, 0))
    A = oracle.decode(p.D1, oracle.F16); B = oracle.decode(p.D2, oracle.F16)
    starts = np.array([5, 5, 17, 3, 119, 60])
    for tol in (0.0, 0.5):
        r = oracle.frm_ex(A, B, 12, 10, starts=starts, max_iter=1, pixel_tol=tol, ret_basin=True)
        u = np.unique(starts)
        assert r["i"].tolist() == u.tolist() and r["j"].tolist() == u.tolist()
        exp_basin = np.full(120, -1); exp_basin[u] = u
        assert r["basin"].tolist() == exp_basin.tolist()
    # pure shift: a start whose counterpart is in range maps to p - dx - dy*W in one round trip
    dx, dy, H, W = 3, -2, 14, 11
    p = synth.make_pair(H, W, 24, synth.F16, 74, sigma=0.0, shift=(dx, dy))
    A = oracle.decode(p.D1, oracle.F16); B = oracle.decode(p.D2, oracle.F16)
    inside = [q for q in range(H * W) if 0 <= q % W - dx < W and 0 <= q // W - dy < H]
    r = oracle.frm_ex(A, B, H, W, starts=np.array(inside), max_iter=1, pixel_tol=0.5)
    assert r["i"].tolist() == inside
    assert r["j"].tolist() == [q - dx - dy * W for q in inside]


def test_frm_ex_rejects_undefined_requests():
    A = synth.random_map(4, 4, 3, synth.F32, 75).astype(np.float64)
    with pytest.raises(ValueError):
        oracle.frm_ex(A, A, 4, 4, grid_stride=2, pixel_tol=1.0)       # the routine has no grid form of it
    with pytest.raises(ValueError):
        oracle.frm_ex(A, A, 4, 4, starts=np.array([16]))
    with pytest.raises(ValueError):
        oracle.frm_ex(A, A, 4, 4)
    r = oracle.frm_ex(A, A, 4, 4, starts=np.zeros(0, np.int64), max_iter=1)
    assert r["i"].size == 0


# ------------------------------------------------------------ Euclidean metric (3D points)
def _np_nn_l2(A, B):
    """NN by squared Euclidean distance from numpy broadcasting: argmin (first = lowest index)."""
    A = A.reshape(-1, A.shape[-1]).astype(np.float64); B = B.reshape(-1, B.shape[-1]).astype(np.float64)
    D = ((A[:, None, :] - B[None, :, :]) ** 2).sum(-1)
    idx = D.argmin(1)
    srt = np.sort(D, axis=1)
    second = srt[:, 1] if D.shape[1] > 1 else np.full(D.shape[0], np.inf)
    return idx, srt[:, 0], second - srt[:, 0]


def test_l2_nn_matches_kdtree():
    from scipy.spatial import cKDTree
    rng = np.random.default_rng(81)
    A = rng.standard_normal((300, 3)); B = rng.standard_normal((500, 3))
    idx, s1, m = oracle.nn(A, B, metric="l2")
    dist, kidx = cKDTree(B).query(A)
    assert np.array_equal(idx, kidx)
    np.testing.assert_allclose(-s1, dist ** 2, rtol=1e-12, atol=1e-15)
    assert np.all(m > 0)


def test_l2_nn_ties_and_numpy():
    rng = np.random.default_rng(82)
    B = rng.standard_normal((64, 3)).astype(np.float32).astype(np.float64)
    B[40] = B[7]; B[50] = B[7]                       # exact duplicates: lowest index wins
    A = np.concatenate([B[[7, 40, 3]], rng.standard_normal((20, 3))])
    idx, s1, m = oracle.nn(A, B, metric="l2")
    e_idx, e_d2, e_m = _np_nn_l2(A, B)
    assert np.array_equal(idx, e_idx) and idx[0] == 7 and idx[1] == 7
    np.testing.assert_allclose(-s1, e_d2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, e_m, rtol=0, atol=1e-12)
    assert m[0] == 0.0


def test_l2_mutual_matches_numpy():
    P1, P2 = synth.pointmap_pair(10, 12, 83, shift=(2, -1), sigma=0.01)
    A = P1.astype(np.float64); B = P2.astype(np.float64)
    m = oracle.mutual(A, B, metric="l2")
    n12 = _np_nn_l2(A, B)[0]; n21 = _np_nn_l2(B, A)[0]
    exp = [(i, int(j)) for i, j in enumerate(n12) if n21[j] == i]
    assert list(zip(m["i"].tolist(), m["j"].tolist())) == exp
    assert len(exp) > 20


@pytest.mark.parametrize("max_iter", [1, 3, 10])
def test_l2_frm_equals_orbit_derivation(max_iter):
    P1, P2 = synth.pointmap_pair(9, 11, 84, shift=(1, 2), sigma=0.02)
    A = P1.astype(np.float64).reshape(-1, 3); B = P2.astype(np.float64).reshape(-1, 3)
    seeds = np.arange(A.shape[0], dtype=np.int32)
    r = oracle.frm_ex(A, B, 9, 11, starts=seeds, max_iter=max_iter, metric="l2")
    nn12 = _np_nn_l2(A, B)[0]; nn21 = _np_nn_l2(B, A)[0]
    f = nn21[nn12]
    for a, s in enumerate(seeds):
        x, m = int(s), 0
        while f[x] != x and m < max_iter:
            x, m = int(f[x]), m + 1
        if f[x] == x and m + 1 <= max_iter:
            assert r["conv_iter"][a] == m + 1 and r["u"][a] == x and r["v"][a] == nn12[x]
        else:
            assert r["conv_iter"][a] == -1


def test_l2_pure_shift_closed_form():
    dx, dy, H, W = 3, -2, 12, 14
    P1, P2 = synth.pointmap_pair(H, W, 85, shift=(dx, dy))
    A = P1.astype(np.float64); B = P2.astype(np.float64)
    inside = [q for q in range(H * W) if 0 <= q % W - dx < W and 0 <= q // W - dy < H]
    r = oracle.frm_ex(A, B, H, W, starts=np.array(inside), max_iter=1, metric="l2")
    assert r["i"].tolist() == inside and r["j"].tolist() == [q - dx - dy * W for q in inside]
    assert np.all(r["s"] == 0.0)


# ------------------------------------------------------------- coarse-to-fine crops
def test_crop_windows_hand_example():
    """Worked by hand: 10 x 10 image 1, 12 x 8 (H x W) image 2, 4 x 4 crops. Tile offsets 0, 4, 6 on
    both axes (the last tile moved back to the border); lower medians; offsets clamped into image 2."""
    x1 = [1, 2, 3, 5, 9, 9, 8]
    y1 = [1, 2, 0, 1, 9, 8, 5]
    x2 = [7, 2, 5, 0, 3, 4, 7]
    y2 = [1, 9, 4, 9, 6, 5, 11]
    c = oracle.crop_windows(10, 10, 12, 8, 4, 4, x1, y1, x2, y2)
    assert c == [(0, 0, 3, 2, 3),       # pairs 0-2: medians x 5, y 4 -> (3, 2)
                 (4, 0, 0, 7, 1),       # pair 3 alone: x 0 - 2 -> 0, y 9 - 2 = 7
                 (6, 0, 0, 0, 0),       # empty
                 (0, 4, 0, 0, 0), (4, 4, 0, 0, 0),
                 (6, 4, 4, 8, 1),       # pair 6: x 7 - 2 = 5 -> 4 (= 8 - 4), y 11 - 2 = 9 -> 8 (= 12 - 4)
                 (0, 6, 0, 0, 0), (4, 6, 0, 0, 0),
                 (6, 6, 1, 3, 2)]       # pairs 4, 5: lower medians x 3, y 5 -> (1, 3)


def test_coarse_to_fine_single_crop_is_frm():
    """factor 1 and one crop covering the whole map: the fine stage is plain FRM on the maps."""
    A = synth.random_map(24, 20, 8, synth.F16, 95).astype(np.float64)
    B = synth.random_map(24, 20, 8, synth.F16, 96).astype(np.float64)
    r = oracle.coarse_to_fine(A, B, factor=1, coarse_stride=3, coarse_iter=10, crop_h=24, crop_w=20,
                              fine_stride=2, fine_iter=10)
    f = oracle.frm(A, B, oracle.seed_grid(24, 20, 2), 10)
    if r["crops"][0][4] > 0:
        assert r["crops"] == [(0, 0, 0, 0, r["crops"][0][4])]
        assert np.array_equal(r["i"], f["i"]) and np.array_equal(r["j"], f["j"])


@pytest.mark.parametrize("dx,dy", [(6, -4), (-4, 10)])
def test_coarse_to_fine_pure_shift(dx, dy):
    """sigma = 0: every fine seed whose counterpart (x - dx, y - dy) lies inside its image-2 crop ends
    on that counterpart, and the first crop holding a pixel reports it. (Even shifts: every other
    pixel of an i.i.d. map keeps its counterpart after subsampling by 2.)"""
    H, W, ch, cw, S = 96, 80, 48, 40, 4
    p = synth.make_pair(H, W, 24, synth.F16, 97, sigma=0.0, shift=(dx, dy))
    A = oracle.decode(p.D1, p.dtype); B = oracle.decode(p.D2, p.dtype)
    r = oracle.coarse_to_fine(A, B, factor=2, coarse_stride=4, coarse_iter=10, crop_h=ch, crop_w=cw,
                              fine_stride=S, fine_iter=10)
    got = dict(zip(r["i"].tolist(), r["j"].tolist()))
    seen, n_checked = set(), 0
    for (x01, y01, x02, y02, n) in r["crops"]:
        if n == 0:
            continue
        for q in oracle.seed_grid(ch, cw, S).tolist():
            x, y = q % cw + x01, q // cw + y01
            I = y * W + x
            if I in seen:
                continue
            seen.add(I)
            cx, cy = x - dx, y - dy
            if x02 <= cx < x02 + cw and y02 <= cy < y02 + ch:
                assert got.get(I) == cy * W + cx, (I, got.get(I))
                n_checked += 1
    assert n_checked > 300
    assert np.all(np.diff(r["i"]) > 0)


def test_merge_first_wins_hand_example():
    i, j, s = oracle.merge_first_wins([(np.array([7, 3]), np.array([70, 30]), np.array([0.7, 0.3])),
                                       (np.array([3, 9, 7]), np.array([31, 90, 71]), np.array([.31, .9, .71])),
                                       (np.array([1]), np.array([10]), np.array([0.1]))])
    assert i.tolist() == [1, 3, 7, 9] and j.tolist() == [10, 30, 70, 90]
    assert s.tolist() == [0.1, 0.3, 0.7, 0.9]


def test_coarse_to_fine_pairs_reciprocal_within_crop():
    """Overlapping crops (68 x 52 tiled by 32 x 24): every reported pair is reciprocal inside the
    first crop (raster order) that holds its image-1 pixel."""
    p = synth.make_pair(68, 52, 16, synth.F16, 98, sigma=0.15, shift=(6, 4))
    A = oracle.decode(p.D1, p.dtype); B = oracle.decode(p.D2, p.dtype)
    r = oracle.coarse_to_fine(A, B, factor=2, coarse_stride=2, coarse_iter=10, crop_h=32, crop_w=24,
                              fine_stride=2, fine_iter=10)
    W = 52
    recip = set()           # full-resolution pairs reciprocal inside some crop pair (numpy NN)
    for b, (x01, y01, x02, y02, n) in enumerate(r["crops"]):
        if n == 0:
            continue
        ca = A[y01:y01 + 32, x01:x01 + 24].reshape(-1, 16); cb = B[y02:y02 + 32, x02:x02 + 24].reshape(-1, 16)
        n12 = _np_nn(ca, cb)[0]; n21 = _np_nn(cb, ca)[0]
        for i in range(ca.shape[0]):
            j = n12[i]
            if n21[j] == i:
                recip.add(((i // 24 + y01) * W + i % 24 + x01, (j // 24 + y02) * W + j % 24 + x02))
    assert len(r["i"]) > 100 and np.all(np.diff(r["i"]) > 0)
    for I, J in zip(r["i"].tolist(), r["j"].tolist()):
        assert (I, J) in recip


# --------------------------------------------------------------------- mutual
@pytest.mark.parametrize("s1,s2,d,seed", [((10, 12), (10, 12), 24, 51), ((7, 9), (11, 5), 3, 52),
                                          ((16, 16), (16, 16), 2, 53)])
def test_mutual_matches_numpy(s1, s2, d, seed):
    A = synth.random_map(*s1, d, synth.F16, seed).astype(np.float64)
    B = synth.random_map(*s2, d, synth.F16, seed + 7).astype(np.float64)
    m = oracle.mutual(A, B)
    S = _scores(A, B)
    r12, c21 = S.argmax(1), S.argmax(0)
    exp = [(i, int(r12[i])) for i in range(S.shape[0]) if c21[r12[i]] == i]
    assert list(zip(m["i"].tolist(), m["j"].tolist())) == exp
    np.testing.assert_allclose(m["s"], [S[i, j] for i, j in exp], atol=1e-12, rtol=0)
    srt = np.sort(S, 1)
    np.testing.assert_allclose(m["m12"], srt[:, -1] - srt[:, -2], atol=1e-12)
    srt = np.sort(S, 0)
    np.testing.assert_allclose(m["m21"], srt[-1] - srt[-2], atol=1e-12)


def test_mutual_symmetry():
    A = synth.random_map(14, 11, 5, synth.F16, 61).astype(np.float64)
    B = synth.random_map(9, 13, 5, synth.F16, 62).astype(np.float64)
    m12 = oracle.mutual(A, B); m21 = oracle.mutual(B, A)
    fwd = set(zip(m12["i"].tolist(), m12["j"].tolist()))
    bwd = set((i, j) for j, i in zip(m21["i"].tolist(), m21["j"].tolist()))
    assert fwd == bwd and len(fwd) > 0
