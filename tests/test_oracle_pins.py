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
