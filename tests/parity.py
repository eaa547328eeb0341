"""Parity rules between the HIP path and the CPU oracle (tau = 1e-4).

R1 (NN): where the oracle's top-1/top-2 margin is >= tau the GPU index equals
the oracle index; otherwise the GPU index must score within tau of the best.
Scores always agree within tau with the exact score of the returned pair.
R2 (mutual): every oracle pair whose two margins are >= tau is found; every GPU
pair is an oracle pair or near-reciprocal (within tau of both maxima); no
image-2 pixel appears twice.
R3 (FRM): seeds whose path never met a margin below tau have identical state
(u, v, iteration of convergence); other seeds, when converged, end on a
near-reciprocal pair; the GPU output is exactly its converged seed states,
unique and ascending; every pair of a non-ambiguous oracle seed is present.
"""
import numpy as np

import oracle

TAU = 1e-4


def exact_scores(A, B, ii, jj):
    A = A.reshape(-1, A.shape[-1]); B = B.reshape(-1, B.shape[-1])
    ii = np.asarray(ii, np.int64); jj = np.asarray(jj, np.int64)
    return np.einsum("nd,nd->n", A[ii], B[jj])


def check_nn(A, B, qrows, g_idx, g_s, tau=TAU, ref=None):
    """R1 for queries A[qrows] (all rows of A when qrows is None) against all rows of B.
    ref: the oracle's (index, best score, margin) for those queries when already computed.
    Returns #ambiguous queries."""
    o_idx, s1, m = ref if ref is not None else oracle.nn(A, B, qrows=qrows)
    g_idx = np.asarray(g_idx); g_s = np.asarray(g_s, np.float64)
    assert g_idx.min() >= 0 and g_idx.max() < B.reshape(-1, B.shape[-1]).shape[0]
    sharp = m >= tau
    bad = np.nonzero(sharp & (g_idx != o_idx))[0]
    assert bad.size == 0, f"{bad.size} sharp queries differ, e.g. q={bad[:5]} gpu={g_idx[bad[:5]]} ref={o_idx[bad[:5]]}"
    rows = np.arange(len(g_idx)) if qrows is None else np.asarray(qrows)
    sg = exact_scores(A, B, rows, g_idx)
    assert np.all(sg >= s1 - tau), "an ambiguous query returned a clearly worse neighbour"
    err = np.abs(g_s - sg)
    assert err.max() <= tau, f"score error {err.max()}"
    return int((~sharp).sum())


def check_mutual(A, B, gi, gj, gs, ref=None, tau=TAU):
    """R2 on tiny inputs (full oracle)."""
    m = ref if ref is not None else oracle.mutual(A, B)
    gi = np.asarray(gi); gj = np.asarray(gj)
    assert np.all(np.diff(gi) > 0), "GPU pairs not strictly ascending in i"
    assert len(np.unique(gj)) == len(gj), "an image-2 pixel appears in two GPU pairs"
    gpu = set(zip(gi.tolist(), gj.tolist()))
    ref_set = set(zip(m["i"].tolist(), m["j"].tolist()))
    sharp = [(i, j) for i, j in ref_set if m["m12"][i] >= tau and m["m21"][j] >= tau]
    missing = [p for p in sharp if p not in gpu]
    assert not missing, f"{len(missing)} sharp reciprocal pairs missing, e.g. {missing[:5]}"
    for i, j in gpu - ref_set:
        s = exact_scores(A, B, [i], [j])[0]
        assert s >= m["s12"][i] - tau and s >= m["s21"][j] - tau, f"GPU pair {(i, j)} not near-reciprocal"
    np.testing.assert_allclose(np.asarray(gs, np.float64), exact_scores(A, B, gi, gj), atol=tau, rtol=0)
    return len(gpu), len(ref_set)


def near_reciprocal(A, B, i, j, tau=TAU):
    return bool(near_reciprocal_many(A, B, [i], [j], tau)[0])


def near_reciprocal_many(A, B, ii, jj, tau=TAU):
    """Per pair (i, j): score(i, j) within tau of row i's best score over B and of column j's
    best score over A (both from the oracle). Returns a bool array."""
    ii = np.asarray(ii, np.int32); jj = np.asarray(jj, np.int32)
    if ii.size == 0:
        return np.zeros(0, bool)
    _, s1, _ = oracle.nn(A, B, qrows=ii)
    _, s2, _ = oracle.nn(B, A, qrows=jj)
    s = exact_scores(A, B, ii, jj)
    return (s >= s1 - tau) & (s >= s2 - tau)


def check_frm(A, B, state, gi, gj, gs, seeds, max_iter, seed_sel=None, ref=None, query_counts=None, tau=TAU):
    """R3. state: GPU per-seed [k, 3] (u, v, conv_iter). seed_sel: indices of seeds to
    run through the oracle (all when None). Returns (#ambiguous, #checked)."""
    state = np.asarray(state)
    sel = np.arange(len(seeds)) if seed_sel is None else np.asarray(seed_sel)
    r = ref if ref is not None else oracle.frm(A, B, np.asarray(seeds)[sel], max_iter, tau)
    g = state[sel]
    amb = r["ambiguous"]
    ok = ~amb
    for col, key in ((0, "u"), (1, "v"), (2, "conv_iter")):
        bad = np.nonzero(ok & (g[:, col] != r[key]))[0]
        assert bad.size == 0, (f"{bad.size} non-ambiguous seeds differ in {key}: seeds {sel[bad[:5]]} "
                               f"gpu={g[bad[:5]]} ref u={r['u'][bad[:5]]} v={r['v'][bad[:5]]} "
                               f"it={r['conv_iter'][bad[:5]]}")
    conv_amb = np.nonzero(amb & (g[:, 2] >= 0))[0]
    near = near_reciprocal_many(A, B, g[conv_amb, 0], g[conv_amb, 1], tau)
    assert near.all(), f"ambiguous seeds {sel[conv_amb[~near][:5]]} end off M"
    # output = converged states, unique, ascending
    conv = state[:, 2] >= 0
    expect = sorted(set(zip(state[conv, 0].tolist(), state[conv, 1].tolist())))
    got = list(zip(np.asarray(gi).tolist(), np.asarray(gj).tolist()))
    assert got == expect, "output pairs are not the unique converged seed states"
    oracle_pairs = set(zip(r["u"][ok & ~r["active"]].tolist(), r["v"][ok & ~r["active"]].tolist()))
    assert oracle_pairs <= set(got)
    if len(gi):
        np.testing.assert_allclose(np.asarray(gs, np.float64), exact_scores(A, B, gi, gj), atol=tau, rtol=0)
    if query_counts is not None and seed_sel is None and not amb.any():
        qc = np.asarray(query_counts).reshape(-1, 2)
        assert qc[:, 0].tolist() == r["n_fwd"].tolist() and qc[:, 1].tolist() == r["n_bwd"].tolist()
    return int(amb.sum()), len(sel)
