"""GPU parity of the HIP path against the CPU oracle at small sizes that still
span several tiles, groups and chunks and end in ragged tails (rules in
tests/parity.py). All calls go through the C ABI via the ctypes binding."""
import numpy as np
import pytest

import oracle
import synth
from parity import TAU, check_frm, check_mutual, check_nn, exact_scores

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def dev(a, dtype):
    from synth.torchio import to_device
    return to_device(a, dtype, "cuda")


def dec(a, dtype):
    return oracle.decode(a, dtype)


# ------------------------------------------------------------------ NN unit
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16, synth.F32])
@pytest.mark.parametrize("M,N,d", [(1, 1, 24), (5, 300, 24), (37, 1000, 8), (513, 4099, 24), (700, 9000, 64),
                                   (64, 2000, 3), (130, 5000, 100), (40, 3000, 128), (17, 777, 32),
                                   # query tiles per wave 3 (and 6 then 2 over two sub-blocks): every tile-count
                                   # variant of the sweep loop, at K blocks 1, 2 and 4
                                   (300, 2500, 24), (1000, 3000, 64), (333, 1500, 128)])
def test_nn_matches_oracle(ddm, dtype, M, N, d):
    Q = synth.gaussian_rows(M, d, dtype, 1000 + M)
    R = synth.gaussian_rows(N, d, dtype, 2000 + N)
    idx, s = ddm.nn(dev(Q, dtype), dev(R, dtype))
    check_nn(dec(Q, dtype), dec(R, dtype), None, idx.cpu().numpy(), s.cpu().numpy())


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_nn_ties_lowest_index(ddm, dtype):
    R = synth.gaussian_rows(3000, 24, dtype, 5)
    dup_src = 2500
    dups = [3, 17, 255, 256, 1024, 1777, 2999]       # duplicates across slots, groups and chunks
    R[dups] = R[dup_src]
    Q = R[[dup_src, dup_src, 40]].copy()
    idx, s = ddm.nn(dev(Q, dtype), dev(R, dtype))
    idx = idx.cpu().numpy()
    assert idx[0] == 3 and idx[1] == 3
    ref, _, _ = oracle.nn(dec(Q, dtype), dec(R, dtype))
    assert idx[2] == ref[2]


def test_nn_gathered_rows(ddm):
    Q = synth.gaussian_rows(5000, 24, synth.F16, 6)
    R = synth.gaussian_rows(7000, 24, synth.F16, 7)
    rows = np.random.default_rng(3).integers(0, 5000, 900).astype(np.int32)
    import torch
    idx, s = ddm.nn(dev(Q, synth.F16), dev(R, synth.F16), q_rows=torch.from_numpy(rows).cuda())
    check_nn(dec(Q, synth.F16), dec(R, synth.F16), rows, idx.cpu().numpy(), s.cpu().numpy())


def test_nn_gather_rows_outside_the_map(ddm):
    """Entries of the gather list outside [0, NQ) read nothing outside Q and report -1 / NaN."""
    import torch
    Q = synth.gaussian_rows(300, 24, synth.F16, 12)
    R = synth.gaussian_rows(2000, 24, synth.F16, 13)
    rows = np.array([5, -1, 299, 300, 1 << 30, -(1 << 30), 0, 17], np.int32)
    idx, s = ddm.nn(dev(Q, synth.F16), dev(R, synth.F16), q_rows=torch.from_numpy(rows).cuda())
    idx, s = idx.cpu().numpy(), s.cpu().numpy()
    bad = (rows < 0) | (rows >= 300)
    assert (idx[bad] == -1).all() and np.isnan(s[bad]).all()
    check_nn(dec(Q, synth.F16), dec(R, synth.F16), rows[~bad], idx[~bad], s[~bad])


def test_nn_all_scores_negative(ddm):
    R = -np.abs(synth.gaussian_rows(1000, 8, synth.F32, 8)).astype(np.float32)
    Q = np.abs(synth.gaussian_rows(50, 8, synth.F32, 9)).astype(np.float32)
    idx, s = ddm.nn(dev(Q, synth.F32), dev(R, synth.F32))
    assert (s.cpu().numpy() < 0).all()
    check_nn(Q.astype(np.float64), R.astype(np.float64), None, idx.cpu().numpy(), s.cpu().numpy())


def test_nn_subnormal_f16_components(ddm):
    Q = synth.gaussian_rows(64, 24, synth.F16, 10)
    R = synth.gaussian_rows(900, 24, synth.F16, 11)
    Q[:, 5] = np.float16(3e-6)        # fp16 subnormals (< 6.1e-5) must not be flushed
    R[:, 5] = np.float16(-5e-6)
    R[100] = np.float16(0); R[100, 5] = np.float16(6e-8)
    Q[0] = np.float16(0); Q[0, 5] = np.float16(6e-8)
    idx, s = ddm.nn(dev(Q, synth.F16), dev(R, synth.F16))
    check_nn(dec(Q, synth.F16), dec(R, synth.F16), None, idx.cpu().numpy(), s.cpu().numpy())


# ------------------------------------------------------------------ FRM
FRM_CASES = [
    # (H1, W1, H2, W2, d, dtype, stride, max_iter, sigma, shift, seed)
    (64, 48, 64, 48, 24, synth.F32, 8, 10, 0.1, (3, 2), 1),
    (64, 48, 64, 48, 24, synth.F16, 4, 10, 0.3, (5, -4), 2),
    (40, 70, 40, 70, 64, synth.BF16, 3, 20, 0.4, (-6, 2), 3),
    (33, 65, 33, 65, 24, synth.F16, 2, 3, 0.5, (1, 1), 4),
    (96, 80, 96, 80, 24, synth.F16, 8, 1, 0.2, (2, 9), 5),
    (50, 50, 50, 50, 100, synth.F16, 5, 10, 0.3, (4, 4), 6),
    (20, 30, 20, 30, 3, synth.F16, 2, 10, 0.1, (1, 0), 7),
]


@pytest.mark.parametrize("case", FRM_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[4]}-{synth.DTYPE_NAMES[c[5]]}-S{c[6]}-it{c[7]}")
def test_frm_matches_oracle(ddm, case):
    H1, W1, H2, W2, d, dt, S, it, sigma, shift, seed = case
    p = synth.make_pair(H1, W1, d, dt, 500 + seed, sigma=sigma, shift=shift)
    i, j, s, st = ddm.frm_match(dev(p.D1, dt), dev(p.D2, dt), S, it, return_state=True)
    A, B = dec(p.D1, dt), dec(p.D2, dt)
    seeds = oracle.seed_grid(H1, W1, S)
    check_frm(A, B, st["state"].cpu().numpy(), i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy(), seeds, it,
              query_counts=st["query_counts"].cpu().numpy())


def test_frm_different_image_sizes(ddm):
    D1 = synth.random_map(30, 41, 24, synth.F16, 31)
    D2 = synth.random_map(57, 23, 24, synth.F16, 32)
    i, j, s, st = ddm.frm_match(dev(D1, synth.F16), dev(D2, synth.F16), 3, 10, return_state=True)
    check_frm(dec(D1, synth.F16), dec(D2, synth.F16), st["state"].cpu().numpy(), i.cpu().numpy(),
              j.cpu().numpy(), s.cpu().numpy(), oracle.seed_grid(30, 41, 3), 10)


def test_frm_grouped_tasks_with_empty_slots(ddm):
    """Sweep tasks that group several 768-row sub-blocks hand their (sub-block, query slot) units out through a
    counter: 316x352 at stride 4 gives 6952 = 9 x 768 + 40 seeds against the 64 reference chunks of a 512x384
    map, so the first sweep groups two sub-blocks per task and the last task's second sub-block (three 16-row
    tiles) leaves five of its eight slots empty."""
    D1 = synth.random_map(316, 352, 24, synth.F16, 61)
    D2 = synth.random_map(512, 384, 24, synth.F16, 62)
    i, j, s, st = ddm.frm_match(dev(D1, synth.F16), dev(D2, synth.F16), 4, 3, return_state=True)
    seeds = oracle.seed_grid(316, 352, 4)
    assert len(seeds) == 6952
    check_frm(dec(D1, synth.F16), dec(D2, synth.F16), st["state"].cpu().numpy(), i.cpu().numpy(),
              j.cpu().numpy(), s.cpu().numpy(), seeds, 3, query_counts=st["query_counts"].cpu().numpy())


def test_frm_identity(ddm):
    p = synth.make_pair(64, 48, 24, synth.F16, 41, sigma=0.0, shift=(0, 0))
    i, j, s, st = ddm.frm_match(dev(p.D1, synth.F16), dev(p.D2, synth.F16), 4, 10, return_state=True)
    seeds = oracle.seed_grid(64, 48, 4)
    assert np.array_equal(i.cpu().numpy(), seeds) and np.array_equal(j.cpu().numpy(), seeds)
    assert (st["state"][:, 2].cpu().numpy() == 1).all()


def test_frm_pure_shift(ddm):
    H, W, dx, dy = 64, 48, 5, -3
    p = synth.make_pair(H, W, 24, synth.F16, 42, sigma=0.0, shift=(dx, dy))
    i, j, s, st = ddm.frm_match(dev(p.D1, synth.F16), dev(p.D2, synth.F16), 4, 10, return_state=True)
    st = st["state"].cpu().numpy()
    seeds = oracle.seed_grid(H, W, 4)
    A = dec(p.D1, synth.F16).reshape(-1, 24)
    for a, sd in enumerate(seeds):
        x, y = sd % W, sd // W
        if 0 <= x - dx < W and 0 <= y - dy < H:
            assert tuple(st[a]) == (sd, sd - dx - dy * W, 1)


def test_frm_no_seeds(ddm):
    D = synth.random_map(3, 3, 24, synth.F16, 1)
    i, j, s = ddm.frm_match(dev(D, synth.F16), dev(D, synth.F16), 8, 10)
    assert i.numel() == 0


def test_frm_batched_equals_single_calls(ddm):
    import torch
    pairs = [synth.make_pair(48, 40, 24, synth.F16, 700 + b, sigma=0.2, shift=(b - 2, 3 - b)) for b in range(5)]
    D1 = torch.stack([dev(p.D1, synth.F16) for p in pairs]); D2 = torch.stack([dev(p.D2, synth.F16) for p in pairs])
    out = ddm.frm_match_batched(D1, D2, 4, 10, return_state=True)
    for b, p in enumerate(pairs):
        i, j, s, st = ddm.frm_match(dev(p.D1, synth.F16), dev(p.D2, synth.F16), 4, 10, return_state=True)
        bi, bj, bs, bst = out[b]
        assert torch.equal(i, bi) and torch.equal(j, bj) and torch.equal(s, bs)
        assert torch.equal(st["state"], bst["state"]) and torch.equal(st["query_counts"], bst["query_counts"])


# ------------------------------------------------------------------ mutual
MUTUAL_CASES = [
    (24, 20, 22, 18, 24, synth.F16, 1),
    (64, 48, 64, 48, 24, synth.F16, 2),
    (50, 61, 47, 70, 24, synth.BF16, 3),
    (40, 40, 40, 40, 64, synth.BF16, 4),
    (3, 5, 4, 3, 8, synth.F16, 5),
    (30, 30, 33, 31, 24, synth.F32, 6),
    (37, 29, 41, 23, 100, synth.F16, 7),
]


@pytest.mark.parametrize("case", MUTUAL_CASES, ids=lambda c: f"{c[0]}x{c[1]}-{c[2]}x{c[3]}x{c[4]}-{synth.DTYPE_NAMES[c[5]]}")
def test_mutual_matches_oracle(ddm, case):
    H1, W1, H2, W2, d, dt, seed = case
    D1 = synth.random_map(H1, W1, d, dt, 900 + seed)
    D2 = synth.random_map(H2, W2, d, dt, 950 + seed)
    i, j, s, nn12, s12 = ddm.mutual_nn(dev(D1, dt), dev(D2, dt), return_nn=True)
    A, B = dec(D1, dt), dec(D2, dt)
    check_nn(A, B, None, nn12.cpu().numpy(), s12.cpu().numpy())
    check_mutual(A, B, i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy())


# ragged sizes: query counts just past a sub-block, reference counts just past / short of an index
# group and a chunk, several K blocks, a single reference
MUTUAL_RAGGED_CASES = [
    (1, 769, 41, 25, 24, synth.F16, 11),      # 769 rows: one past a 768-row sub-block; 1025 references
    (32, 32, 32, 32, 24, synth.F16, 12),
    (17, 61, 3, 341, 16, synth.BF16, 13),     # 1037 rows, 1023 references
    (45, 47, 45, 47, 64, synth.BF16, 14),     # d = 64: two K blocks
    (20, 26, 50, 62, 48, synth.F16, 15),
    (9, 9, 1, 1, 8, synth.F16, 16),           # one reference
]


@pytest.mark.parametrize("case", MUTUAL_RAGGED_CASES,
                         ids=lambda c: f"{c[0]}x{c[1]}-{c[2]}x{c[3]}x{c[4]}-{synth.DTYPE_NAMES[c[5]]}")
def test_mutual_ragged_sizes_match_oracle(ddm, case):
    """The fused mutual pass at ragged sizes meets the oracle under R1 (row NN table) and R2."""
    H1, W1, H2, W2, d, dt, seed = case
    D1 = synth.random_map(H1, W1, d, dt, 1900 + seed)
    D2 = synth.random_map(H2, W2, d, dt, 1950 + seed)
    i, j, s, nn12, s12 = ddm.mutual_nn(dev(D1, dt), dev(D2, dt), return_nn=True)
    A, B = dec(D1, dt), dec(D2, dt)
    check_nn(A, B, None, nn12.cpu().numpy(), s12.cpu().numpy())
    check_mutual(A, B, i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy())


def test_mutual_several_sub_blocks_per_workgroup(ddm):
    """Workgroups that sweep several 768-row sub-blocks hand their (sub-block, query slot) units out through a
    counter: 6952 = 9 x 768 + 40 rows against 64 reference chunks of 3072 gives five query blocks of two
    sub-blocks each, and the last sub-block's 40 rows (three 16-row tiles) leave five of its eight slots empty."""
    H1, W1, H2, W2, d, dt = 79, 88, 512, 384, 24, synth.F16
    D1 = synth.random_map(H1, W1, d, dt, 2101)
    D2 = synth.random_map(H2, W2, d, dt, 2102)
    i, j, s, nn12, s12 = ddm.mutual_nn(dev(D1, dt), dev(D2, dt), return_nn=True)
    A, B = dec(D1, dt), dec(D2, dt)
    check_nn(A, B, None, nn12.cpu().numpy(), s12.cpu().numpy())
    check_mutual(A, B, i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy())


def test_mutual_shifted_pair_dense_matches(ddm):
    p = synth.make_pair(96, 64, 24, synth.F16, 77, sigma=0.05, shift=(3, -2))
    i, j, s = ddm.mutual_nn(dev(p.D1, synth.F16), dev(p.D2, synth.F16))
    A, B = dec(p.D1, synth.F16), dec(p.D2, synth.F16)
    n_gpu, n_ref = check_mutual(A, B, i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy())
    assert n_ref > 0.8 * 96 * 64


def test_mutual_symmetry(ddm):
    D1 = synth.random_map(40, 30, 24, synth.F16, 61)
    D2 = synth.random_map(35, 33, 24, synth.F16, 62)
    i, j, _ = ddm.mutual_nn(dev(D1, synth.F16), dev(D2, synth.F16))
    i2, j2, _ = ddm.mutual_nn(dev(D2, synth.F16), dev(D1, synth.F16))
    assert set(zip(i.tolist(), j.tolist())) == set(zip(j2.tolist(), i2.tolist()))
