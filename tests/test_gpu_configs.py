"""GPU parity at the five full-size workloads, in the launch configuration the
benchmark times (rules in tests/parity.py).

  tiny_frm_64x48x24_f32           full oracle
  frm_512x384x24_f16              full oracle (all 3072 seeds), query counts too
  mutual_512x384x24_f16           full oracle: both NN tables over every pixel, reciprocal set
  batched_frm_16x512x384x24_f16   batch == 16 single calls; full oracle on every seed of every pair
  hard_frm_512x512x64_bf16        full oracle (all 16384 seeds), query counts too
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


def _frm_run(ddm, p, S, it):
    i, j, s, st = ddm.frm_match(dev(p.D1, p.dtype), dev(p.D2, p.dtype), S, it, return_state=True)
    return (i.cpu().numpy(), j.cpu().numpy(), s.cpu().numpy(), st["state"].cpu().numpy(),
            st["query_counts"].cpu().numpy())


def test_tiny_frm_full(ddm):
    (p,) = synth.make_config("tiny_frm_64x48x24_f32")
    i, j, s, st, qc = _frm_run(ddm, p, 8, 10)
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    seeds = oracle.seed_grid(64, 48, 8)
    assert len(seeds) == 48
    amb, n = check_frm(A, B, st, i, j, s, seeds, 10, query_counts=qc)
    assert len(i) > 30


def test_frm_512x384_full(ddm):
    (p,) = synth.make_config("frm_512x384x24_f16")
    i, j, s, st, qc = _frm_run(ddm, p, 8, 10)
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    seeds = oracle.seed_grid(512, 384, 8)
    assert len(seeds) == 3072
    amb, n = check_frm(A, B, st, i, j, s, seeds, 10, query_counts=qc)
    print(f"pairs={len(i)} ambiguous seeds={amb} query counts={qc.tolist()}")
    assert len(i) > 2500


def test_mutual_512x384_full(ddm):
    """The whole exhaustive mutual-NN workload against the oracle: both NN tables over all
    196,608 pixels of each image (the image-2 -> image-1 table through ddm_nn), and the
    reciprocal set under R2 with every GPU pair checked."""
    (p,) = synth.make_config("mutual_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    gi, gj, gs, nn12, s12 = ddm.mutual_nn(D1, D2, return_nn=True)
    nn21, s21 = ddm.nn(D2.reshape(-1, 24), D1.reshape(-1, 24))
    gi, gj, gs, nn12, s12, nn21, s21 = (t.cpu().numpy() for t in (gi, gj, gs, nn12, s12, nn21, s21))
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    N = 512 * 384
    assert len(nn12) == N and len(nn21) == N
    ref = oracle.mutual(A, B)
    amb12 = check_nn(A, B, None, nn12, s12, ref=(ref["nn12"], ref["s12"], ref["m12"]))
    amb21 = check_nn(B, A, None, nn21, s21, ref=(ref["nn21"], ref["s21"], ref["m21"]))
    assert np.array_equal(nn12[gi], gj) and np.array_equal(s12[gi], gs)
    n_gpu, n_ref = check_mutual(A, B, gi, gj, gs, ref=ref)
    extra = len(set(zip(gi.tolist(), gj.tolist())) - set(zip(ref["i"].tolist(), ref["j"].tolist())))
    print(f"mutual 512x384: gpu pairs {n_gpu} oracle pairs {n_ref} gpu-only (near-reciprocal) {extra} "
          f"ambiguous rows {amb12} ambiguous columns {amb21}")
    assert n_gpu > 1000


def test_batched_frm_16_pairs_full(ddm):
    """All 16 pairs of the batched workload: the batch equals 16 single calls, and every seed of
    every pair (16 x 3072) is checked against the oracle under R3."""
    import torch
    pairs = synth.make_config("batched_frm_16x512x384x24_f16")
    D1 = torch.stack([dev(p.D1, p.dtype) for p in pairs]); D2 = torch.stack([dev(p.D2, p.dtype) for p in pairs])
    out = ddm.frm_match_batched(D1, D2, 8, 10, return_state=True)
    seeds = oracle.seed_grid(512, 384, 8)
    amb_all = []
    for b, p in enumerate(pairs):
        i, j, s, st, qc = _frm_run(ddm, p, 8, 10)
        bi, bj, bs, bst = out[b]
        assert np.array_equal(i, bi.cpu().numpy()) and np.array_equal(j, bj.cpu().numpy())
        assert np.array_equal(s, bs.cpu().numpy()) and np.array_equal(st, bst["state"].cpu().numpy())
        assert np.array_equal(qc, bst["query_counts"].cpu().numpy())
        A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
        amb, n = check_frm(A, B, st, i, j, s, seeds, 10, query_counts=qc)
        assert n == 3072
        amb_all.append(amb)
    print(f"batched 16 x 512x384: ambiguous seeds per pair {amb_all}")


def test_hard_frm_512x512x64_bf16_full(ddm):
    """The hard workload (rotation, noise 0.3, occlusion, 20 iterations): all 16,384 seeds against
    the oracle under R3, including the per-iteration query counts when no seed is ambiguous."""
    (p,) = synth.make_config("hard_frm_512x512x64_bf16")
    i, j, s, st, qc = _frm_run(ddm, p, 4, 20)
    A, B = oracle.decode(p.D1, p.dtype), oracle.decode(p.D2, p.dtype)
    seeds = oracle.seed_grid(512, 512, 4)
    assert len(seeds) == 16384
    amb, n = check_frm(A, B, st, i, j, s, seeds, 20, query_counts=qc)
    assert n == 16384 and qc[0] == 16384 and qc[1] == 16384
    print(f"hard 512x512x64: pairs={len(i)} ambiguous seeds={amb} query counts={qc.tolist()}")


def test_determinism_full_size(ddm):
    """20 FRM calls and 10 mutual calls on the full-size pairs give bit-identical outputs
    (the maxima are order-independent; survivor lists may be ordered differently from call
    to call, which no output depends on)."""
    import torch
    (p,) = synth.make_config("frm_512x384x24_f16")
    a = _frm_run(ddm, p, 8, 10); b = _frm_run(ddm, p, 8, 10)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    buf = ddm.FrmBuffers(1, 512, 384, 512, 384, 24, torch.float16, 8, 10, D1.device)
    ref = None
    for rep in range(20):
        ddm.frm_match_into(D1, D2, 8, 10, buf)
        got = _frm_outputs(buf)
        if ref is None:
            ref = got
        else:
            _assert_same(got, ref, f"FRM repeat {rep}")
    (q,) = synth.make_config("mutual_512x384x24_f16")
    D1, D2 = dev(q.D1, q.dtype), dev(q.D2, q.dtype)
    r1 = ddm.mutual_nn(D1, D2)
    for rep in range(9):
        r2 = ddm.mutual_nn(D1, D2)
        for x, y in zip(r1, r2):
            assert torch.equal(x, y), f"mutual repeat {rep + 1}"


def _frm_outputs(buf):
    n = buf.count.cpu().numpy()
    cap = buf.cap
    outs = []
    for b, nb in enumerate(n.tolist()):
        assert nb >= 0
        o = b * cap
        outs.append((buf.out_i[o:o + nb].cpu().numpy(), buf.out_j[o:o + nb].cpu().numpy(),
                     buf.out_s[o:o + nb].cpu().numpy()))
    st = buf.state.cpu().numpy() if buf.state is not None else None
    return n, outs, st, buf.qcounts.cpu().numpy()


def _assert_same(a, b, what):
    na, oa, sa, qa = a
    nb, ob, sb, qb = b
    assert np.array_equal(na, nb), what
    for x, y in zip(oa, ob):
        for u, v in zip(x, y):
            assert np.array_equal(u, v), what
    if sa is not None:
        k = len(sa) // 4
        assert np.array_equal(sa.reshape(-1, 4)[:, :3], sb.reshape(-1, 4)[:, :3]), what
    assert np.array_equal(qa, qb), what


def test_frm_graph_replays_match_direct_launches(ddm):
    """Per-half-step FRM calls with unchanged arguments replay a cached HIP graph;
    every replay, with unrelated work and host synchronisation in between, must
    equal a call made with direct launches (sweep timing on forces those)."""
    import torch
    (p,) = synth.make_config("frm_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    buf = ddm.FrmBuffers(1, 512, 384, 512, 384, 24, torch.float16, 8, 10, D1.device)
    ddm.frm_set_mode(ddm.FRM_PER_HALF_STEP)
    try:
        ddm.profile_enable(2)
        ddm.frm_match_into(D1, D2, 8, 10, buf)
        torch.cuda.synchronize()
        ddm.profile_read()
        ddm.profile_enable(0)
        ref = _frm_outputs(buf)
        for rep in range(4):
            for t in (buf.out_i, buf.out_j, buf.state, buf.qcounts):
                t.fill_(-7)
            buf.out_s.fill_(float("nan")); buf.count.zero_()
            x = torch.randn(1 << 20, device=D1.device).sum()      # unrelated work between replays
            ddm.frm_match_into(D1, D2, 8, 10, buf)
            torch.cuda.synchronize()
            _assert_same(_frm_outputs(buf), ref, f"replay {rep}")
            del x
    finally:
        ddm.profile_enable(0)
        ddm.frm_set_mode(ddm.FRM_DEFAULT)


FRM_MODE_CASES = [
    # (config, stride, max_iter, batched)
    ("tiny_frm_64x48x24_f32", 8, 10, False),
    ("tiny_frm_64x48x24_f32", 3, 1, False),
    ("frm_512x384x24_f16", 8, 10, False),
    ("frm_512x384x24_f16", 8, 2, False),
    ("frm_512x384x24_f16", 1000, 10, False),          # no seeds
    ("batched_frm_16x512x384x24_f16", 8, 10, True),
    ("hard_frm_512x512x64_bf16", 4, 20, False),
]


def _set_exec(ddm, mode, tail_after=-1):
    ddm.frm_set_mode(mode)
    ddm.frm_set_tail_after(tail_after)


# (mode, iterations before the tail kernel, sweep timing on = direct launches)
MODE_RUNS = ((0, 2, True), (0, 2, False), (0, 2, False), (1, 2, False), (1, 2, False), (1, 2, True),
             (2, 2, False), (2, 2, False), (2, 2, True), (2, 0, False), (2, 1, False), (2, 3, False),
             (2, -1, False), (2, -1, True))


@pytest.mark.parametrize("name,S,it,batched", FRM_MODE_CASES)
def test_frm_modes_agree(ddm, name, S, it, batched):
    """Per-half-step launches, the loop kernel and the tail kernel (taking over
    after 0 to 3 iterations) give the same bits: pairs, scores, per-seed states
    and query counts; repeated calls on one workspace agree too (the barrier and
    ticket counters restart every call), and so do direct launches (sweep timing
    on) and graph replays."""
    import torch
    pairs = synth.make_config(name)
    D1 = torch.stack([dev(p.D1, p.dtype) for p in pairs]); D2 = torch.stack([dev(p.D2, p.dtype) for p in pairs])
    if not batched:
        D1, D2 = D1[0], D2[0]
    p0 = pairs[0]
    buf = ddm.FrmBuffers(len(pairs), p0.H1, p0.W1, p0.H2, p0.W2, p0.d, D1.dtype, S, it, D1.device)
    runs = []
    try:
        for mode, after, timed in MODE_RUNS:
            _set_exec(ddm, mode, after)
            ddm.profile_enable(2 if timed else 0)
            buf.count.fill_(-3); buf.qcounts.fill_(-3); buf.state.fill_(-3)
            ddm.frm_match_into(D1, D2, S, it, buf, batched=batched)
            torch.cuda.synchronize()
            ddm.profile_read()
            runs.append(((mode, after, timed), _frm_outputs(buf)))
    finally:
        ddm.profile_enable(0)
        _set_exec(ddm, ddm.FRM_DEFAULT)
    ref = runs[0][1]
    for what, r in runs[1:]:
        _assert_same(r, ref, f"{name} {what}")
    print(f"{name} S={S} it={it}: counts={ref[0].tolist()[:4]} queries={ref[3].reshape(len(pairs), -1)[0][:8].tolist()}")


GRID_CAP_CASES = [
    # (pairs, stride, max_iter, batched, caps)
    (lambda: synth.make_config("tiny_frm_64x48x24_f32"), 8, 10, False, (1, 2)),
    (lambda: [synth.make_pair(128, 96, 24, synth.F16, 71, sigma=0.2, shift=(5, -3))], 4, 10, False, (1, 3, 7)),
    (lambda: [synth.make_pair(96, 80, 64, synth.BF16, 72 + b, sigma=0.3, shift=(b, -b)) for b in range(4)],
     4, 10, True, (1, 5)),
    (lambda: synth.make_config("frm_512x384x24_f16"), 8, 10, False, (1,)),
]


@pytest.mark.parametrize("case", range(len(GRID_CAP_CASES)))
def test_frm_grid_cap_does_not_change_results(ddm, case):
    """The FRM phase kernels spread their tasks over the grid they get; with the grid capped at
    1, a few or many workgroups, in every execution mode (the tail kernel taking over after 0 or
    2 iterations), every output is bit-identical (no dependence on how tasks spread over
    concurrent workgroups)."""
    import torch
    make, S, it, batched, caps = GRID_CAP_CASES[case]
    pairs = make()
    D1 = torch.stack([dev(p.D1, p.dtype) for p in pairs]); D2 = torch.stack([dev(p.D2, p.dtype) for p in pairs])
    if not batched:
        D1, D2 = D1[0], D2[0]
    p0 = pairs[0]
    buf = ddm.FrmBuffers(len(pairs), p0.H1, p0.W1, p0.H2, p0.W2, p0.d, D1.dtype, S, it, D1.device)
    ref = None
    try:
        for mode, after in ((ddm.FRM_PER_HALF_STEP, 2), (ddm.FRM_LOOP, 2), (ddm.FRM_TAIL, 0), (ddm.FRM_TAIL, 2)):
            _set_exec(ddm, mode, after)
            for cap in (0,) + tuple(caps):
                ddm.debug_set_grid_cap(cap)
                buf.count.fill_(-3); buf.qcounts.fill_(-3); buf.state.fill_(-3)
                ddm.frm_match_into(D1, D2, S, it, buf, batched=batched)
                got = _frm_outputs(buf)
                if ref is None:
                    ref = got
                else:
                    _assert_same(got, ref, f"mode {mode} after {after} cap {cap}")
    finally:
        ddm.debug_set_grid_cap(0)
        _set_exec(ddm, ddm.FRM_DEFAULT)


OUTPUT_PATH_CASES = [
    ("tiny_frm_64x48x24_f32", 8, 10, False),
    ("frm_512x384x24_f16", 8, 10, False),
    ("frm_512x384x24_f16", 1000, 10, False),          # no seeds
    ("batched_frm_16x512x384x24_f16", 8, 10, True),
    ("hard_frm_512x512x64_bf16", 4, 20, False),
]


@pytest.mark.parametrize("name,S,it,batched", OUTPUT_PATH_CASES)
def test_frm_output_paths_agree(ddm, name, S, it, batched):
    """The one-workgroup bitmap output and the collection kernel + multi-workgroup compaction give
    the same bits: pairs, scores, per-seed states, query counts (in the default mode)."""
    import torch
    pairs = synth.make_config(name)
    D1 = torch.stack([dev(p.D1, p.dtype) for p in pairs]); D2 = torch.stack([dev(p.D2, p.dtype) for p in pairs])
    if not batched:
        D1, D2 = D1[0], D2[0]
    p0 = pairs[0]
    buf = ddm.FrmBuffers(len(pairs), p0.H1, p0.W1, p0.H2, p0.W2, p0.d, D1.dtype, S, it, D1.device)
    runs = []
    try:
        for limit in (-1, 0, -1):
            ddm.debug_set_output_bitmap_limit(limit)
            buf.count.fill_(-3); buf.qcounts.fill_(-3); buf.state.fill_(-3)
            buf.out_i.fill_(-5); buf.out_j.fill_(-5)
            ddm.frm_match_into(D1, D2, S, it, buf, batched=batched)
            torch.cuda.synchronize()
            runs.append(_frm_outputs(buf))
    finally:
        ddm.debug_set_output_bitmap_limit(-1)
    for r in runs[1:]:
        _assert_same(r, runs[0], f"{name} output paths")


def test_frm_output_paths_agree_with_routine_options(ddm):
    """Explicit starts (with repeats and out-of-map entries), pixel_tol and the basin map through
    both output paths."""
    import torch
    (p,) = synth.make_config("frm_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    rng = np.random.default_rng(9)
    starts = torch.tensor(np.concatenate([rng.integers(0, p.H1 * p.W1, 3000), [5, 5, -1, p.H1 * p.W1]]),
                          dtype=torch.int32, device="cuda")
    runs = []
    try:
        for limit in (-1, 0):
            ddm.debug_set_output_bitmap_limit(limit)
            runs.append(ddm.frm_match_ex(D1, D2, starts=starts, max_iter=4, pixel_tol=1.5, ret_basin=True,
                                         return_state=True))
    finally:
        ddm.debug_set_output_bitmap_limit(-1)
    a, b = runs
    assert a[0].numel() > 100
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)
    assert torch.equal(a[-1]["state"], b[-1]["state"]) and torch.equal(a[-1]["query_counts"], b[-1]["query_counts"])


OUTPUT_LIMIT_CASES = [
    # (H1, W1, stride or None, explicit starts) around the one-workgroup output's limits
    (1024, 512, 16, None),          # 2^19 image-1 pixels: the largest bitmap (128 KB of LDS), 2048 seeds
    (1025, 512, 16, None),          # one row more: the multi-workgroup path
    (512, 512, 8, None),            # exactly 4096 grid seeds
    (384, 256, None, 4096),         # 4096 explicit starts (with repeats)
    (384, 256, None, 4097),         # 4097: the multi-workgroup path
]


@pytest.mark.parametrize("H,W,S,nstarts", OUTPUT_LIMIT_CASES)
def test_frm_output_paths_at_their_limits(ddm, H, W, S, nstarts):
    """Both output paths, bit for bit, at and just past the pixel and seed limits of the
    one-workgroup bitmap output."""
    import torch
    p = synth.make_pair(H, W, 24, synth.F16, 97, sigma=0.1, shift=(6, -5))
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    runs = []
    try:
        for limit in (-1, 0):
            ddm.debug_set_output_bitmap_limit(limit)
            if nstarts is None:
                runs.append(ddm.frm_match(D1, D2, S, 10, return_state=True))
            else:
                starts = torch.tensor(np.random.default_rng(nstarts).integers(0, H * W, nstarts), dtype=torch.int32,
                                      device="cuda")
                runs.append(ddm.frm_match_ex(D1, D2, starts=starts, max_iter=5, pixel_tol=1.5, return_state=True))
    finally:
        ddm.debug_set_output_bitmap_limit(-1)
    a, b = runs
    assert a[0].numel() > 500
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert torch.equal(a[-1]["state"], b[-1]["state"]) and torch.equal(a[-1]["query_counts"], b[-1]["query_counts"])
