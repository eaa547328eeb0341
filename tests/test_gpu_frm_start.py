"""The two ways an FRM call starts give the same bits.

With grid seeds, nothing image-1-sized to clear and a first half-step launched
on its own, the first sweep derives the seed pixels and its update writes the
seeds' initial state; every other execution (loop mode, the tail kernel from
half-step 0, the multi-workgroup output path) starts with the init kernel.
Cases: image 2 narrower and shorter than image 1 (the grid follows image 1's
width), seed counts that are not a multiple of the 16-query update block,
max_iter 1 and 4, one to three batched pairs, fp16, bf16 and fp32 maps. All four per-seed state
columns (u, v, conv_iter, u_old), pairs, scores and query counts must agree,
and the implicit start must match the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_frm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


# (mode, half-steps before the tail kernel, output limit): the first two start without
# the init kernel, the others with it
STARTS = (("per-half-step", 0, -1, None), ("tail default", 2, -1, None), ("tail after 1", 2, 1, None),
          ("loop", 1, -1, None), ("tail from 0", 2, 0, None), ("dense output", 2, -1, 0))


def _maps(B, seed, dtype):
    """B pairs of a 100 x 90 image 1 and a 96 x 70 image 2 cut from a noisy shifted copy."""
    D1, D2 = [], []
    for b in range(B):
        p = synth.make_pair(100, 90, 24, dtype, seed + b, sigma=0.15, shift=(3, -2))
        D1.append(p.D1)
        D2.append(np.ascontiguousarray(p.D2[2:98, 5:75]))
    return D1, D2, p.dtype


def _outputs(buf, B, k):
    n = buf.count.cpu().numpy().copy()
    outs = []
    for b in range(B):
        o, nb = b * buf.cap, int(n[b])
        assert nb >= 0
        outs.append(tuple(t[o:o + nb].cpu().numpy().copy() for t in (buf.out_i, buf.out_j, buf.out_s)))
    return n, outs, buf.state.cpu().numpy().reshape(B, -1, 4)[:, :k].copy(), buf.qcounts.cpu().numpy().copy()


@pytest.mark.parametrize("B,S,it,dtype", [(1, 7, 1, "f16"), (1, 7, 4, "f16"), (3, 7, 4, "f16"), (3, 11, 1, "f16"),
                                          (1, 7, 4, "bf16"), (2, 7, 4, "f32")])
def test_frm_implicit_start_equals_init_start(ddm, B, S, it, dtype):
    import torch
    from synth.torchio import to_device
    sdt, tdt = {"f16": (synth.F16, torch.float16), "bf16": (synth.BF16, torch.bfloat16),
                "f32": (synth.F32, torch.float32)}[dtype]
    D1n, D2n, dt = _maps(B, 500 + 10 * S + it, sdt)
    D1 = torch.stack([to_device(a, dt, "cuda") for a in D1n])
    D2 = torch.stack([to_device(a, dt, "cuda") for a in D2n])
    if B == 1:
        D1, D2 = D1[0], D2[0]
    seeds = oracle.seed_grid(100, 90, S)
    k = len(seeds)
    assert k % 16 != 0
    buf = ddm.FrmBuffers(B, 100, 90, 96, 70, 24, tdt, S, it, D1.device)
    runs = []
    try:
        for what, mode, after, limit in STARTS:
            ddm.frm_set_mode(mode)
            ddm.frm_set_tail_after(after)
            ddm.debug_set_output_bitmap_limit(1 << 19 if limit is None else limit)
            for t in (buf.out_i, buf.out_j, buf.state, buf.qcounts, buf.count):
                t.fill_(-5)
            buf.out_s.fill_(float("nan"))
            ddm.frm_match_into(D1, D2, S, it, buf, batched=B > 1)
            torch.cuda.synchronize()
            runs.append((what, _outputs(buf, B, k)))
    finally:
        ddm.debug_set_output_bitmap_limit(1 << 19)
        ddm.frm_set_mode(ddm.FRM_DEFAULT)
        ddm.frm_set_tail_after(-1)
    ref = runs[0][1]
    for what, r in runs[1:]:
        assert np.array_equal(r[0], ref[0]), what
        for x, y in zip(r[1], ref[1]):
            for u, v in zip(x, y):
                assert np.array_equal(u, v), what
        assert np.array_equal(r[2], ref[2]), what
        assert np.array_equal(r[3], ref[3]), what
    n, outs, st, qc = ref
    qc = qc.reshape(B, -1)
    for b in range(B):
        A, Bm = oracle.decode(D1n[b], dt), oracle.decode(D2n[b], dt)
        gi, gj, gs = outs[b]
        check_frm(A, Bm, st[b][:, :3], gi, gj, gs, seeds, it, query_counts=qc[b])
    assert (qc[:, 0] == k).all()
