"""Calls on a caller-created stream and inside the caller's own graph capture.

Every entry point enqueues on the caller's stream: a cached graph replay
normally, direct launches while that stream is being captured (so the calls
become nodes of the caller's graph; none of them is a memset). Results must
equal a plain call on the default stream, stay ordered with the caller's work
on the same stream, and every replay of the caller's graph, with eager work
and synchronisation between replays, must reproduce them.
"""
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def maps():
    from synth.torchio import to_device
    p = synth.make_pair(128, 96, 24, synth.F16, 61, sigma=0.1, shift=(5, -3))
    return to_device(p.D1, p.dtype, "cuda"), to_device(p.D2, p.dtype, "cuda")


def _frm(ddm, D1, D2):
    import torch
    buf = ddm.FrmBuffers(1, 128, 96, 128, 96, 24, torch.float16, 4, 10, D1.device)
    return buf


def _frm_out(buf):
    n = int(buf.count[0].item())
    return (buf.out_i[:n].clone(), buf.out_j[:n].clone(), buf.out_s[:n].clone(), buf.state.clone(),
            buf.qcounts.clone())


def _mut_out(buf):
    n = int(buf.count[0].item())
    return buf.out_i[:n].clone(), buf.out_j[:n].clone(), buf.out_s[:n].clone()


def _same(a, b):
    import torch
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _scribble(fb, mb):
    for t in (fb.out_i, fb.out_j, fb.state, fb.qcounts, fb.count, mb.out_i, mb.out_j, mb.count):
        t.fill_(-7)
    fb.out_s.fill_(float("nan")); mb.out_s.fill_(float("nan"))


def test_side_stream(ddm, maps):
    import torch
    D1, D2 = maps
    fb = _frm(ddm, D1, D2)
    mb = ddm.MutualBuffers(128, 96, 128, 96, 24, torch.float16, D1.device)
    ddm.frm_match_into(D1, D2, 4, 10, fb)
    ddm.mutual_nn_into(D1, D2, mb)
    torch.cuda.synchronize()
    ref_f, ref_m = _frm_out(fb), _mut_out(mb)
    assert ref_f[0].numel() > 100 and ref_m[0].numel() > 100
    s = torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(s):
            _scribble(fb, mb)                        # caller work on the same stream, before the calls
            ddm.frm_match_into(D1, D2, 4, 10, fb)
            ddm.mutual_nn_into(D1, D2, mb)
            got_f, got_m = _frm_out(fb), _mut_out(mb)
        s.synchronize()
        _same(got_f, ref_f)
        _same(got_m, ref_m)


def test_inside_caller_graph_capture(ddm, maps):
    import torch
    D1, D2 = maps
    fb = _frm(ddm, D1, D2)
    mb = ddm.MutualBuffers(128, 96, 128, 96, 24, torch.float16, D1.device)
    ddm.frm_match_into(D1, D2, 4, 10, fb)
    ddm.mutual_nn_into(D1, D2, mb)
    torch.cuda.synchronize()
    ref_f, ref_m = _frm_out(fb), _mut_out(mb)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ddm.frm_match_into(D1, D2, 4, 10, fb)
        ddm.mutual_nn_into(D1, D2, mb)
    for rep in range(4):
        _scribble(fb, mb)
        x = torch.randn(1 << 18, device=D1.device).sum()     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_frm_out(fb), ref_f)
        _same(_mut_out(mb), ref_m)
        del x


def test_concurrent_calls_on_two_streams(ddm):
    """Two FRM calls (each with its own buffers) and a mutual call enqueued on two streams at once,
    several times over: the ticket-ordered tail kernels of concurrent calls compete for the CUs and
    must still finish with the results of lone calls (their waits only depend on workgroups of
    their own launch that already run)."""
    import torch
    p = synth.make_pair(512, 384, 24, synth.F16, 83, sigma=0.15, shift=(9, -4))
    q = synth.make_pair(256, 192, 24, synth.F16, 84, sigma=0.2, shift=(-5, 6))
    from synth.torchio import to_device
    A1, A2 = to_device(p.D1, p.dtype, "cuda"), to_device(p.D2, p.dtype, "cuda")
    B1, B2 = to_device(q.D1, q.dtype, "cuda"), to_device(q.D2, q.dtype, "cuda")
    fa = ddm.FrmBuffers(1, 512, 384, 512, 384, 24, torch.float16, 8, 10, A1.device)
    fb = ddm.FrmBuffers(1, 256, 192, 256, 192, 24, torch.float16, 4, 10, B1.device)
    mb = ddm.MutualBuffers(256, 192, 256, 192, 24, torch.float16, B1.device)
    ddm.frm_match_into(A1, A2, 8, 10, fa)
    ddm.frm_match_into(B1, B2, 4, 10, fb)
    ddm.mutual_nn_into(B1, B2, mb)
    torch.cuda.synchronize()
    ref_a, ref_b, ref_m = _frm_out(fa), _frm_out(fb), _mut_out(mb)
    assert ref_a[0].numel() > 1000 and ref_b[0].numel() > 1000
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        _scribble(fa, mb)
        _scribble(fb, mb)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            ddm.frm_match_into(A1, A2, 8, 10, fa)
        with torch.cuda.stream(s2):
            ddm.frm_match_into(B1, B2, 4, 10, fb)
            ddm.mutual_nn_into(B1, B2, mb)
        with torch.cuda.stream(s1):
            ddm.frm_match_into(A1, A2, 8, 10, fa)       # a second call on s1 overlapping s2's mutual
        torch.cuda.synchronize()
        _same(_frm_out(fa), ref_a)
        _same(_frm_out(fb), ref_b)
        _same(_mut_out(mb), ref_m)
