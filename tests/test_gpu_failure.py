"""Failure path of the FRM loop and tail modes, forced from the host.

The loop kernel's grid barriers wait a bounded number of polls. Lowering that
bound to one poll makes the waits time out on purpose: every workgroup still
ends (a timed-out wait returns, the others see the error flag or time out at
the next barrier), and the call reports failure through out_count = -1, which
the binding raises as DDMError. Coarse-to-fine passes the failure of its inner
FRM calls on. The tail kernel's waits are bounded the same way. Calls made
after restoring the default bound are unaffected.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ddm():
    import dense_descriptor_matching_amd as m
    m.lib()
    return m


def dev(a, dtype):
    from synth.torchio import to_device
    return to_device(a, dtype, "cuda")


def _run(ddm, D1, D2):
    i, j, s, st = ddm.frm_match(D1, D2, 8, 10, return_state=True)
    return [t.cpu().numpy() for t in (i, j, s, st["state"], st["query_counts"])]


def test_loop_barrier_timeout_reports_failure(ddm):
    (p,) = synth.make_config("frm_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    ddm.frm_set_mode(ddm.FRM_PER_HALF_STEP)
    ref = _run(ddm, D1, D2)
    q = synth.make_pair(256, 192, 24, synth.F16, 301, sigma=0.1, shift=(12, -8))
    F1, F2 = dev(q.D1, q.dtype), dev(q.D2, q.dtype)
    c2f_args = dict(factor=2, coarse_stride=4, coarse_iter=10, crop=(128, 96), fine_stride=4, fine_iter=10)
    c2f_ref = [t.cpu().numpy() for t in ddm.c2f_match(F1, F2, **c2f_args)]
    try:
        ddm.frm_set_mode(ddm.FRM_LOOP)
        ddm.frm_set_barrier_polls(1)
        print("frm 512x384 f16, loop mode, one poll per barrier wait", flush=True)
        with pytest.raises(ddm.DDMError):
            ddm.frm_match(D1, D2, 8, 10)
        print("c2f 256x192 f16, loop mode, one poll per barrier wait", flush=True)
        with pytest.raises(ddm.DDMError):
            ddm.c2f_match(F1, F2, **c2f_args)
    finally:
        ddm.frm_set_barrier_polls(0)
    try:
        print("frm 512x384 f16, loop mode, default bound", flush=True)
        got = _run(ddm, D1, D2)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        got = [t.cpu().numpy() for t in ddm.c2f_match(F1, F2, **c2f_args)]
        for a, b in zip(got, c2f_ref):
            assert np.array_equal(a, b)
    finally:
        ddm.frm_set_mode(ddm.FRM_DEFAULT)


def test_tail_wait_bound_ends_cleanly(ddm):
    """One poll per wait of the tail kernel (taking over at once): every workgroup still leaves
    the kernel; the call either reports the failure or, when no wait had to poll twice, returns
    the exact result. The next calls at the default bound return the same bits as before."""
    (p,) = synth.make_config("frm_512x384x24_f16")
    D1, D2 = dev(p.D1, p.dtype), dev(p.D2, p.dtype)
    ddm.frm_set_mode(ddm.FRM_PER_HALF_STEP)
    ref = _run(ddm, D1, D2)
    try:
        ddm.frm_set_mode(ddm.FRM_TAIL)
        ddm.frm_set_tail_after(0)
        ddm.frm_set_barrier_polls(1)
        print("frm 512x384 f16, tail kernel from half-step 0, one poll per wait", flush=True)
        try:
            got = _run(ddm, D1, D2)
            print("no wait ran past one poll", flush=True)
            for a, b in zip(got, ref):
                assert np.array_equal(a, b)
        except ddm.DDMError:
            print("failure reported", flush=True)
        ddm.frm_set_barrier_polls(0)
        for after in (0, 2):
            ddm.frm_set_tail_after(after)
            print(f"frm 512x384 f16, tail kernel after {after} iterations, default bound", flush=True)
            got = _run(ddm, D1, D2)
            for a, b in zip(got, ref):
                assert np.array_equal(a, b)
    finally:
        ddm.frm_set_barrier_polls(0)
        ddm.frm_set_tail_after(-1)
        ddm.frm_set_mode(ddm.FRM_DEFAULT)
