"""The C ABI driven from plain host code (tests/c_abi_demo.cpp, built with the library):
hipMalloc'd buffers, workspace sizes from the queries, the default stream. Its FRM and
mutual-NN outputs must equal the binding's (the same library) and satisfy the parity rules
against the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from parity import check_mutual, exact_scores, near_reciprocal, TAU

pytestmark = pytest.mark.gpu
DEMO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_demo")


def _read_pairs(buf, off):
    status, count = np.frombuffer(buf, np.int32, 2, off)
    off += 8
    n = max(int(count), 0)
    i = np.frombuffer(buf, np.int32, n, off); off += 4 * n
    j = np.frombuffer(buf, np.int32, n, off); off += 4 * n
    s = np.frombuffer(buf, np.float32, n, off); off += 4 * n
    return int(status), int(count), i, j, s, off


@pytest.mark.parametrize("dt", [synth.F16, synth.BF16, synth.F32])
def test_c_program_through_the_abi(tmp_path, dt):
    assert os.path.exists(DEMO), "tests/c_abi_demo is missing: build with __graft_entry__.build()"
    p = synth.make_pair(48, 40, 24, dt, 81, sigma=0.1, shift=(3, -2))
    hdr = np.array([48, 40, 48, 40, 24, dt, 4, 10], np.int32)
    src = tmp_path / "in.bin"; dst = tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(hdr.tobytes()); f.write(np.ascontiguousarray(p.D1).tobytes()); f.write(np.ascontiguousarray(p.D2).tobytes())
    r = subprocess.run([DEMO, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    buf = dst.read_bytes()
    fs, fc, fi, fj, fsc, off = _read_pairs(buf, 0)
    ms, mc, mi, mj, msc, off = _read_pairs(buf, off)
    assert fs == 0 and ms == 0 and fc > 0 and mc > 0 and off == len(buf)
    # the same calls through the Python binding give the same bits
    import dense_descriptor_matching_amd as ddm
    from synth.torchio import to_device
    D1, D2 = to_device(p.D1, dt, "cuda"), to_device(p.D2, dt, "cuda")
    bi, bj, bs = (t.cpu().numpy() for t in ddm.frm_match(D1, D2, 4, 10))
    assert np.array_equal(bi, fi) and np.array_equal(bj, fj) and np.array_equal(bs, fsc)
    ci, cj, cs = (t.cpu().numpy() for t in ddm.mutual_nn(D1, D2))
    assert np.array_equal(ci, mi) and np.array_equal(cj, mj) and np.array_equal(cs, msc)
    # and the parity rules against the oracle
    A, B = oracle.decode(p.D1, dt), oracle.decode(p.D2, dt)
    check_mutual(A, B, mi, mj, msc)
    assert np.all(np.diff(fi) > 0)
    for a, b in zip(fi.tolist(), fj.tolist()):
        assert near_reciprocal(A, B, a, b)
    np.testing.assert_allclose(fsc, exact_scores(A, B, fi, fj), atol=TAU, rtol=0)
