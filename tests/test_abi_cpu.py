"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ddm.h declares, and rejects bad arguments before
enqueueing anything (so fake device pointers are never touched)."""
import ctypes as C
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddm.h")


@pytest.fixture(scope="module")
def L():
    import dense_descriptor_matching_amd as ddm
    if not os.path.exists(ddm.LIB_PATH):
        pytest.fail("libddm.so not built: run __graft_entry__.build()")
    return ddm.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddm_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(L):
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), f"{n} declared in ddm.h but not exported"


def test_frm_mode_switch(L):
    assert L.ddm_frm_get_mode() == 2                 # first iterations per half-step, then the tail kernel
    assert L.ddm_frm_set_mode(1) == 0 and L.ddm_frm_get_mode() == 1
    assert L.ddm_frm_set_mode(0) == 0 and L.ddm_frm_get_mode() == 0
    assert L.ddm_frm_set_mode(3) == -1 and L.ddm_frm_set_mode(-1) == -1
    assert L.ddm_frm_get_mode() == 0                 # a rejected value changes nothing
    assert L.ddm_frm_set_mode(2) == 0 and L.ddm_frm_get_mode() == 2


def test_tail_after_setter(L):
    assert L.ddm_frm_set_tail_after(-2) == -1
    assert L.ddm_frm_set_tail_after(65) == -1        # beyond DDM_MAX_ITER
    for n in (0, 64, 2, -1):                         # -1: automatic (the default)
        assert L.ddm_frm_set_tail_after(n) == 0


def test_grid_cap_setter(L):
    assert L.ddm_debug_set_grid_cap(-1) == -1
    assert L.ddm_debug_set_grid_cap(4) == 0
    assert L.ddm_debug_set_grid_cap(0) == 0


def test_output_bitmap_limit_setter(L):
    assert L.ddm_debug_set_output_bitmap_limit(-2) == -1
    for n in (0, 1000, 1 << 30, -1):                 # above the maximum it is clamped; -1 = default
        assert L.ddm_debug_set_output_bitmap_limit(n) == 0


def test_barrier_polls_setter(L):
    assert L.ddm_frm_set_barrier_polls(-1) == -1
    assert L.ddm_frm_set_barrier_polls(3) == 0
    assert L.ddm_frm_set_barrier_polls(0) == 0      # back to the default bound


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert L.ddm_status_str(code)
    assert L.ddm_status_str(99) == b"unknown status"


def test_seed_count_closed_forms(L):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "seed_grid.json")))
    for c in g["cases"]:
        assert L.ddm_seed_count(c["H"], c["W"], c["S"]) == c["k"]
    assert L.ddm_seed_count(10, 10, 0) == -1


def test_workspace_sizes(L):
    assert L.ddm_frm_workspace_bytes(1, 512, 384, 512, 384, 24, 1, 8, 10) > 0
    assert L.ddm_frm_workspace_bytes(16, 512, 384, 512, 384, 24, 1, 8, 10) > \
        L.ddm_frm_workspace_bytes(1, 512, 384, 512, 384, 24, 1, 8, 10)
    assert L.ddm_mutual_workspace_bytes(512, 384, 512, 384, 24, 1) > 0
    assert L.ddm_nn_workspace_bytes(100, 100, 1000, 24, 1) > 0
    # invalid requests report 0
    assert L.ddm_frm_workspace_bytes(1, 512, 384, 512, 384, 0, 1, 8, 10) == 0
    assert L.ddm_frm_workspace_bytes(1, 512, 384, 512, 384, 24, 9, 8, 10) == 0
    assert L.ddm_frm_workspace_bytes(1, 512, 384, 512, 384, 24, 1, 8, 0) == 0
    assert L.ddm_mutual_workspace_bytes(0, 384, 512, 384, 24, 1) == 0
    assert L.ddm_nn_workspace_bytes(1, 1, 1, 129, 1) == 0
    # the per-map pixel limit (2^27, H*W*16 < 2^31): at the limit sizes are reported, above it 0
    assert L.ddm_frm_workspace_bytes(1, 1 << 13, 1 << 14, 64, 48, 24, 1, 1024, 1) > 0
    assert L.ddm_frm_workspace_bytes(1, 1 << 14, 1 << 14, 64, 48, 24, 1, 1024, 1) == 0
    assert L.ddm_mutual_workspace_bytes(1 << 14, 1 << 14, 4, 4, 24, 1) == 0


FAKE = 1 << 40        # 16-byte aligned, never dereferenced: every case fails validation first


def _frm(L, **kw):
    a = dict(D1=FAKE, H1=64, W1=48, D2=FAKE, H2=64, W2=48, d=24, dtype=1, S=8, it=10, oi=FAKE, oj=FAKE, os=FAKE,
             cap=48, cnt=FAKE, st=None, qc=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.ddm_frm_match(a["D1"], a["H1"], a["W1"], a["D2"], a["H2"], a["W2"], a["d"], a["dtype"], a["S"], a["it"],
                           a["oi"], a["oj"], a["os"], a["cap"], a["cnt"], a["st"], a["qc"], a["ws"], a["wsb"], None)


def test_frm_rejects_bad_arguments(L):
    assert _frm(L, D1=None) == -1
    assert _frm(L, D2=None) == -1
    assert _frm(L, oi=None) == -1
    assert _frm(L, cnt=None) == -1
    assert _frm(L, H1=0) == -1
    assert _frm(L, W2=-3) == -1
    assert _frm(L, S=0) == -1
    assert _frm(L, it=0) == -1
    assert _frm(L, it=65) == -1
    assert _frm(L, d=0) == -4
    assert _frm(L, d=129) == -4
    assert _frm(L, dtype=3) == -4
    assert _frm(L, cap=47) == -2
    assert _frm(L, ws=None) == -3
    assert _frm(L, wsb=16) == -3
    assert _frm(L, H1=1 << 14, W1=1 << 14) == -1          # 2^28 pixels: above the per-map limit
    assert _frm(L, H2=1 << 13, W2=(1 << 14) + 1) == -1    # just above 2^27
    assert _frm(L, D1=FAKE + 2) == -1          # fp16 map not 16-byte aligned
    assert _frm(L, D2=FAKE + 2, dtype=0) == -1          # fp32 map not 4-byte aligned


def _frm_ex(L, **kw):
    a = dict(D1=FAKE, H1=64, W1=48, D2=FAKE, H2=64, W2=48, d=24, dtype=1, metric=0, S=8, starts=FAKE, n=100,
             it=1, tol=0.0, basin=None, oi=FAKE, oj=FAKE, os=FAKE, cap=100, cnt=FAKE, st=None, qc=None, ws=FAKE,
             wsb=1 << 40)
    a.update(kw)
    return L.ddm_frm_match_ex(a["D1"], a["H1"], a["W1"], a["D2"], a["H2"], a["W2"], a["d"], a["dtype"], a["metric"],
                              a["S"],
                              a["starts"], a["n"], a["it"], a["tol"], a["basin"], a["oi"], a["oj"], a["os"],
                              a["cap"], a["cnt"], a["st"], a["qc"], a["ws"], a["wsb"], None)


def test_frm_ex_rejects_bad_arguments(L):
    import math
    assert _frm_ex(L, starts=None, n=5) == -1              # a count without a list
    assert _frm_ex(L, n=-1) == -1
    assert _frm_ex(L, tol=-0.5) == -1
    assert _frm_ex(L, tol=math.nan) == -1
    assert _frm_ex(L, tol=math.inf) == -1
    assert _frm_ex(L, starts=None, n=0, tol=1.0) == -1     # pixel_tol needs explicit starts
    assert _frm_ex(L, cap=99) == -2                        # capacity below the number of starts
    assert _frm_ex(L, starts=None, n=0, cap=47) == -2      # grid: 48 seeds
    assert _frm_ex(L, it=0) == -1
    assert _frm_ex(L, wsb=16) == -3
    assert _frm_ex(L, D1=FAKE + 2) == -1
    # workspace: explicit starts need room for their marks and states; invalid requests report 0
    g = L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 24, 1, 0, 8, -1, 10)
    assert g == L.ddm_frm_workspace_bytes(1, 64, 48, 64, 48, 24, 1, 8, 10) > 0
    assert L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 24, 1, 0, 8, 5000, 1) > g
    assert L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 24, 1, 0, 0, -1, 10) == 0
    assert L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 24, 1, 0, 0, 10, 1) > 0     # stride unused with starts


def test_metric_validation(L):
    # the Euclidean metric takes fp32 maps with d + 2 <= 128; unknown metrics are unsupported
    assert L.ddm_nn_ex_workspace_bytes(100, 100, 1000, 3, 0, 1) > 0
    assert L.ddm_nn_ex_workspace_bytes(100, 100, 1000, 3, 1, 1) == 0
    assert L.ddm_nn_ex_workspace_bytes(100, 100, 1000, 127, 0, 1) == 0
    assert L.ddm_nn_ex_workspace_bytes(100, 100, 1000, 3, 0, 2) == 0
    assert L.ddm_nn_ex_workspace_bytes(100, 100, 1000, 24, 1, 0) == L.ddm_nn_workspace_bytes(100, 100, 1000, 24, 1)
    assert L.ddm_mutual_ex_workspace_bytes(64, 48, 64, 48, 3, 0, 1) > 0
    assert L.ddm_mutual_ex_workspace_bytes(64, 48, 64, 48, 3, 2, 1) == 0
    assert L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 3, 0, 1, 8, -1, 10) > 0
    assert L.ddm_frm_ex_workspace_bytes(64, 48, 64, 48, 3, 1, 1, 8, -1, 10) == 0
    assert _frm_ex(L, metric=1) == -4                     # fp16 maps under the Euclidean metric
    assert _frm_ex(L, metric=7) == -4
    r = L.ddm_nn_ex(FAKE, 100, None, 100, FAKE, 1000, 3, 1, 1, FAKE, FAKE, FAKE, 1 << 40, None)
    assert r == -4
    r = L.ddm_mutual_nn_ex(FAKE, 64, 48, FAKE, 64, 48, 3, 0, 3, FAKE, FAKE, FAKE, 3072, FAKE, None, None, FAKE,
                           1 << 40, None)
    assert r == -4


def test_c2f_rejects_bad_arguments(L):
    def c(**kw):
        a = dict(F1=FAKE, H1=1024, W1=768, F2=FAKE, H2=1024, W2=768, d=24, dtype=1, f=2, cs=8, ci=10, ch=512, cw=384,
                 fs=8, fi=10, oi=FAKE, oj=FAKE, os=FAKE, cap=1 << 20, cnt=FAKE, info=None, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return L.ddm_c2f_match(a["F1"], a["H1"], a["W1"], a["F2"], a["H2"], a["W2"], a["d"], a["dtype"], a["f"],
                               a["cs"], a["ci"], a["ch"], a["cw"], a["fs"], a["fi"], a["oi"], a["oj"], a["os"],
                               a["cap"], a["cnt"], a["info"], a["ws"], a["wsb"], None)
    assert c(f=0) == -1
    assert c(ch=1025) == -1 and c(cw=0) == -1 and c(H2=500) == -1
    assert c(cs=0) == -1 and c(fi=0) == -1
    assert c(d=23) == -4                                   # rows must be whole 32-bit words
    assert c(W2=20000, H2=600) == -4                       # median histograms would not fit in LDS
    assert c(cap=100) == -2                                # 4 tiles x 3072 fine seeds
    assert c(wsb=16) == -3
    assert c(F1=FAKE + 2) == -1
    assert L.ddm_c2f_workspace_bytes(1024, 768, 1024, 768, 24, 1, 2, 8, 10, 512, 384, 8, 10) > 0
    assert L.ddm_c2f_workspace_bytes(1024, 768, 1024, 768, 24, 1, 2, 8, 10, 1024, 384, 8, 10) > 0
    assert L.ddm_c2f_workspace_bytes(1024, 768, 1024, 768, 24, 1, 2, 8, 10, 1025, 384, 8, 10) == 0


def test_frm_batched_rejects_bad_batch(L):
    r = L.ddm_frm_match_batched(0, FAKE, 64, 48, FAKE, 64, 48, 24, 1, 8, 10, FAKE, FAKE, FAKE, 48, FAKE, None,
                                None, FAKE, 1 << 40, None)
    assert r == -1


def test_mutual_rejects_bad_arguments(L):
    def m(**kw):
        a = dict(D1=FAKE, D2=FAKE, d=24, dtype=1, cap=3072, ws=FAKE, wsb=1 << 40, nn=None, s=None)
        a.update(kw)
        return L.ddm_mutual_nn(a["D1"], 64, 48, a["D2"], 64, 48, a["d"], a["dtype"], FAKE, FAKE, FAKE, a["cap"],
                               FAKE, a["nn"], a["s"], a["ws"], a["wsb"], None)
    assert m(D1=None) == -1
    assert m(cap=3071) == -2
    assert m(wsb=0) == -3
    assert m(dtype=5) == -4
    assert m(nn=FAKE) == -1              # nn12 without s12


def test_nn_rejects_bad_arguments(L):
    def n(**kw):
        a = dict(Q=FAKE, NQ=10, rows=None, M=10, R=FAKE, N=100, d=24, dtype=1, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return L.ddm_nn(a["Q"], a["NQ"], a["rows"], a["M"], a["R"], a["N"], a["d"], a["dtype"], FAKE, FAKE,
                        a["ws"], a["wsb"], None)
    assert n(M=0) == -1
    assert n(N=0) == -1
    assert n(NQ=5) == -1                 # identity queries need NQ >= M
    assert n(R=None) == -1
    assert n(wsb=8) == -3
    assert n(d=200) == -4


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import dense_descriptor_matching_amd as ddm
    x = torch.zeros(4, 4, 24, dtype=torch.float16)
    with pytest.raises(TypeError):
        ddm.frm_match(x, x)
    with pytest.raises(TypeError):
        ddm.mutual_nn(x, x)


def test_c_abi_demo_is_built_and_links():
    """The plain host program of the GPU ABI test exists and resolves libddm.so (no args:
    it prints its usage before touching the GPU)."""
    import os
    import subprocess
    demo = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_demo")
    assert os.path.exists(demo), "build with __graft_entry__.build()"
    r = subprocess.run([demo], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def test_frm_stats_from_query_counts():
    """ddm_stats from the per-iteration query counts (host-only; no device involved)."""
    import dense_descriptor_matching_amd as ddm
    qc = [3072, 3072, 700, 650, 40, 30, 0, 0, 0, 0,
          5, 5, 0, 0, 0, 0, 0, 0, 0, 0]
    st = ddm.frm_stats(qc, 5, 196608, 1000)
    assert st[0]["iters"] == 3 and st[1]["iters"] == 1
    assert st[0]["active"] == qc[:10] and st[1]["active"] == qc[10:]
    assert st[0]["dot_products"] == (3072 + 700 + 40) * 1000 + (3072 + 650 + 30) * 196608
    assert st[1]["dot_products"] == 5 * 1000 + 5 * 196608
    L = ddm.lib()
    import ctypes as C
    bad = (C.c_int32 * 2)(1, -1)
    out = ddm.FrmStats()
    assert L.ddm_frm_stats(C.cast(bad, C.c_void_p), 1, 1, 10, 10, C.byref(out)) == -1
    assert L.ddm_frm_stats(C.cast(bad, C.c_void_p), 1, 65, 10, 10, C.byref(out)) == -1
    assert L.ddm_frm_stats(None, 1, 1, 10, 10, C.byref(out)) == -1


def test_mutual_workspace_is_linear_in_the_pixel_counts(L):
    """The mutual pass keeps one merged key per row and per column: its workspace grows with N1 + N2,
    not with N1 x N2 / chunk (28 bytes per pixel of a square pair, plus block counts and alignment)."""
    for H, W in ((512, 384), (1024, 768), (2048, 1536)):
        n = H * W
        b = L.ddm_mutual_workspace_bytes(H, W, H, W, 24, 1)
        assert 28 * n <= b <= 28 * n + n // 16 + 4096, (H, W, b)
