"""CPU oracle for dense descriptor matching (fp64, plain loops, OpenMP over queries).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library and
its binding never do, and the two share no code.

The arithmetic lives in ``oracle.c`` (built into ``liboracle.so`` next to it);
this module only marshals numpy arrays. What each function computes, and the
passages of the pages it follows, is documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, F16, BF16 = 0, 1, 2
METRICS = {"dot": 0, "l2": 1}     # score = dot product, or minus the squared Euclidean distance


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (IEEE double semantics: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = C.CDLL(path)
    P = C.c_void_p
    i64, i32, dbl = C.c_int64, C.c_int, C.c_double
    lib.orc_decode.argtypes = [P, i32, i64, P]
    lib.orc_decode.restype = i32
    lib.orc_nn.argtypes = [P, P, i64, P, i64, i32, P, P, P]
    lib.orc_nn.restype = None
    lib.orc_seed_grid.argtypes = [i32, i32, i32, P]
    lib.orc_seed_grid.restype = i64
    lib.orc_frm.argtypes = [P, i64, P, i64, i32, P, i64, i32, dbl, P, P, P, P, P, P, P, P]
    lib.orc_frm.restype = i32
    lib.orc_frm_ex.argtypes = [P, i64, P, i64, i32, i32, P, i64, i32, dbl, i32, P, P, P, P, P, P, P, P, P, P]
    lib.orc_nn_m.argtypes = [P, P, i64, P, i64, i32, i32, P, P, P]
    lib.orc_nn_m.restype = None
    lib.orc_mutual_m.argtypes = [P, i64, P, i64, i32, i32, P, P, P, P, P, P, P, P, P]
    lib.orc_mutual_m.restype = i64
    lib.orc_frm_ex.restype = i32
    lib.orc_frm_select.argtypes = [P, P, P, i64, i32, dbl, i32, P, P]
    lib.orc_frm_select.restype = None
    lib.orc_merge.argtypes = [P, P, P, P, i64, P, P, P]
    lib.orc_merge.restype = i64
    lib.orc_mutual.argtypes = [P, i64, P, i64, i32, P, P, P, P, P, P, P, P, P]
    lib.orc_mutual.restype = i64
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


class use_library:
    """Context manager: route every oracle call through another build of oracle.c
    (the mutation tests use it to check that the pins catch planted mistakes)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def decode(stored: np.ndarray, dtype: int) -> np.ndarray:
    """Stored float32 / float16 / bfloat16-bits array -> float64 array of the same shape."""
    lib = _load()
    src = np.ascontiguousarray(stored)
    want = {F32: np.float32, F16: np.float16, BF16: np.uint16}[dtype]
    if src.dtype != want:
        raise TypeError(f"stored dtype {src.dtype} does not match code {dtype}")
    out = np.empty(src.shape, dtype=np.float64)
    if lib.orc_decode(_p(src), dtype, src.size, _p(out)) != 0:
        raise ValueError("bad dtype")
    return out


def _rows(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-1])


def nn(Q: np.ndarray, R: np.ndarray, qrows=None, metric: str = "dot"):
    """Brute-force NN of rows of Q (or of Q[qrows]) over all rows of R.

    metric "dot": score = dot product; "l2": score = minus the squared Euclidean
    distance (the NN is the nearest point). Returns (idx int32, s1 float64, margin float64)."""
    lib = _load()
    Q, R = _rows(Q), _rows(R)
    d = Q.shape[1]
    if qrows is not None:
        qrows = np.ascontiguousarray(qrows, dtype=np.int32)
        nq = qrows.size
    else:
        nq = Q.shape[0]
    idx = np.empty(nq, np.int32)
    s1 = np.empty(nq, np.float64)
    s2 = np.empty(nq, np.float64)
    lib.orc_nn_m(_p(Q), _p(qrows) if qrows is not None else None, nq, _p(R), R.shape[0], d, METRICS[metric],
                 _p(idx), _p(s1), _p(s2))
    return idx, s1, s1 - s2


def seed_grid(H: int, W: int, S: int) -> np.ndarray:
    lib = _load()
    k = lib.orc_seed_grid(H, W, S, None)
    out = np.empty(max(k, 0), np.int32)
    lib.orc_seed_grid(H, W, S, _p(out) if k > 0 else None)
    return out


def frm(D1: np.ndarray, D2: np.ndarray, seeds: np.ndarray, max_iter: int, tau: float = 1e-4):
    """FRM from the given image-1 seeds. D1, D2: float64 [N, d] or [H, W, d].

    Returns a dict: per-seed u, v, score, conv_iter, active, ambiguous; the merged
    unique pairs i, j, s (ascending i); niter; n_fwd / n_bwd = queries per iteration."""
    lib = _load()
    A, B = _rows(D1), _rows(D2)
    seeds = np.ascontiguousarray(seeds, dtype=np.int32)
    k = seeds.size
    u = np.empty(k, np.int32); v = np.empty(k, np.int32)
    score = np.empty(k, np.float64); conv = np.empty(k, np.int32)
    active = np.empty(k, np.uint8); amb = np.empty(k, np.uint8)
    nf = np.zeros(max(max_iter, 1), np.int64); nb = np.zeros(max(max_iter, 1), np.int64)
    niter = lib.orc_frm(_p(A), A.shape[0], _p(B), B.shape[0], A.shape[1], _p(seeds), k, max_iter, tau,
                        _p(u), _p(v), _p(score), _p(conv), _p(active), _p(amb), _p(nf), _p(nb))
    if niter < 0:
        raise MemoryError
    oi = np.empty(k, np.int32); oj = np.empty(k, np.int32); os_ = np.empty(k, np.float64)
    n = lib.orc_merge(_p(u), _p(v), _p(score), _p(active), k, _p(oi), _p(oj), _p(os_))
    return dict(u=u, v=v, score=score, conv_iter=conv, active=active.astype(bool),
                ambiguous=amb.astype(bool), i=oi[:n].copy(), j=oj[:n].copy(), s=os_[:n].copy(),
                niter=int(niter), n_fwd=nf[:max_iter], n_bwd=nb[:max_iter])


def frm_ex(D1: np.ndarray, D2: np.ndarray, H1: int, W1: int, *, grid_stride: int | None = None,
           starts: np.ndarray | None = None, max_iter: int = 10, pixel_tol: float = 0.0, ret_basin: bool = False,
           tau: float = 1e-4, metric: str = "dot"):
    """The FRM routine with its options ("DUSt3R和MASt3R论文阅读", section MASt3R matching, the quoted
    fast_reciprocal_NNs routine):

    - seeds: the stride grid (``grid_stride``) or the given image-1 pixels (``starts``, linear
      p = x + W1*y), made unique and ascending;
    - ``pixel_tol == 0``: a seed is kept when it is no longer active at exit; its pair is (u, v);
    - ``pixel_tol > 0`` (given starts only; the routine has no grid form of it): a seed is kept when
      the Euclidean pixel distance between u_old, as the loop leaves it, and u is below pixel_tol; the
      reported image-1 pixel is u_old (the start itself in a one-iteration call);
    - ``ret_basin``: the forward test is off and basin[p] (N1 entries, -1 elsewhere) records, for each
      backward query, where a seed that stood at p moved to;
    - ``metric``: "dot" (descriptors) or "l2" (3D points: nearest by Euclidean distance; scores are
      then minus squared distances).

    Returns a dict with the per-seed state (seeds, u, v, u_old, score, conv_iter, active, ambiguous),
    the unique pairs i, j, s ascending in (i, j), basin (or None), niter, n_fwd, n_bwd."""
    lib = _load()
    A, B = _rows(D1), _rows(D2)
    N1 = A.shape[0]
    if N1 != H1 * W1:
        raise ValueError("D1 does not hold H1 x W1 rows")
    if (grid_stride is None) == (starts is None):
        raise ValueError("give exactly one of grid_stride and starts")
    if pixel_tol > 0 and starts is None:
        raise ValueError("pixel_tol > 0 needs explicit starts")
    if starts is not None:
        st = np.asarray(starts, dtype=np.int64).ravel()
        if st.size and (st.min() < 0 or st.max() >= N1):
            raise ValueError("start outside image 1")
        seeds = np.unique(st).astype(np.int32)
    else:
        seeds = seed_grid(H1, W1, grid_stride)
    k = seeds.size
    u = np.empty(k, np.int32); v = np.empty(k, np.int32); u_old = np.empty(k, np.int32)
    score = np.empty(k, np.float64); conv = np.empty(k, np.int32)
    active = np.empty(k, np.uint8); amb = np.empty(k, np.uint8)
    nf = np.zeros(max(max_iter, 1), np.int64); nb = np.zeros(max(max_iter, 1), np.int64)
    basin = np.full(N1, -1, np.int32) if ret_basin else None
    niter = lib.orc_frm_ex(_p(A), N1, _p(B), B.shape[0], A.shape[1], METRICS[metric], _p(seeds), k, max_iter, tau,
                           0 if ret_basin else 1, _p(basin) if ret_basin else None, _p(u_old),
                           _p(u), _p(v), _p(score), _p(conv), _p(active), _p(amb), _p(nf), _p(nb))
    if niter < 0:
        raise MemoryError
    act = active.astype(bool)
    keep = np.empty(k, np.uint8); rep_i = np.empty(k, np.int32)
    lib.orc_frm_select(_p(u), _p(u_old), _p(active), k, W1, float(pixel_tol), 1 if starts is not None else 0,
                       _p(keep), _p(rep_i))
    keep = keep.astype(bool)
    pi, pj, ps = rep_i[keep], v[keep], score[keep]
    order = np.lexsort((pj, pi))
    pi, pj, ps = pi[order], pj[order], ps[order]
    first = np.ones(pi.size, bool)
    first[1:] = (pi[1:] != pi[:-1]) | (pj[1:] != pj[:-1])
    return dict(seeds=seeds, u=u, v=v, u_old=u_old, score=score, conv_iter=conv, active=act,
                ambiguous=amb.astype(bool), i=pi[first].copy(), j=pj[first].copy(), s=ps[first].copy(),
                basin=basin, niter=int(niter), n_fwd=nf[:max_iter], n_bwd=nb[:max_iter])


def mutual(D1: np.ndarray, D2: np.ndarray, metric: str = "dot"):
    """Exhaustive mutual NN. Returns dict with pairs i, j, s and both NN tables with margins
    (metric as in :func:`nn`)."""
    lib = _load()
    A, B = _rows(D1), _rows(D2)
    N1, N2, d = A.shape[0], B.shape[0], A.shape[1]
    nn12 = np.empty(N1, np.int32); s12 = np.empty(N1); m12 = np.empty(N1)
    nn21 = np.empty(N2, np.int32); s21 = np.empty(N2); m21 = np.empty(N2)
    oi = np.empty(min(N1, N2), np.int32); oj = np.empty(min(N1, N2), np.int32); os_ = np.empty(min(N1, N2))
    n = lib.orc_mutual_m(_p(A), N1, _p(B), N2, d, METRICS[metric], _p(nn12), _p(s12), _p(m12),
                         _p(nn21), _p(s21), _p(m21), _p(oi), _p(oj), _p(os_))
    if n < 0:
        raise MemoryError
    return dict(i=oi[:n].copy(), j=oj[:n].copy(), s=os_[:n].copy(), nn12=nn12, s12=s12, m12=m12,
                nn21=nn21, s21=s21, m21=m21)


# ---------------------------------------------------------------------------
# Coarse-to-fine matching of maps larger than the network's 512 px: the "MASt3R"
# note on cv-learn.com (section 手法とアーキテクチャ, 粗密マッチング paragraph) says
# high-resolution images are matched coarsely first, the coarse correspondences
# guide the matching of enumerated local crops, and the fine matches are mapped
# back to the original resolution. The steps below are this package's reading
# of that paragraph (the page gives no further rule):
#   coarse maps   every factor-th row and column of each map (starting at 0), a
#                 stand-in for the network run on the downscaled image;
#   coarse pairs  FRM on the coarse maps (grid seeds), positions scaled back by factor;
#   image-1 crops the tiling of image 1 by crop_h x crop_w windows, the last window
#                 of a row / column moved back to end at the border;
#   image-2 crops for each image-1 crop holding coarse pairs, the window of the same
#                 size centred on the lower medians of their image-2 x and y (window
#                 offset = median - size // 2, clamped into image 2);
#   fine pairs    FRM on every crop pair (grid seeds), mapped to full-resolution
#                 indices; a pixel claimed by several crops keeps the first crop's
#                 pair (crops in raster order); pairs ascending in i.
# ---------------------------------------------------------------------------
def crop_windows(H1, W1, H2, W2, crop_h, crop_w, x1, y1, x2, y2):
    """Crop enumeration from full-resolution coarse pair positions (x1, y1) -> (x2, y2).
    Returns a list of (x0_1, y0_1, x0_2, y0_2, n) in raster order of the image-1 tiling."""
    x1, y1, x2, y2 = (np.asarray(a, np.int64) for a in (x1, y1, x2, y2))
    out = []
    for ty in range(-(-H1 // crop_h)):
        for tx in range(-(-W1 // crop_w)):
            y0 = min(ty * crop_h, H1 - crop_h)
            x0 = min(tx * crop_w, W1 - crop_w)
            inside = (y1 >= y0) & (y1 < y0 + crop_h) & (x1 >= x0) & (x1 < x0 + crop_w)
            n = int(inside.sum())
            if n:
                mx = int(np.sort(x2[inside])[(n - 1) // 2])
                my = int(np.sort(y2[inside])[(n - 1) // 2])
                x02 = min(max(mx - crop_w // 2, 0), W2 - crop_w)
                y02 = min(max(my - crop_h // 2, 0), H2 - crop_h)
            else:
                x02 = y02 = 0
            out.append((x0, y0, x02, y02, n))
    return out


def coarse_to_fine(F1, F2, *, factor, coarse_stride, coarse_iter, crop_h, crop_w, fine_stride, fine_iter,
                   tau: float = 1e-4):
    """Coarse-to-fine FRM (reading above). F1, F2: float64 [H, W, d].
    Returns dict(i, j, s, crops, coarse=(ci, cj), fine=[per-crop frm results or None])."""
    F1 = np.asarray(F1, np.float64); F2 = np.asarray(F2, np.float64)
    H1, W1, d = F1.shape
    H2, W2, _ = F2.shape
    if not (1 <= crop_h <= min(H1, H2) and 1 <= crop_w <= min(W1, W2)) or factor < 1:
        raise ValueError("bad crop size or factor")
    C1 = np.ascontiguousarray(F1[::factor, ::factor]); C2 = np.ascontiguousarray(F2[::factor, ::factor])
    Hc1, Wc1 = C1.shape[:2]; Wc2 = C2.shape[1]
    cr = frm(C1, C2, seed_grid(Hc1, Wc1, coarse_stride), coarse_iter, tau)
    ci, cj = cr["i"], cr["j"]
    x1 = (ci % Wc1) * factor; y1 = (ci // Wc1) * factor
    x2 = (cj % Wc2) * factor; y2 = (cj // Wc2) * factor
    crops = crop_windows(H1, W1, H2, W2, crop_h, crop_w, x1, y1, x2, y2)
    fine, per_crop = [], []
    seeds = seed_grid(crop_h, crop_w, fine_stride)
    for b, (x01, y01, x02, y02, n) in enumerate(crops):
        if n == 0:
            fine.append(None)
            continue
        A = np.ascontiguousarray(F1[y01:y01 + crop_h, x01:x01 + crop_w])
        B = np.ascontiguousarray(F2[y02:y02 + crop_h, x02:x02 + crop_w])
        r = frm(A, B, seeds, fine_iter, tau)
        fine.append(r)
        I = (r["i"] // crop_w + y01) * W1 + (r["i"] % crop_w + x01)
        J = (r["j"] // crop_w + y02) * W2 + (r["j"] % crop_w + x02)
        per_crop.append((I, J, r["s"]))
    i, j, s = merge_first_wins(per_crop)
    return dict(i=i, j=j, s=s, crops=crops, coarse=(ci, cj), fine=fine)


def merge_first_wins(per_crop):
    """Merge per-crop full-resolution pairs [(I, J, s), ...] given in crop order: a pixel I
    reported by several crops keeps the first crop's pair. Returns (i, j, s) ascending in i."""
    owner = {}
    for I, J, S in per_crop:
        for a, b, c in zip(np.asarray(I).tolist(), np.asarray(J).tolist(), np.asarray(S).tolist()):
            if a not in owner:
                owner[a] = (b, c)
    keys = sorted(owner)
    return (np.array(keys, np.int32), np.array([owner[k][0] for k in keys], np.int32),
            np.array([owner[k][1] for k in keys], np.float64))
