"""MI355X-native dense descriptor matching: Fast Reciprocal Matching and mutual NN.

Thin ctypes binding over the C ABI of ``libddm.so`` (declared in
``include/ddm.h``). It only marshals arguments: torch supplies device memory and
the current HIP stream, every step of the computation runs in the library's
HIP kernels. There is no CPU fallback: if the library is missing the calls
raise.

Matching follows MASt3R: unit-norm descriptor maps D1, D2 of shape [H, W, d];
NN = arg-max of the dot product; the reciprocal set M = {(i, j) : j = NN2(i),
i = NN1(j)}; Fast Reciprocal Matching iterates NN round trips from a regular
seed grid and keeps the seeds that cycle ("MASt3R" note on cv-learn.com,
section 手法とアーキテクチャ, FRM paragraph; the fast_reciprocal_NNs routine
quoted in "DUSt3R和MASt3R论文阅读", section MASt3R matching).
Pixel indices are linear, p = x + W * y; :func:`to_xy` converts.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddm.so")

DDM_F32, DDM_F16, DDM_BF16 = 0, 1, 2
METRICS = {"dot": 0, "l2": 1}   # dot product (descriptors) / Euclidean distance (3D points, fp32)
_DT = {torch.float32: DDM_F32, torch.float16: DDM_F16, torch.bfloat16: DDM_BF16}
STATUS = {0: "ok", -1: "invalid argument", -2: "output capacity too small",
          -3: "workspace missing or too small", -4: "unsupported dtype or descriptor dimension",
          -5: "HIP error while enqueueing"}

_lib = None


class DDMError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


def _declare(lib):
    P, I, I64, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    lib.ddm_status_str.argtypes = [I]; lib.ddm_status_str.restype = C.c_char_p
    lib.ddm_seed_count.argtypes = [I, I, I]; lib.ddm_seed_count.restype = I64
    lib.ddm_nn_workspace_bytes.argtypes = [I, I, I, I, I]; lib.ddm_nn_workspace_bytes.restype = SZ
    lib.ddm_nn.argtypes = [P, I, P, I, P, I, I, I, P, P, P, SZ, P]; lib.ddm_nn.restype = I
    lib.ddm_frm_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]; lib.ddm_frm_workspace_bytes.restype = SZ
    lib.ddm_frm_match.argtypes = [P, I, I, P, I, I, I, I, I, I, P, P, P, I, P, P, P, P, SZ, P]
    lib.ddm_frm_match.restype = I
    lib.ddm_frm_match_batched.argtypes = [I, P, I, I, P, I, I, I, I, I, I, P, P, P, I, P, P, P, P, SZ, P]
    lib.ddm_frm_match_batched.restype = I
    lib.ddm_mutual_workspace_bytes.argtypes = [I, I, I, I, I, I]; lib.ddm_mutual_workspace_bytes.restype = SZ
    lib.ddm_mutual_nn.argtypes = [P, I, I, P, I, I, I, I, P, P, P, I, P, P, P, P, SZ, P]
    lib.ddm_mutual_nn.restype = I
    lib.ddm_frm_ex_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I, I]
    lib.ddm_frm_ex_workspace_bytes.restype = SZ
    lib.ddm_frm_match_ex.argtypes = [P, I, I, P, I, I, I, I, I, I, P, I, I, C.c_double, P,
                                     P, P, P, I, P, P, P, P, SZ, P]
    lib.ddm_nn_ex_workspace_bytes.argtypes = [I, I, I, I, I, I]; lib.ddm_nn_ex_workspace_bytes.restype = SZ
    lib.ddm_nn_ex.argtypes = [P, I, P, I, P, I, I, I, I, P, P, P, SZ, P]; lib.ddm_nn_ex.restype = I
    lib.ddm_mutual_ex_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.ddm_mutual_ex_workspace_bytes.restype = SZ
    lib.ddm_mutual_nn_ex.argtypes = [P, I, I, P, I, I, I, I, I, P, P, P, I, P, P, P, P, SZ, P]
    lib.ddm_mutual_nn_ex.restype = I
    lib.ddm_frm_match_ex.restype = I
    lib.ddm_c2f_workspace_bytes.argtypes = [I] * 13; lib.ddm_c2f_workspace_bytes.restype = SZ
    lib.ddm_c2f_match.argtypes = [P, I, I, P, I, I, I, I, I, I, I, I, I, I, I, P, P, P, I, P, P, P, SZ, P]
    lib.ddm_c2f_match.restype = I
    lib.ddm_frm_set_mode.argtypes = [I]; lib.ddm_frm_set_mode.restype = I
    lib.ddm_frm_get_mode.argtypes = []; lib.ddm_frm_get_mode.restype = I
    lib.ddm_frm_set_tail_after.argtypes = [I]; lib.ddm_frm_set_tail_after.restype = I
    lib.ddm_frm_set_barrier_polls.argtypes = [I]; lib.ddm_frm_set_barrier_polls.restype = I
    lib.ddm_debug_set_grid_cap.argtypes = [I]; lib.ddm_debug_set_grid_cap.restype = I
    lib.ddm_debug_set_output_bitmap_limit.argtypes = [I]; lib.ddm_debug_set_output_bitmap_limit.restype = I
    lib.ddm_profile_enable.argtypes = [I]; lib.ddm_profile_enable.restype = I
    lib.ddm_profile_read.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int64)]; lib.ddm_profile_read.restype = I
    lib.ddm_release_cached_resources.argtypes = []; lib.ddm_release_cached_resources.restype = I
    lib.ddm_frm_stats.argtypes = [P, I, I, I64, I64, P]; lib.ddm_frm_stats.restype = I
    lib.ddm_frm_match_noalloc.argtypes = [P, I, I, P, I, I, I, I, I, I, P, P, P, I, P, P, P, P]
    lib.ddm_frm_match_noalloc.restype = I
    return lib


DDM_MAX_ITER = 64


class FrmStats(C.Structure):
    """ddm_stats: iterations run, active seeds per half-step, NN dot products."""
    _fields_ = [("iters", C.c_int32), ("active", C.c_int32 * (2 * DDM_MAX_ITER)), ("dot_products", C.c_int64)]


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build() "
                               "(python -m dense_descriptor_matching_amd.build)")
        _lib = _declare(C.CDLL(LIB_PATH))
        # The library's cached HIP graphs, capture streams and events are released while the
        # HIP runtime is still up (interpreter exit runs before the runtime's own teardown).
        atexit.register(_release_at_exit)
    return _lib


def _release_at_exit():
    if _lib is not None:
        _lib.ddm_release_cached_resources()     # a failure this late has no one left to report to


def release_cached_resources():
    """Destroy the library's cached HIP graphs, capture streams and timing events (they are
    recreated on demand). Runs at interpreter exit; callable any time no call is in flight."""
    if _lib is not None:
        _rc(_lib.ddm_release_cached_resources(), "ddm_release_cached_resources")


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on(*tensors):
    """Make the tensors' device current for the call (the library launches on the current
    device and the caller's current stream there); all tensors must share that device."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t is not None and t.device != dev:
            raise ValueError(f"tensors on {dev} and {t.device}: one device per call")
    return torch.cuda.device(dev)


def _check_map(D, name):
    if not isinstance(D, torch.Tensor) or not D.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if D.dtype not in _DT:
        raise TypeError(f"{name}: unsupported dtype {D.dtype}")
    if not D.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _rc(status, what):
    if status != 0:
        raise DDMError(status, what)


def seed_count(H: int, W: int, grid_stride: int) -> int:
    return int(lib().ddm_seed_count(H, W, grid_stride))


def to_xy(idx: torch.Tensor, W: int):
    """Linear pixel index -> (x, y)."""
    return idx % W, torch.div(idx, W, rounding_mode="floor")


FRM_PER_HALF_STEP = 0      # one sweep + one update launch per half-step
FRM_LOOP = 1               # every iteration in one cooperative loop kernel
FRM_TAIL = 2               # first iterations per half-step, the rest in one ticket-ordered tail kernel
FRM_DEFAULT = FRM_TAIL


def frm_set_mode(mode: int):
    """Select how FRM calls execute (process-wide; results are identical)."""
    _rc(lib().ddm_frm_set_mode(mode), "ddm_frm_set_mode")


def frm_get_mode() -> int:
    return lib().ddm_frm_get_mode()


def frm_set_tail_after(iterations: int):
    """Iterations run per half-step before the tail kernel takes over in FRM_TAIL mode
    (-1, the default: 2 to 8 half-steps, later for larger problems)."""
    _rc(lib().ddm_frm_set_tail_after(iterations), "ddm_frm_set_tail_after")


def frm_set_barrier_polls(polls: int):
    """Polls a wait of the loop or tail kernel makes before it gives up (0: the default).
    A test aid: a tiny value makes loop-mode calls report failure instead of matches."""
    _rc(lib().ddm_frm_set_barrier_polls(polls), "ddm_frm_set_barrier_polls")


def debug_set_grid_cap(max_workgroups: int):
    """Cap the grid of the FRM phase kernels (0: no cap); outputs must not change with it.
    A test aid against dependences between concurrent workgroups."""
    _rc(lib().ddm_debug_set_grid_cap(max_workgroups), "ddm_debug_set_grid_cap")


def debug_set_output_bitmap_limit(max_pixels: int):
    """Largest image 1 (pixels) whose FRM output is collected and ordered in one workgroup per pair
    through an LDS bitmap (-1: the default 2^19; 0: always the multi-workgroup compaction).
    A test aid: both paths must give identical outputs."""
    _rc(lib().ddm_debug_set_output_bitmap_limit(max_pixels), "ddm_debug_set_output_bitmap_limit")


def profile_enable(mask: int):
    """Bracket later sweep launches with HIP events (bit 0: mutual sweep, bit 1: NN and FRM
    sweeps and the FRM loop kernel as a whole)."""
    _rc(lib().ddm_profile_enable(mask), "ddm_profile_enable")


def profile_read():
    """(summed sweep milliseconds, number of timed launches) since the last read."""
    ms = C.c_double(0.0); n = C.c_int64(0)
    _rc(lib().ddm_profile_read(C.byref(ms), C.byref(n)), "ddm_profile_read")
    return ms.value, n.value


# ------------------------------------------------------------------- NN
def nn(Q: torch.Tensor, R: torch.Tensor, q_rows: torch.Tensor | None = None, metric: str = "dot"):
    """Nearest neighbour of rows of Q (or Q[q_rows]) among all rows of R.

    Q: [NQ, d] (or [..., d]), R: [N, d]. metric "dot" (largest dot product) or "l2" (nearest
    point, fp32; the score is then the squared distance). Returns (idx int32 [M], score float32 [M])."""
    _check_map(Q, "Q"); _check_map(R, "R")
    d = Q.shape[-1]
    if R.shape[-1] != d or Q.dtype != R.dtype:
        raise ValueError("Q and R must share d and dtype")
    NQ, N = Q.numel() // d, R.numel() // d
    if q_rows is not None:
        q_rows = q_rows.to(device=Q.device, dtype=torch.int32).contiguous()
        M = q_rows.numel()
    else:
        M = NQ
    out_idx = torch.empty(M, dtype=torch.int32, device=Q.device)
    out_s = torch.empty(M, dtype=torch.float32, device=Q.device)
    L = lib()
    mt = METRICS[metric]
    nbytes = L.ddm_nn_ex_workspace_bytes(NQ, M, N, d, _DT[Q.dtype], mt)
    if nbytes == 0:
        raise DDMError(-4, "ddm_nn_ex_workspace_bytes (unsupported dtype, d or metric)")
    ws = _workspace(nbytes, Q.device)
    with _on(Q, R, q_rows, out_idx, ws):
        _rc(L.ddm_nn_ex(_ptr(Q), NQ, _ptr(q_rows), M, _ptr(R), N, d, _DT[Q.dtype], mt, _ptr(out_idx), _ptr(out_s),
                        _ptr(ws), ws.numel(), _stream()), "ddm_nn_ex")
    return out_idx, out_s


# ------------------------------------------------------------------- FRM
def frm_stats(query_counts, max_iter: int, N1: int, N2: int):
    """ddm_stats of each pair from an FRM call's per-iteration query counts ([B * 2 * max_iter],
    device or host; read after the call): list of dicts with iters, active (per half-step) and
    dot_products."""
    qc = torch.as_tensor(query_counts).to("cpu", torch.int32).contiguous()
    B = qc.numel() // (2 * max_iter)
    if B < 1 or qc.numel() != B * 2 * max_iter:
        raise ValueError("query_counts must hold B * 2 * max_iter entries")
    out = (FrmStats * B)()
    _rc(lib().ddm_frm_stats(C.c_void_p(qc.data_ptr()), B, max_iter, N1, N2, C.cast(out, C.c_void_p)),
        "ddm_frm_stats")
    return [dict(iters=o.iters, active=list(o.active[:2 * max_iter]), dot_products=o.dot_products) for o in out]


def _count(n) -> int:
    n = int(n)
    if n < 0:
        raise DDMError(-5, "FRM loop-kernel grid synchronisation failed (out_count = -1)")
    return n


class FrmBuffers:
    """Preallocated outputs + workspace for repeated FRM calls on one shape."""

    def __init__(self, B, H1, W1, H2, W2, d, dtype, grid_stride, max_iter, device, with_state=True):
        L = lib()
        self.k = seed_count(H1, W1, grid_stride)
        self.cap = max(self.k, 1)
        dev = device
        self.out_i = torch.empty(B * self.cap, dtype=torch.int32, device=dev)
        self.out_j = torch.empty(B * self.cap, dtype=torch.int32, device=dev)
        self.out_s = torch.empty(B * self.cap, dtype=torch.float32, device=dev)
        self.count = torch.zeros(B, dtype=torch.int32, device=dev)
        self.state = torch.empty(B * self.cap * 4, dtype=torch.int32, device=dev) if with_state else None
        self.qcounts = torch.zeros(B * 2 * max_iter, dtype=torch.int32, device=dev)
        nbytes = L.ddm_frm_workspace_bytes(B, H1, W1, H2, W2, d, _DT[dtype], grid_stride, max_iter)
        if nbytes == 0:
            raise DDMError(-1, "ddm_frm_workspace_bytes")
        self.ws = _workspace(nbytes, dev)


def frm_match_into(D1, D2, grid_stride, max_iter, buf: FrmBuffers, batched: bool = False):
    """Enqueue FRM into preallocated buffers (no host synchronisation)."""
    _check_map(D1, "D1"); _check_map(D2, "D2")
    if D1.dtype != D2.dtype or D1.shape[-1] != D2.shape[-1]:
        raise ValueError("D1 and D2 must share dtype and d")
    L = lib()
    dt = _DT[D1.dtype]
    if batched:
        B, H1, W1, d = D1.shape
        B2, H2, W2, _ = D2.shape
        if B2 != B:
            raise ValueError("batch sizes differ")
        with _on(D1, D2, buf.out_i, buf.ws):
            _rc(L.ddm_frm_match_batched(B, _ptr(D1), H1, W1, _ptr(D2), H2, W2, d, dt, grid_stride, max_iter,
                                        _ptr(buf.out_i), _ptr(buf.out_j), _ptr(buf.out_s), buf.cap, _ptr(buf.count),
                                        _ptr(buf.state), _ptr(buf.qcounts), _ptr(buf.ws), buf.ws.numel(), _stream()),
                "ddm_frm_match_batched")
    else:
        H1, W1, d = D1.shape
        H2, W2, _ = D2.shape
        with _on(D1, D2, buf.out_i, buf.ws):
            _rc(L.ddm_frm_match(_ptr(D1), H1, W1, _ptr(D2), H2, W2, d, dt, grid_stride, max_iter,
                                _ptr(buf.out_i), _ptr(buf.out_j), _ptr(buf.out_s), buf.cap, _ptr(buf.count),
                                _ptr(buf.state), _ptr(buf.qcounts), _ptr(buf.ws), buf.ws.numel(), _stream()),
                "ddm_frm_match")


def frm_match(D1: torch.Tensor, D2: torch.Tensor, grid_stride: int = 8, max_iter: int = 10,
              return_state: bool = False):
    """Fast Reciprocal Matching of [H1, W1, d] and [H2, W2, d] maps.

    Returns (i, j, score): converged reciprocal pairs, unique, ascending in i.
    With return_state, also a dict with per-seed (u, v, conv_iter) [k, 3] and the
    forward/backward query counts per iteration [2 * max_iter]."""
    H1, W1, d = D1.shape
    H2, W2, _ = D2.shape
    buf = FrmBuffers(1, H1, W1, H2, W2, d, D1.dtype, grid_stride, max_iter, D1.device, with_state=return_state)
    frm_match_into(D1, D2, grid_stride, max_iter, buf)
    n = _count(buf.count[0].item())
    res = (buf.out_i[:n].clone(), buf.out_j[:n].clone(), buf.out_s[:n].clone())
    if not return_state:
        return res
    st = buf.state.view(-1, 4)[:buf.k, :3].clone()
    return res + (dict(state=st, query_counts=buf.qcounts.clone()),)


def frm_match_batched(D1: torch.Tensor, D2: torch.Tensor, grid_stride: int = 8, max_iter: int = 10,
                      return_state: bool = False):
    """B independent pairs: D1 [B, H1, W1, d], D2 [B, H2, W2, d]. Returns a list of (i, j, score)."""
    B, H1, W1, d = D1.shape
    _, H2, W2, _ = D2.shape
    buf = FrmBuffers(B, H1, W1, H2, W2, d, D1.dtype, grid_stride, max_iter, D1.device, with_state=return_state)
    frm_match_into(D1, D2, grid_stride, max_iter, buf, batched=True)
    counts = buf.count.cpu().tolist()
    out = []
    for b in range(B):
        o = b * buf.cap
        n = _count(counts[b])
        item = (buf.out_i[o:o + n].clone(), buf.out_j[o:o + n].clone(), buf.out_s[o:o + n].clone())
        if return_state:
            st = buf.state.view(B, buf.cap, 4)[b, :buf.k, :3].clone()
            qc = buf.qcounts.view(B, -1)[b].clone()
            item = item + (dict(state=st, query_counts=qc),)
        out.append(item)
    return out


def frm_match_ex(D1: torch.Tensor, D2: torch.Tensor, *, grid_stride: int = 8, starts=None,
                 max_iter: int | None = None, pixel_tol: float = 0.0, ret_basin: bool = False,
                 return_state: bool = False, metric: str = "dot"):
    """FRM with the routine's options (explicit starts, pixel tolerance, basin map); one pair.

    ``starts``: None for the stride grid; an int tensor of linear image-1 pixels (p = x + W1*y);
    or a pair (x, y) of int tensors. Entries outside image 1 are ignored, the rest are made
    unique and ascending. ``max_iter`` defaults to 1 with starts (the routine's value) and 10
    on the grid. ``pixel_tol > 0`` needs starts: a seed is kept when its image-1 pixel moved by
    less than pixel_tol over the last iteration, and is reported at its pixel before that
    iteration. ``ret_basin`` turns the forward test off and returns basin [H1*W1] int32
    (where a backward query from each pixel went, -1 if none). ``metric`` "l2" matches fp32
    pointmaps by Euclidean distance (scores are then squared distances).

    Returns (i, j, score) [+ basin] [+ dict(state=[k, 4] (u, v, conv_iter, u_old), query_counts)]."""
    _check_map(D1, "D1"); _check_map(D2, "D2")
    if D1.dtype != D2.dtype or D1.shape[-1] != D2.shape[-1] or D1.dim() != 3 or D2.dim() != 3:
        raise ValueError("D1, D2 must be [H, W, d] maps of one dtype and d")
    H1, W1, d = D1.shape
    H2, W2, _ = D2.shape
    dev = D1.device
    if starts is not None:
        if isinstance(starts, (tuple, list)):
            x, y = starts
            starts = torch.as_tensor(x, device=dev).long() + W1 * torch.as_tensor(y, device=dev).long()
        starts = torch.as_tensor(starts, device=dev).to(torch.int32).contiguous().view(-1)
        n = starts.numel()
        if n == 0:                     # a null list would select the grid: pass a real pointer
            starts = torch.zeros(1, dtype=torch.int32, device=dev)
        if max_iter is None:
            max_iter = 1
    else:
        n = -1
        if max_iter is None:
            max_iter = 10
    L = lib()
    dt = _DT[D1.dtype]
    k = n if n >= 0 else seed_count(H1, W1, grid_stride)
    cap = max(k, 1)
    out_i = torch.empty(cap, dtype=torch.int32, device=dev)
    out_j = torch.empty(cap, dtype=torch.int32, device=dev)
    out_s = torch.empty(cap, dtype=torch.float32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    state = torch.empty(cap * 4, dtype=torch.int32, device=dev) if return_state else None
    qc = torch.zeros(2 * max_iter, dtype=torch.int32, device=dev) if return_state else None
    basin = torch.empty(H1 * W1, dtype=torch.int32, device=dev) if ret_basin else None
    mt = METRICS[metric]
    nbytes = L.ddm_frm_ex_workspace_bytes(H1, W1, H2, W2, d, dt, mt, grid_stride, n, max_iter)
    if nbytes == 0:
        raise DDMError(-1, "ddm_frm_ex_workspace_bytes")
    ws = _workspace(nbytes, dev)
    with _on(D1, D2, out_i, ws):
        _rc(L.ddm_frm_match_ex(_ptr(D1), H1, W1, _ptr(D2), H2, W2, d, dt, mt, grid_stride,
                               _ptr(starts) if n >= 0 else None, max(n, 0), max_iter, float(pixel_tol), _ptr(basin),
                               _ptr(out_i), _ptr(out_j), _ptr(out_s), cap, _ptr(count), _ptr(state), _ptr(qc),
                               _ptr(ws), ws.numel(), _stream()), "ddm_frm_match_ex")
    m = _count(count[0].item())
    res = (out_i[:m].clone(), out_j[:m].clone(), out_s[:m].clone())
    if ret_basin:
        res = res + (basin,)
    if return_state:
        # seeds = distinct valid starts: the forward queries of the first iteration
        kk = int(qc[0].item()) if n >= 0 else k
        res = res + (dict(state=state.view(-1, 4)[:kk].clone(), query_counts=qc.clone()),)
    return res


# ------------------------------------------------------------------- coarse-to-fine
def c2f_match(F1: torch.Tensor, F2: torch.Tensor, *, factor: int = 2, coarse_stride: int = 8, coarse_iter: int = 10,
              crop=(512, 384), fine_stride: int = 8, fine_iter: int = 10, return_crops: bool = False):
    """Coarse-to-fine FRM of maps larger than a crop: coarse FRM on maps subsampled by ``factor``,
    image-1 tiles of size ``crop`` (H, W), image-2 crops centred on the median coarse target of each
    tile, batched fine FRM on the crop pairs, fine matches mapped back to full resolution (first
    tile wins). Returns (i, j, score) [+ crops int32 [tiles, 5]: x0_1, y0_1, x0_2, y0_2, n_coarse]."""
    _check_map(F1, "F1"); _check_map(F2, "F2")
    if F1.dtype != F2.dtype or F1.shape[-1] != F2.shape[-1] or F1.dim() != 3 or F2.dim() != 3:
        raise ValueError("F1, F2 must be [H, W, d] maps of one dtype and d")
    H1, W1, d = F1.shape
    H2, W2, _ = F2.shape
    ch, cw = crop
    dev = F1.device
    L = lib()
    dt = _DT[F1.dtype]
    nbytes = L.ddm_c2f_workspace_bytes(H1, W1, H2, W2, d, dt, factor, coarse_stride, coarse_iter, ch, cw,
                                       fine_stride, fine_iter)
    if nbytes == 0:
        raise DDMError(-1, "ddm_c2f_workspace_bytes (bad sizes, crop, dtype or d)")
    tiles = (-(-H1 // ch)) * (-(-W1 // cw))
    cap = max(1, min(H1 * W1, tiles * seed_count(ch, cw, fine_stride)))
    out_i = torch.empty(cap, dtype=torch.int32, device=dev)
    out_j = torch.empty(cap, dtype=torch.int32, device=dev)
    out_s = torch.empty(cap, dtype=torch.float32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    crops = torch.empty(tiles * 5, dtype=torch.int32, device=dev)
    ws = _workspace(nbytes, dev)
    with _on(F1, F2, out_i, ws):
        _rc(L.ddm_c2f_match(_ptr(F1), H1, W1, _ptr(F2), H2, W2, d, dt, factor, coarse_stride, coarse_iter, ch, cw,
                            fine_stride, fine_iter, _ptr(out_i), _ptr(out_j), _ptr(out_s), cap, _ptr(count),
                            _ptr(crops), _ptr(ws), ws.numel(), _stream()), "ddm_c2f_match")
    n = _count(count[0].item())
    res = (out_i[:n].clone(), out_j[:n].clone(), out_s[:n].clone())
    return res + (crops.view(tiles, 5),) if return_crops else res


# ------------------------------------------------------------------- mutual NN
class MutualBuffers:
    def __init__(self, H1, W1, H2, W2, d, dtype, device, with_nn=False, metric: str = "dot"):
        L = lib()
        self.cap = min(H1 * W1, H2 * W2)
        self.out_i = torch.empty(self.cap, dtype=torch.int32, device=device)
        self.out_j = torch.empty(self.cap, dtype=torch.int32, device=device)
        self.out_s = torch.empty(self.cap, dtype=torch.float32, device=device)
        self.count = torch.zeros(1, dtype=torch.int32, device=device)
        self.nn12 = torch.empty(H1 * W1, dtype=torch.int32, device=device) if with_nn else None
        self.s12 = torch.empty(H1 * W1, dtype=torch.float32, device=device) if with_nn else None
        self.metric = METRICS[metric]
        nbytes = L.ddm_mutual_ex_workspace_bytes(H1, W1, H2, W2, d, _DT[dtype], self.metric)
        if nbytes == 0:
            raise DDMError(-1, "ddm_mutual_ex_workspace_bytes")
        self.ws = _workspace(nbytes, device)


def mutual_nn_into(D1, D2, buf: MutualBuffers):
    _check_map(D1, "D1"); _check_map(D2, "D2")
    if D1.dtype != D2.dtype or D1.shape[-1] != D2.shape[-1]:
        raise ValueError("D1 and D2 must share dtype and d")
    H1, W1, d = D1.shape
    H2, W2, _ = D2.shape
    with _on(D1, D2, buf.out_i, buf.ws):
        _rc(lib().ddm_mutual_nn_ex(_ptr(D1), H1, W1, _ptr(D2), H2, W2, d, _DT[D1.dtype], buf.metric,
                                   _ptr(buf.out_i), _ptr(buf.out_j), _ptr(buf.out_s), buf.cap, _ptr(buf.count),
                                   _ptr(buf.nn12), _ptr(buf.s12), _ptr(buf.ws), buf.ws.numel(), _stream()),
            "ddm_mutual_nn_ex")


def mutual_nn(D1: torch.Tensor, D2: torch.Tensor, return_nn: bool = False, metric: str = "dot"):
    """Exhaustive reciprocal nearest neighbours. Returns (i, j, score) ascending in i
    (and, with return_nn, NN2 index and score of every pixel of image 1). metric "l2":
    fp32 pointmaps by Euclidean distance, scores are squared distances."""
    H1, W1, d = D1.shape
    H2, W2, _ = D2.shape
    buf = MutualBuffers(H1, W1, H2, W2, d, D1.dtype, D1.device, with_nn=return_nn, metric=metric)
    mutual_nn_into(D1, D2, buf)
    n = int(buf.count[0].item())
    res = (buf.out_i[:n].clone(), buf.out_j[:n].clone(), buf.out_s[:n].clone())
    if return_nn:
        return res + (buf.nn12, buf.s12)
    return res


__all__ = ["nn", "frm_match", "frm_match_batched", "frm_match_into", "frm_match_ex", "c2f_match", "mutual_nn",
           "mutual_nn_into", "seed_count", "to_xy", "FrmBuffers", "MutualBuffers", "DDMError", "lib", "LIB_PATH",
           "profile_enable", "profile_read", "frm_set_mode", "frm_get_mode", "frm_set_barrier_polls",
           "debug_set_grid_cap", "debug_set_output_bitmap_limit", "frm_set_tail_after",
           "FRM_PER_HALF_STEP", "FRM_LOOP", "FRM_TAIL", "FRM_DEFAULT", "METRICS"]
