"""Seeded synthetic descriptor maps for tests and benchmarks.

This module only draws inputs. It holds none of the matching arithmetic: no dot
products, no nearest-neighbour search, no seed grid. Both the CPU oracle
(``oracle/``) and the HIP library are fed from here, and neither imports the other.

What the inputs imitate
-----------------------
MASt3R's matching head emits one unit-norm d-vector per pixel, giving maps
D1, D2 in R^{H x W x d} (MASt3R note on cv-learn.com, section
"手法とアーキテクチャ", matching-head paragraph). Images are at most 512 px per
side (same note, coarse-to-fine paragraph). The real maps come from a trained
network on image pairs; here a Gaussian map stands in for D1 and D2 is a
warped, noisy copy of it, so that most pixels have a true counterpart.

Recipe (every step in float64, one ``numpy.random.Generator(PCG64(seed))``):

1. D1: i.i.d. N(0, 1) components, shape (H, W, d), each pixel divided by its
   L2 norm.
2. noise: i.i.d. N(0, 1), shape (H, W, d), always drawn (fixed draw order).
3. D2 at pixel (x, y) takes its source pixel from D1: (x + dx, y + dy) for a
   shift, or the nearest pixel of a rotation about the image centre. In range:
   normalise(D1[src] + sigma * noise[y, x]). With sigma == 0 the stored bits of
   D1[src] are copied unchanged, so a pure shift is exact.
   Out of range: a fresh unit vector, drawn in raster order after the noise.
4. Occlusion (optional): a rectangle of D2 is overwritten by fresh unit
   vectors, drawn after its top-left corner.
5. Storage cast: float32 (round to nearest even from float64), float16
   (numpy's round-to-nearest-even cast from float64) or bfloat16 (round to
   nearest even from the float32 value).

Layout: row-major [H][W][d]; linear pixel index p = x + W * y.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
TAU = 1e-4  # score margin under which either nearest neighbour is accepted


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast_stored(x64: np.ndarray, dtype: int) -> np.ndarray:
    """float64 -> stored representation: float32, float16 or uint16 bfloat16 bits."""
    if dtype == F32:
        return x64.astype(np.float32)
    if dtype == F16:
        return x64.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(x64.astype(np.float32))
    raise ValueError(f"unknown dtype {dtype}")


def stored_to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Stored representation -> float64 through numpy's own conversions."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


@dataclass
class Pair:
    """One synthetic descriptor-map pair in stored form."""
    D1: np.ndarray          # [H1, W1, d] float32 / float16 / uint16 (bf16 bits)
    D2: np.ndarray          # [H2, W2, d]
    dtype: int
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def H1(self): return self.D1.shape[0]
    @property
    def W1(self): return self.D1.shape[1]
    @property
    def H2(self): return self.D2.shape[0]
    @property
    def W2(self): return self.D2.shape[1]
    @property
    def d(self): return self.D1.shape[2]


def make_pair(H: int, W: int, d: int, dtype: int, seed: int, *, sigma: float,
              shift: tuple[int, int] | None = None, rotate_deg: float | None = None,
              occlusion_frac: float | None = None, rng: np.random.Generator | None = None,
              name: str = "") -> Pair:
    """Draw D1 and a warped, noisy D2 of the same H x W x d (recipe in the module doc).

    ``shift = (dx, dy)``: D2(x, y) comes from D1(x + dx, y + dy).
    ``rotate_deg``: D2(p) comes from D1(round(R(theta) (p - c) + c)), c the image
    centre ((W-1)/2, (H-1)/2), x right / y down, round(t) = floor(t + 0.5).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    D1_64 = _unit(rng.standard_normal((H, W, d)))
    noise = rng.standard_normal((H, W, d))
    D1s = cast_stored(D1_64, dtype)

    ys, xs = np.mgrid[0:H, 0:W]
    if rotate_deg is not None:
        th = math.radians(rotate_deg)
        cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
        qx = math.cos(th) * (xs - cx) - math.sin(th) * (ys - cy) + cx
        qy = math.sin(th) * (xs - cx) + math.cos(th) * (ys - cy) + cy
        sx = np.floor(qx + 0.5).astype(np.int64)
        sy = np.floor(qy + 0.5).astype(np.int64)
    else:
        dx, dy = shift if shift is not None else (0, 0)
        sx, sy = xs + dx, ys + dy
    inr = (sx >= 0) & (sx < W) & (sy >= 0) & (sy < H)
    sxc, syc = np.clip(sx, 0, W - 1), np.clip(sy, 0, H - 1)

    D2_64 = _unit(D1_64[syc, sxc] + sigma * noise)
    n_out = int((~inr).sum())
    fresh = _unit(rng.standard_normal((n_out, d)))
    D2_64[~inr] = fresh                      # boolean indexing walks raster order
    D2s = cast_stored(D2_64, dtype)
    if sigma == 0.0:
        D2s[inr] = D1s[syc[inr], sxc[inr]]   # exact copy of stored bits

    meta = dict(H=H, W=W, d=d, sigma=sigma, shift=shift, rotate_deg=rotate_deg,
                out_of_range=n_out, seed=seed)
    if occlusion_frac is not None:
        h = int(math.floor(math.sqrt(occlusion_frac) * H + 0.5))
        w = int(math.floor(math.sqrt(occlusion_frac) * W + 0.5))
        y0 = int(rng.integers(0, H - h + 1))
        x0 = int(rng.integers(0, W - w + 1))
        occ = _unit(rng.standard_normal((h, w, d)))
        D2s[y0:y0 + h, x0:x0 + w] = cast_stored(occ, dtype)
        meta.update(occlusion=(x0, y0, w, h))
    return Pair(D1s, D2s, dtype, name=name, meta=meta)


# ---------------------------------------------------------------------------
# The five workloads. Sizes read "A x B (x d)" as H x W (x d).
# ---------------------------------------------------------------------------
CONFIGS = {
    "tiny_frm_64x48x24_f32":   dict(H=64, W=48, d=24, dtype=F32, seed=1001, sigma=0.1, shift=(3, 2),
                                    stride=8, max_iter=10, mode="frm"),
    "frm_512x384x24_f16":      dict(H=512, W=384, d=24, dtype=F16, seed=1002, sigma=0.1, shift=(17, -9),
                                    stride=8, max_iter=10, mode="frm"),
    "mutual_512x384x24_f16":   dict(H=512, W=384, d=24, dtype=F16, seed=1003, sigma=0.2, shift=(17, -9),
                                    mode="mutual"),
    "batched_frm_16x512x384x24_f16": dict(B=16, H=512, W=384, d=24, dtype=F16, seed=4000, sigma=0.15,
                                          shift_range=32, stride=8, max_iter=10, mode="frm_batched"),
    "hard_frm_512x512x64_bf16": dict(H=512, W=512, d=64, dtype=BF16, seed=1005, sigma=0.3, rotate_deg=20.0,
                                     occlusion_frac=0.3, stride=4, max_iter=20, mode="frm"),
}
CONFIG_ORDER = list(CONFIGS)


def make_config(name: str) -> list[Pair]:
    """All pairs of one workload (one pair, or B pairs for the batched one)."""
    c = CONFIGS[name]
    if c["mode"] == "frm_batched":
        pairs = []
        for b in range(c["B"]):
            rng = np.random.Generator(np.random.PCG64(c["seed"] + b))
            r = c["shift_range"]
            dx, dy = (int(v) for v in rng.integers(-r, r + 1, size=2))
            pairs.append(make_pair(c["H"], c["W"], c["d"], c["dtype"], c["seed"] + b, sigma=c["sigma"],
                                   shift=(dx, dy), rng=rng, name=f"{name}[{b}]"))
        return pairs
    return [make_pair(c["H"], c["W"], c["d"], c["dtype"], c["seed"], sigma=c["sigma"],
                      shift=c.get("shift"), rotate_deg=c.get("rotate_deg"),
                      occlusion_frac=c.get("occlusion_frac"), name=name)]


def random_map(H: int, W: int, d: int, dtype: int, seed: int) -> np.ndarray:
    """A single unit-norm Gaussian map in stored form (small parity cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return cast_stored(_unit(rng.standard_normal((H, W, d))), dtype)


def large_shift_pair(H: int, W: int, d: int, dtype: int, seed: int, shift) -> Pair:
    """A large noise-free shifted pair built in float32 to bound host memory: D1 unit
    Gaussian; D2(x, y) = D1(x + dx, y + dy) with the same stored bits, fresh unit rows
    where that pixel is outside image 1. Used for property checks at sizes the oracle
    cannot sweep (the shift fixes every reciprocal pair)."""
    dx, dy = shift
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((H, W, d), dtype=np.float32)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    D1 = cast_stored(x, dtype)
    del x
    fresh = rng.standard_normal((H, W, d), dtype=np.float32)
    fresh /= np.linalg.norm(fresh, axis=-1, keepdims=True)
    D2 = cast_stored(fresh, dtype)
    del fresh
    ys, xs = slice(max(0, -dy), min(H, H - dy)), slice(max(0, -dx), min(W, W - dx))
    D2[ys, xs] = D1[max(0, dy):min(H, H + dy), max(0, dx):min(W, W + dx)]
    return Pair(D1, D2, dtype, name=f"large_shift_{H}x{W}x{d}", meta={"shift": (dx, dy)})


def large_shift_pair_device(H: int, W: int, d: int, dtype: int, seed: int, shift, device, band: int = 256):
    """As large_shift_pair, drawn on the device (torch's seeded Philox generator, fp32, in
    bands of rows) for maps too large to build on the host: returns (D1, D2) device tensors
    of the stored type (torch.float16 / torch.bfloat16)."""
    import torch
    tdt = {F16: torch.float16, BF16: torch.bfloat16}[dtype]
    dx, dy = shift
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw():
        out = torch.empty((H, W, d), dtype=tdt, device=device)
        for y0 in range(0, H, band):
            x = torch.randn((min(band, H - y0), W, d), generator=g, device=device, dtype=torch.float32)
            x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
            out[y0:y0 + x.shape[0]] = x.to(tdt)
            del x
        return out

    D1 = draw()
    D2 = draw()
    D2[max(0, -dy):min(H, H - dy), max(0, -dx):min(W, W - dx)] = \
        D1[max(0, dy):min(H, H + dy), max(0, dx):min(W, W + dx)]
    return D1, D2


def gaussian_rows(n: int, d: int, dtype: int, seed: int, unit: bool = True) -> np.ndarray:
    """n descriptor rows [n, d] in stored form (NN unit cases with arbitrary n)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d))
    return cast_stored(_unit(x) if unit else x, dtype)


# ---------------------------------------------------------------------------
# Pointmaps (3D points per pixel), for nearest-neighbour search by Euclidean
# distance: the pages match 3D points with K-d trees ("DUSt3R和MASt3R论文阅读",
# section MASt3R matching, d = 3). A pointmap gives, per pixel, the 3D point
# seen along its ray (same blog, DUSt3R section on PointMap).
# ---------------------------------------------------------------------------
def _surface_points(xs: np.ndarray, ys: np.ndarray, H: int, W: int, waves: np.ndarray) -> np.ndarray:
    """Points of a smooth random depth surface seen by a pinhole camera: depth
    z(x, y) = 2 + sum_k a_k sin(f_k . (x, y) / W + phi_k), point = (z (x - W/2) / W,
    z (y - H/2) / W, z). Defined for any real pixel coordinates."""
    z = 2.0 + np.zeros_like(xs, dtype=np.float64)
    for a, fx, fy, ph in waves:
        z += a * np.sin((fx * xs + fy * ys) / W + ph)
    return np.stack([z * (xs - W / 2) / W, z * (ys - H / 2) / W, z], axis=-1)


def pointmap_pair(H: int, W: int, seed: int, *, shift=(0, 0), sigma: float = 0.0,
                  H2: int | None = None, W2: int | None = None):
    """Two float32 pointmaps [H, W, 3] of one surface in one world frame:
    P1(x, y) = surface(x, y); P2(x, y) = surface(x + dx, y + dy) + sigma * N(0, 1) per
    coordinate (noise drawn after the surface). With sigma == 0 and an integer shift,
    the in-range pixels of P2 hold exactly the float32 points of P1 at the source."""
    rng = np.random.Generator(np.random.PCG64(seed))
    waves = np.stack([rng.uniform(0.05, 0.3, 6), rng.uniform(-12, 12, 6), rng.uniform(-12, 12, 6),
                      rng.uniform(0, 2 * math.pi, 6)], axis=1)
    H2 = H if H2 is None else H2
    W2 = W if W2 is None else W2
    ys, xs = np.mgrid[0:H, 0:W].astype(np.float64)
    P1 = _surface_points(xs, ys, H, W, waves).astype(np.float32)
    ys2, xs2 = np.mgrid[0:H2, 0:W2].astype(np.float64)
    P2 = _surface_points(xs2 + shift[0], ys2 + shift[1], H, W, waves)
    noise = rng.standard_normal(P2.shape)
    if sigma > 0:
        P2 = P2 + sigma * noise
    return P1, P2.astype(np.float32)
