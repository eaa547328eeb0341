"""Seeded input generators (no method arithmetic): the relations the GPU property tests rely on."""
import numpy as np

import synth


def test_large_shift_pair_is_an_exact_shift():
    H, W, dx, dy = 40, 56, 7, -5
    p = synth.large_shift_pair(H, W, 8, synth.F16, 3, (dx, dy))
    assert p.D1.dtype == np.float16 and p.D1.shape == (H, W, 8) and p.D2.shape == (H, W, 8)
    ys, xs = np.mgrid[0:H, 0:W]
    inside = (xs + dx >= 0) & (xs + dx < W) & (ys + dy >= 0) & (ys + dy < H)
    src = p.D1[np.clip(ys + dy, 0, H - 1), np.clip(xs + dx, 0, W - 1)]
    assert np.array_equal(p.D2[inside], src[inside])
    # fresh rows elsewhere, and every row near unit norm
    assert not np.array_equal(p.D2[~inside], src[~inside])
    n = np.linalg.norm(p.D2.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 2e-3
    again = synth.large_shift_pair(H, W, 8, synth.F16, 3, (dx, dy))
    assert np.array_equal(again.D1, p.D1) and np.array_equal(again.D2, p.D2)


def test_same_seed_same_bits_and_shapes():
    a = synth.make_pair(40, 30, 24, synth.F16, 5, sigma=0.1, shift=(3, -2))
    b = synth.make_pair(40, 30, 24, synth.F16, 5, sigma=0.1, shift=(3, -2))
    c = synth.make_pair(40, 30, 24, synth.F16, 6, sigma=0.1, shift=(3, -2))
    assert a.D1.shape == a.D2.shape == (40, 30, 24) and a.D1.dtype == np.float16
    assert np.array_equal(a.D1, b.D1) and np.array_equal(a.D2, b.D2)
    assert not np.array_equal(a.D1, c.D1)
    bf = synth.make_pair(8, 6, 16, synth.BF16, 5, sigma=0.1)
    assert bf.D1.dtype == np.uint16 and bf.D1.shape == (8, 6, 16)


def test_bf16_rounding_is_nearest_even():
    # halfway cases between two bf16 values (low 16 bits 0x8000) round to the even one
    x = np.array([0x3F808000, 0x3F818000, 0x3F80_7FFF, 0x3F80_8001, 0xBF818000], np.uint32).view(np.float32)
    got = synth.f32_to_bf16_bits(x)
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F80, 0x3F81, 0xBF82]
    # and every value lands on the nearer neighbour
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000).astype(np.float32)
    r = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)).astype(np.float64)
    u = v.view(np.uint32)
    lo = (u & 0xFFFF0000).view(np.float32).astype(np.float64)
    hi = ((u & 0xFFFF0000) + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.all(np.abs(r - v) <= np.minimum(np.abs(v - lo), np.abs(v - hi)) + 0)


def test_fp16_rounding_matches_numpy_nearest_even():
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -11)], np.float64)   # exact halfway cases
    got = synth.cast_stored(x, synth.F16)
    assert got.tolist() == [1.0, 1 + 2 ** -9, -1.0]


def test_shift_in_range_fraction_and_rows():
    H, W, dx, dy = 512, 384, 17, -9
    p = synth.make_pair(H, W, 8, synth.F32, 3, sigma=0.1, shift=(dx, dy))
    frac_out = p.meta["out_of_range"] / (H * W)
    expect = 1 - (W - abs(dx)) * (H - abs(dy)) / (H * W)
    assert abs(frac_out - expect) < 1e-12 and 0.05 < frac_out < 0.07      # ≈ 6.1 % at the headline shift
    n = np.linalg.norm(p.D2.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-6


def test_occlusion_area_near_thirty_percent():
    (p,) = synth.make_config("hard_frm_512x512x64_bf16")
    x0, y0, w, h = p.meta["occlusion"]
    assert w == h == 280 and abs(w * h / (512 * 512) - 0.3) < 0.01
    assert 0 <= x0 <= 512 - w and 0 <= y0 <= 512 - h
    assert p.meta["rotate_deg"] == 20.0


def test_batched_config_shifts_in_range():
    pairs = synth.make_config("batched_frm_16x512x384x24_f16")
    assert len(pairs) == 16
    shifts = [pr.meta["shift"] for pr in pairs]
    assert all(-32 <= dx <= 32 and -32 <= dy <= 32 for dx, dy in shifts)
    assert len(set(shifts)) > 8


def test_device_drawn_shift_pair_is_an_exact_shift():
    """The device-side generator of the pixel-limit test, run on the CPU device at a tiny size."""
    import torch
    H, W, dx, dy = 24, 40, 5, -3
    D1, D2 = synth.large_shift_pair_device(H, W, 8, synth.F16, 9, (dx, dy), "cpu", band=7)
    assert D1.dtype == torch.float16 and D1.shape == (H, W, 8)
    a, b = D1.numpy(), D2.numpy()
    for y in range(H):
        for x in range(W):
            if 0 <= x + dx < W and 0 <= y + dy < H:
                assert np.array_equal(b[y, x], a[y + dy, x + dx])
    assert np.abs(np.linalg.norm(a.astype(np.float64), axis=-1) - 1).max() < 2e-3
    E1, _ = synth.large_shift_pair_device(H, W, 8, synth.F16, 9, (dx, dy), "cpu", band=7)
    assert torch.equal(E1, D1)
