"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutation edits one spot of a private copy of oracle/oracle.c (a dropped
term, a flipped comparison, a wrong index, a swapped operand, an off-by-one),
builds it with gcc into a temporary directory and runs the pins of
test_oracle_pins.py against that build. At least one pin must fail for every
mutation; the unmodified source must pass them all.
"""
import os
import subprocess
import sys

import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "dropped_first_term": ("for (int c = 0; c < d; ++c) s += a[c] * b[c];",
                           "for (int c = 1; c < d; ++c) s += a[c] * b[c];"),
    "dropped_last_term": ("for (int c = 0; c < d; ++c) s += a[c] * b[c];",
                          "for (int c = 0; c + 1 < d; ++c) s += a[c] * b[c];"),
    "wrong_sign": ("s += a[c] * b[c];", "s -= a[c] * b[c];"),
    "ties_to_highest": ("if (s > b1) { b2 = b1;", "if (s >= b1) { b2 = b1;"),
    "no_second_best": ("else if (s > b2) { b2 = s; }", "else if (s > b1) { b2 = s; }"),
    "half_exponent_bias": ("v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    "half_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "seed_offset_zero": ("for (int y = S / 2; y < H; y += S)", "for (int y = 0; y < H; y += S)"),
    "seed_index_transposed": ("if (out) out[k] = x + W * y;", "if (out) out[k] = y + H * x;"),
    "forward_test_vs_u": ("if (fwd_test && active[a] && v[a] == v_old[a])",
                          "if (fwd_test && active[a] && v[a] == u_old[a])"),
    "backward_test_vs_v": ("if (active[a] && u[a] == u_old[a])", "if (active[a] && u[a] == v_old[a])"),
    "no_forward_test": ("if (fwd_test && active[a] && v[a] == v_old[a])", "if (0 && v[a] == v_old[a])"),
    "max_iter_off_by_one": ("if (niter >= max_iter) break;", "if (niter > max_iter) break;"),
    "old_not_updated": ("for (int64_t a = 0; a < k; ++a) { v_old[a] = v[a]; u_old[a] = u[a]; }",
                        "for (int64_t a = 0; a < k; ++a) { v_old[a] = v[a]; }"),
    "backward_against_own_map": ("nn_one_m(D2 + (int64_t)v[a] * d, D1, N1, d, metric, &i, &s1, &s2);",
                                 "nn_one_m(D2 + (int64_t)v[a] * d, D2, N2, d, metric, &i, &s1, &s2);"),
    "forward_query_from_wrong_map": ("nn_one_m(D1 + (int64_t)u[a] * d, D2, N2, d, metric, &j, &s1, &s2);",
                                     "nn_one_m(D2 + (int64_t)u[a] * d, D2, N2, d, metric, &j, &s1, &s2);"),
    "l2_unsquared": ("        s -= t * t;", "        s -= t < 0 ? -t : t;"),
    "l2_sign_flipped": ("        s -= t * t;", "        s += t * t;"),
    "l2_metric_ignored": ("double s = metric == ORC_L2 ? neg_sqdist(q, R + j * d, d) : dot(q, R + j * d, d);",
                          "double s = dot(q, R + j * d, d);"),
    "converged_keeps_active": ("if (active[a]) continue;\n        buf[3 * m]", "if (!active[a]) continue;\n        buf[3 * m]"),
    "basin_at_new_pixel": ("if (active[a]) basin[u_old[a]] = u[a];", "if (active[a]) basin[u[a]] = u[a];"),
    "u_old_export_is_u": ("u_old_out[a] = u_old[a];", "u_old_out[a] = u[a];"),
    "fwd_test_flag_ignored": ("if (fwd_test && active[a] && v[a] == v_old[a])",
                              "if (active[a] && v[a] == v_old[a])"),
    "tol_not_strict": ("keep[a] = sqrt(dy * dy + dx * dx) < pixel_tol;",
                       "keep[a] = sqrt(dy * dy + dx * dx) <= pixel_tol;"),
    "tol_reports_new_pixel": ("rep_i[a] = report_old ? u_old[a] : u[a];", "rep_i[a] = u[a];"),
    "tol_distance_ignores_rows": ("const double dy = (double)(u_old[a] / W1 - u[a] / W1);",
                                  "const double dy = 0.0;"),
    "mutual_check_wrong_table": ("if (nn21[j] == (int32_t)i) {", "if (nn12[j] == (int32_t)i) {"),
    "mutual_score_wrong": ("out_s[n] = s12[i];", "out_s[n] = s21[i];"),
}

# Planted mistakes in the Python part of the oracle (the coarse-to-fine reading).
PY_MUTATIONS = {
    "c2f_upper_median": ("mx = int(np.sort(x2[inside])[(n - 1) // 2])", "mx = int(np.sort(x2[inside])[n // 2])"),
    "c2f_no_clamp_right": ("x02 = min(max(mx - crop_w // 2, 0), W2 - crop_w)", "x02 = max(mx - crop_w // 2, 0)"),
    "c2f_centre_not_halved": ("y02 = min(max(my - crop_h // 2, 0), H2 - crop_h)",
                              "y02 = min(max(my - crop_h, 0), H2 - crop_h)"),
    "c2f_last_crop_wins": ("            if a not in owner:\n", "            if True:\n"),
    "c2f_factor_ignored": ("x1 = (ci % Wc1) * factor; y1 = (ci // Wc1) * factor",
                           "x1 = (ci % Wc1); y1 = (ci // Wc1)"),
    "c2f_last_tile_not_moved": ("x0 = min(tx * crop_w, W1 - crop_w)", "x0 = tx * crop_w"),
}
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

# pins, as callables with fixed arguments
PINS = [
    P.test_decode_f16_all_patterns,
    lambda: P.test_nn_matches_numpy_argmax(37, 53, 24, 1),
    lambda: P.test_nn_matches_numpy_argmax(5, 9, 1, 3),
    P.test_nn_ties_take_lowest_index,
    P.test_nn_score_is_exact_for_f16_inputs,
    P.test_seed_grid_closed_forms,
    lambda: P.test_frm_handworked_fixture("row"),
    lambda: P.test_frm_equals_orbit_derivation((12, 9), (12, 9), 24, 23, 10),
    lambda: P.test_frm_equals_orbit_derivation((6, 10), (9, 7), 2, 22, 2),
    lambda: P.test_frm_pairs_are_reciprocal_and_inside_mutual_set(31),
    P.test_frm_identity_map,
    lambda: P.test_frm_pure_shift_closed_form(3, 2),
    lambda: P.test_mutual_matches_numpy((7, 9), (11, 5), 3, 52),
    P.test_mutual_symmetry,
] + [(lambda c=c: P.test_frm_ex_handworked_fixture(c)) for c in range(8)] + [
    lambda: P.test_frm_ex_equals_orbit_derivation((6, 10), 2, 62, 3, 0.0, True),
    lambda: P.test_frm_ex_equals_orbit_derivation((12, 9), 24, 63, 2, 2.5, False),
    lambda: P.test_frm_ex_equals_orbit_derivation((1, 40), 2, 64, 10, 1.0, False),
    P.test_frm_ex_identity_and_shift_closed_forms,
    P.test_l2_nn_matches_kdtree,
    P.test_l2_nn_ties_and_numpy,
    P.test_l2_mutual_matches_numpy,
    lambda: P.test_l2_frm_equals_orbit_derivation(3),
    P.test_crop_windows_hand_example,
    P.test_coarse_to_fine_single_crop_is_frm,
    lambda: P.test_coarse_to_fine_pure_shift(6, -4),
    P.test_coarse_to_fine_pairs_reciprocal_within_crop,
    P.test_merge_first_wins_hand_example,
]


def _build(src_text, out_dir, name):
    c_path = os.path.join(out_dir, f"{name}.c")
    so_path = os.path.join(out_dir, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", so_path, c_path, "-lm"], check=True)
    return so_path


def count_failures(so_path):
    """Run every pin against one oracle build; returns how many fail."""
    failed = 0
    with oracle.use_library(so_path):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, IndexError, ValueError, MemoryError):
                failed += 1
    return failed


_RUNNER = """
import sys
sys.path[:0] = sys.argv[2:]
import test_oracle_mutations as M
sys.exit(min(M.count_failures(sys.argv[1]), 100))
"""


def _failures(so_path, py_root=None):
    # A mutant may read or write out of bounds and crash; run it in its own
    # process. A crash counts as a failed pin (the mistake was noticed).
    # py_root: a directory holding a mutated copy of the oracle package, put first on the path.
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    paths = ([py_root] if py_root else []) + [here, root]
    r = subprocess.run([sys.executable, "-c", _RUNNER, so_path, *paths], capture_output=True, text=True,
                       timeout=600)
    if r.returncode < 0 or r.returncode > 100:
        return 1
    return r.returncode


def test_unmodified_source_passes_all_pins(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert _failures(_build(text, str(tmp_path), "orig")) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    with open(SRC) as f:
        text = f.read()
    old, new = MUTATIONS[name]
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(old, new, 1)
    assert _failures(_build(mutated, str(tmp_path), name)) >= 1, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_planted_python_mistake_is_caught(name, tmp_path):
    with open(PY_SRC) as f:
        text = f.read()
    old, new = PY_MUTATIONS[name]
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(text.replace(old, new, 1))
    with open(SRC) as f:
        so = _build(f.read(), str(tmp_path), "orig")
    (pkg / "oracle.c").write_text(open(SRC).read())
    assert _failures(so, str(tmp_path)) >= 1, f"no pin caught mutation {name}"
