"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a copy of the oracle's C source with one plausible slip (a
dropped term, a wrong sign, a swapped axis or index), compiled on the CPU into
a temporary library. The pins of test_oracle_pins.py then run against it; a
mutant that passes them all would mean the pins cannot see that kind of
mistake.
"""
import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = {
    "no_dilation": ("ref = x[a] + dil[a] * (idx[a] - (k[a] - 1) / 2)", "ref = x[a] + (idx[a] - (k[a] - 1) / 2)"),
    "point_order_w_slowest": ("{p / (k[1] * k[2]), (p / k[2]) % k[1], p % k[2]}",
                              "{p % k[0], (p / k[0]) % k[1], p / (k[0] * k[1])}"),
    "offset_sign": ("pos[a] = (float)ref + dlt[a];", "pos[a] = (float)ref - dlt[a];"),
    "offset_axes_reversed": ("pos[a] = (float)ref + dlt[a];", "pos[a] = (float)ref + dlt[2 - a];"),
    "trunc_not_floor": ("float fl = floorf(pos[a]);", "float fl = truncf(pos[a]);"),
    "weight_flipped_t": ("at = ct ? ft : 1.0 - ft", "at = ct ? 1.0 - ft : ft"),
    "frac_axes_swapped": ("ft = frac[0], fh = frac[1]", "ft = frac[1], fh = frac[0]"),
    "corner_axis_mixup": ("x = (int64_t)base[2] + cw", "x = (int64_t)base[2] + ch"),
    "deriv_sign": ("st = ct ? 1.0 : -1.0", "st = ct ? -1.0 : 1.0"),
    "deriv_wrong_factor": ("dw[1] = at * sh * aw;", "dw[1] = at * sh * ah;"),
    "lse_without_max": ("*lse = m + log(z);", "*lse = log(z);"),
    "unnormalised_softmax": ("a[p] = exp(s[p] - m) / z;", "a[p] = exp(s[p] - m);"),
    "no_scale_on_logits": ("s[p] = scale * acc;", "s[p] = acc;"),
    "dq_without_centering": ("acc += a[p] * (da[p] - sum_ada) * kp[(long)p * d + e];",
                             "acc += a[p] * da[p] * kp[(long)p * d + e];"),
    "dk_without_scale": ("gk[e] = pr->scale * ds * qi[e];", "gk[e] = ds * qi[e];"),
    "dv_without_weight": ("gv[e] = a[p] * gi[e];", "gv[e] = gi[e];"),
    "doff_without_value_term": ("dot += gk[e] * Kc[e] + gv[e] * Vc[e];", "dot += gk[e] * Kc[e];"),
    "dk_missing_corner_weight": ("dK[r * d + e] += w * gk[e];", "dK[r * d + e] += gk[e];"),
    "border_wraps": ("if (t < 0 || t >= pr->T ||", "if (t < -1 || t >= pr->T ||"),
    # hybrid attention (global tokens in the softmax)
    "hybrid_dgk_without_scale": ("dGK[(long)g * d + e] += pr->scale * ds * qi[e];",
                                 "dGK[(long)g * d + e] += ds * qi[e];"),
    "hybrid_dgv_unweighted": ("dGV[(long)g * d + e] += a[P + g] * gi[e];", "dGV[(long)g * d + e] += gi[e];"),
    "hybrid_keys_from_values": ("kp[(long)P * d + e] = GK[e];", "kp[(long)P * d + e] = GV[e];"),
    "hybrid_dq_without_global_rows": ("for (int j = 0; j < R; ++j) acc += a[j] * (da[j] - sum_ada) * kp[(long)j * d + e];",
                                      "for (int j = 0; j < P; ++j) acc += a[j] * (da[j] - sum_ada) * kp[(long)j * d + e];"),
}

# a quick selection of the pins (each is a plain function of the loaded oracle)
PIN_CALLS = [
    ("zero_offsets", lambda: pins.test_zero_offsets_equal_fixed_window_attention((3, 5, 5), (1, 2, 2))),
    ("integer_gathers", pins.test_integer_offsets_are_exact_gathers),
    ("grid_sample_route", lambda: pins.test_matches_grid_sample_route_with_autograd((3, 3, 3), (1, 2, 2), 1.3)),
    ("grid_sample_route_p75", lambda: pins.test_matches_grid_sample_route_with_autograd((3, 5, 5), (1, 1, 1), 2.0)),
    ("geometry", pins.test_geometry_is_single_precision_floor_and_fraction),
    ("affine", pins.test_affine_field_is_reproduced_at_the_sample_position),
    ("softmax", pins.test_attention_weights_are_a_distribution_and_uniform_for_zero_keys),
    ("hybrid_route", lambda: pins.test_hybrid_matches_grid_sample_route_with_global_keys((3, 3, 3), (1, 1, 1), 0.8, 5)),
]


def _fails_some_pin():
    for name, fn in PIN_CALLS:
        try:
            fn()
        except Exception:  # an assertion or an oracle error both count as caught
            return name
    return None


def test_unmutated_source_passes_the_selection(tmp_path):
    path = oracle.build_variant(oracle.source_text(), str(tmp_path / "liborc_same.so"))
    prev = oracle._use_library(path)
    try:
        assert _fails_some_pin() is None
    finally:
        oracle._restore_library(prev)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    path = oracle.build_variant(src.replace(old, new), str(tmp_path / f"liborc_{name}.so"))
    prev = oracle._use_library(path)
    try:
        caught = _fails_some_pin()
    finally:
        oracle._restore_library(prev)
    assert caught is not None, f"no pin catches the planted mistake '{name}'"
