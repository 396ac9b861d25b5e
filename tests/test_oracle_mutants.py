"""Each oracle pin catches a plausible mistake: the oracle's source is copied, one mistake is planted in one
function (a dropped term, a wrong sign or index, a transposed operand, a missing update), the copy is built, and a
pin that the real oracle passes must fail against it. CPU only; the oracle itself is never changed."""
import numpy as np
import pytest

import oracle
import oracle_mutants
import test_oracle_backward as bwd
import test_oracle_composite as comp
import test_oracle_isect as isect
import test_oracle_sort_offsets as sortoff


def _isect_brute_force():
    from tile_binned_gaussian_amd import synth
    isect.check_against_brute(oracle, synth.random_scene(41, 3, 80, 50, 40, 8, elliptical=True), sort=False)


def _sort_ties():
    sortoff.test_sort_matches_numpy_stable(oracle, 30000, 100)


MUTANTS = [
    # (name, function, old text, new text, pin)
    ("floor taken as ceil for x0", "orc_bounds", "bounds[0] = orc_clamp_tile(floorf(", "bounds[0] = orc_clamp_tile(ceilf(",
     lambda: isect.test_hand_example(oracle)),
    ("row and column of the rectangle swapped", "orc_isect_emit",
     "row = r[1] + k / w, column = r[0] + k % w", "row = r[1] + k % w, column = r[0] + k / w",
     lambda: isect.test_hand_example(oracle)),
    ("camera dropped from the key", "orc_isect_emit", "orc_pack_key((uint64_t)(i / N),", "orc_pack_key(0,",
     _isect_brute_force),
    ("ties merged right-first (unstable)", "orc_sort_pairs", "if (sk[b] < sk[a])", "if (sk[b] <= sk[a])",
     _sort_ties),
    ("offsets shifted by one tile", "orc_tile_offsets", "offsets[t - 1] + per_tile[t - 1]",
     "offsets[t - 1] + per_tile[t]", lambda: sortoff.test_offsets_match_bincount(oracle)),
    ("a Taylor term dropped from the exponential", "orc_exp_neg", "    p = fmaf(p, r, 1.0f / 24.0f);\n", "",
     lambda: comp.test_exp_accuracy_dense_sweep(oracle)),
    ("sign of the quadratic form's cross term", "orc_evaluate", "+ b * e.dx * e.dy", "- b * e.dx * e.dy",
     lambda: comp.test_pixel_centre_and_cross_term(oracle)),
    ("early-out taken after compositing", "orc_composite_pixel_traced",
     "if (T_next <= transmittance_threshold) break;", "if (T_next <= transmittance_threshold && 0) break;",
     lambda: comp.test_transmittance_early_out_stack(oracle)),
    ("behind-colour not divided by 1 - alpha", "orc_rasterize_bwd", "- S[k] / one_minus", "- S[k]",
     bwd.test_two_splats_closed_form),
    ("transmittance not advanced", "orc_rasterize_bwd", "T *= 1.0 - (double)e.alpha;", ";",
     bwd.test_two_splats_closed_form),
    ("conic entries swapped in the mean term", "orc_rasterize_bwd", "d_sigma * (a * dx + b * dy)",
     "d_sigma * (c * dx + b * dy)", lambda: bwd.test_finite_differences(0)),
    ("clamp ignored", "orc_rasterize_bwd", "st->unclamped ? d_alpha : 0.0", "d_alpha",
     bwd.test_clamped_splat_has_no_shape_or_opacity_gradient),
    ("background gradient without the transmittance", "orc_rasterize_bwd", "gk[k] * T_f, fabs(gk[k]) * T_f",
     "gk[k], fabs(gk[k])", bwd.test_background_gradient_is_sum_of_transmittance),
]


@pytest.mark.parametrize("name,function,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_its_pin(tmp_path, name, function, old, new, pin):
    path = oracle_mutants.build(tmp_path, function, old, new)
    with oracle.variant(path):
        with pytest.raises(AssertionError):
            pin()
    pin()  # the real oracle passes it
