"""The CPU oracle against its pins, and the pins against planted mistakes.

The planted mistakes are made in copies of the oracle's C source, compiled
into a temporary directory; the real oracle is never modified.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins
from means_nearest_centroid_amd import workloads as W


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# (name, text in the source, replacement): each is a plausible slip.
MUTANTS = [
    ("dropped_norm_term", "double s = n[k] - 2.0 * dot;", "double s = -2.0 * dot;"),
    ("wrong_sign", "double s = n[k] - 2.0 * dot;", "double s = n[k] + 2.0 * dot;"),
    ("missing_factor_two", "double s = n[k] - 2.0 * dot;", "double s = n[k] - dot;"),
    ("ties_to_highest", "return a < b;", "return a <= b;"),
    ("transposed_operand", "dot += x[j] * cw[k * D + j];",
     "dot += x[j] * cw[j * K + k];"),
    ("nan_ranked_first", "    if (isnan(a))\n        return 0;\n    if (isnan(b))\n        return 1;",
     "    if (isnan(a))\n        return 1;\n    if (isnan(b))\n        return 0;"),
    ("bad_widening", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("dist_wrong_row", "double e = x[j] - cw[(int64_t)lab * D + j];",
     "double e = x[j] - cw[(int64_t)0 * D + j];"),
    ("runner_up_not_tracked", "                    sec = b;\n", ""),
    ("norm_not_squared", "            n += c * c;\n        }\n        norms[k] = n;",
     "            n += c;\n        }\n        norms[k] = n;"),
    # the checker helpers (score of a given label, distance to a given label)
    ("score_for_dropped_norm", "        s[i] = n - 2.0 * dot;", "        s[i] = -2.0 * dot;"),
    ("score_for_wrong_sign", "        s[i] = n - 2.0 * dot;", "        s[i] = n + 2.0 * dot;"),
    ("score_for_norm_not_squared", "            n += c * c;\n            dot +=",
     "            n += c;\n            dot +="),
    ("score_for_wrong_row",
     "const uint16_t *cr = C + (int64_t)labels[i] * D;\n        double n = 0.0, dot = 0.0;",
     "const uint16_t *cr = C + (int64_t)labels[i > 0 ? i - 1 : 0] * D;\n"
     "        double n = 0.0, dot = 0.0;"),
    ("sqdist_for_wrong_row",
     "const uint16_t *cr = C + (int64_t)labels[i] * D;\n        double d = 0.0;",
     "const uint16_t *cr = C + (int64_t)labels[0] * D;\n        double d = 0.0;"),
    ("sqdist_for_not_squared", "            d += e * e;\n        }\n        dist[i] = d;",
     "            d += fabs(e);\n        }\n        dist[i] = d;"),
    ("sqdist_for_wrong_element", "double e = widen_bf16(xr[j]) - widen_bf16(cr[j]);",
     "double e = widen_bf16(xr[j]) - widen_bf16(C[j + labels[i]]);"),
    # centroid update and its bf16 rounding
    ("mean_over_all_points", "means[k * D + j] /= (double)counts[k];",
     "means[k * D + j] /= (double)N;"),
    ("empty_cluster_zeroed", "C_new[k * D + j] = C_old[k * D + j];", "C_new[k * D + j] = 0;"),
    ("stray_labels_to_zero", "        if (k < 0 || k >= K)\n            continue;",
     "        if (k < 0 || k >= K)\n            k = 0;"),
    ("rounding_truncates", "double r = nearbyint(q);", "double r = floor(q);"),
    ("ties_away_from_zero", "double r = nearbyint(q);", "double r = round(q);"),
    ("rounding_through_fp32", "    double q = ldexp(a, 7 - e);",
     "    a = (double)(float)a;\n    double q = ldexp(a, 7 - e);"),
    ("subnormal_spacing", "        e = -126;", "        e = -127;"),
    ("overflow_kept_finite", "        return (uint16_t)(sign | 0x7F80u);\n    float f",
     "        m = largest;\n    float f"),
    ("nan_sign_dropped", "        return (uint16_t)(sign | 0x7FC0u);", "        return (uint16_t)0x7FC0u;"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, mutant_dir):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    bad = src.replace(old, new, 1)
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(bad)
    so = os.path.join(mutant_dir, f"lib_{name}.so")
    oracle.build(source=path, output=so)
    lib = oracle.load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_generator_sanity(oracle_lib):
    """Generator: points land on their generating centre (not a parity check)."""
    X, C, a = W.gaussian_mixture(4096, 64, 256, 17)
    r = oracle.assign(X, C, lib=oracle_lib)
    assert (r["labels"] == a).mean() >= 0.999


def test_adversarial_oracle_structure(oracle_lib):
    """Oracle on a scaled-down adversarial set: duplicates and equal rows."""
    X, C, meta = W.adversarial(6000, 32, 2048, 29, n_dyadic_pairs=64)
    r = oracle.assign(X, C, lib=oracle_lib)
    lab = r["labels"]
    for s, t in meta["dup_pairs"]:
        assert not np.any(lab == t), "a duplicate's higher index won"
    eq = meta["equal_rows"]
    assert not np.any(np.isin(lab, eq[1:])), "a non-lowest equal row won"
    assert np.any(lab == eq[0]), "no point on the equal rows"
    idx = meta["dyadic_points"]
    assert np.array_equal(lab[idx], meta["dyadic_labels"])
    assert np.array_equal(r["dist"][idx], meta["dyadic_sqdist"])
