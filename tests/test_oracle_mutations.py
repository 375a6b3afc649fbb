"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/kvarn_oracle.c (in a
temporary directory), builds it with the oracle's own flags, and runs the
oracle's pin tests against that build (KVARN_ORACLE_LIB); at least one pin
must fail.  The mistakes cover the normalisation (axis order, std form,
exponent sign, iteration count, flat groups), the rotation, rounding and
packing, the binary16 conversion, the dequantisation and every attention
variant (softmax, GQA head mapping, score scale, paged slots and tail, the
fp16-cache baseline).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvarn_oracle.c")

MUTATIONS = {
    "ddof1": ("return sqrt(q / n);", "return sqrt(q / (n - 1));"),
    "std_about_zero": ("double d = v[i] - m;", "double d = v[i];"),
    "exp_sign": ("y[(size_t)t * D + j] = xt[(size_t)t * D + j] * exp(-lr[t] - lc[j]);",
                 "y[(size_t)t * D + j] = xt[(size_t)t * D + j] * exp(-lr[t] + lc[j]);"),
    "rotation_unscaled": ("row[j] *= inv;\n    }\n}", "row[j] *= 1.0;\n    }\n}"),
    "fold_wrong_axis": ("meta[j] = oracle_double_to_half(exp(lc[j]) * s[j]);           /* SK */",
                        "meta[j] = oracle_double_to_half(exp(lr[j % 128]) * s[j]);           /* SK */"),
    "levels_2b": ("int levels = (1 << bits) - 1;", "int levels = (1 << bits);"),
    "floor_not_rint": ("double r = rint(ui);", "double r = floor(ui);"),
    "pack_layouts_swapped": ("int64_t e = is_key ? (int64_t)t * D + j : (int64_t)j * TILE + t;\n            int64_t bit = e * bits;\n            out",
                             "int64_t e = !is_key ? (int64_t)t * D + j : (int64_t)j * TILE + t;\n            int64_t bit = e * bits;\n            out"),
    "fwht_sign": ("x[j + h] = a - b;", "x[j + h] = b - a;"),
    "half_ties_away": ("double r = nearbyint(ldexp(a, 10 - E));", "double r = floor(ldexp(a, 10 - E) + 0.5);"),
    "softmax_perturbed": ("sc[t] = exp(sc[t] - mx);", "sc[t] = exp(sc[t] - mx) * (1.0 + 1e-9 * t);"),
    "v_dequant_wrong": ("row[j] = cv * (c * sv + zv);", "row[j] = cv * (c * sv + zv * cv);"),
    "one_more_iteration": ("for (int it = 0; it < n_iters; ++it) {", "for (int it = 0; it <= n_iters; ++it) {"),
    "flat_groups_rescaled": ("if (all_equal(grp, TILE))\n                continue;", "if (0)\n                continue;"),
    "gqa_head_map": ("int h = g * group + hh;", "int h = g + hh;"),
    "scores_unscaled": ("sc[t] = sm_scale * acc;", "sc[t] = acc;"),
    "paged_slot_ignores_head": ("int64_t tile = (int64_t)block_table[(size_t)b * max_blocks + i] * n_kv_heads + g;",
                                "int64_t tile = (int64_t)block_table[(size_t)b * max_blocks + i] * n_kv_heads;"),
    "paged_tail_short": ("for (int t = 0; t < tl; ++t)", "for (int t = 0; t < tl - 1; ++t)"),
    "fp16_cache_k_is_v": ("K[e] = oracle_half_to_double(kb[e]);", "K[e] = oracle_half_to_double(vb[e]);"),
    "row_pass_first": None,   # the two passes of an iteration swapped (built below)
}


def _mutant(src, name):
    if name == "row_pass_first":
        i0 = src.index("        /* column pass")
        i1 = src.index("        /* row pass")
        i2 = src.index("    }\n}\n\n/* Gauge", i1)
        return src[:i0] + src[i1:i2] + src[i0:i1] + src[i2:]
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    return src.replace(old, new)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    c = tmp_path / "mutant.c"
    c.write_text(_mutant(src, name))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", str(c), "-o", str(lib), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, KVARN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "oracle and not mutation", "tests/"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "mistake %s not caught:\n%s" % (name, r.stdout[-2000:])
