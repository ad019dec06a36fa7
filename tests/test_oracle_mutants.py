"""Plants plausible mistakes in copies of the oracle's C source (on the CPU)
and checks that the oracle pins fail for every one of them.

Each mutant is compiled into a temporary directory and the oracle test
files are re-run against it through MGS_ORACLE_LIB; a mutant that passes
every pin would mean the pins cannot tell that mistake from the method.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mgs_oracle.c")

MUTANTS = {
    "eps_1e-10": ("const float eps = 1e-12f;", "const float eps = 1e-10f;"),
    "pow2_rounds_up": ("s = ldexpf(1.0f, ex - 1);", "s = ldexpf(1.0f, ex);"),
    "signed_amax_dim0": ("float a = fabsf(oracle_bf16_to_f32(x[r * K + k]));",
                         "float a = oracle_bf16_to_f32(x[r * K + k]);"),
    "skip_first_row_of_group": ("for (r = r0; r < r1; ++r)\n            for (k = 0; k < K; ++k) {\n                float a",
                                "for (r = r0 + 1; r < r1; ++r)\n            for (k = 0; k < K; ++k) {\n                float a"),
    "ties_round_down": ("r = (((int64_t)fl & 1) == 0) ? fl : fl + 1.0;", "r = fl;"),
    "ties_away": ("r = (((int64_t)fl & 1) == 0) ? fl : fl + 1.0;", "r = fl + 1.0;"),
    "no_saturation": ("        a = 448.0;                          /* clamp", "        a = a;                          /* clamp"),
    "dim1_scale_transposed": ("scales[r * G + g] = s;", "scales[(int64_t)g * M + r] = s;"),
    "unrounded_product": ("float v = oracle_bf16_to_f32(x[r * K + k]) * srow[k];",
                          "double v = (double)oracle_bf16_to_f32(x[r * K + k]) * srow[k];"),
    "rceil_ge": ("while ((double)amax > ldexp(448.0, e))", "while ((double)amax >= ldexp(448.0, e))"),
    "floor_minus_7": ("e = E - 8;", "e = E - 7;"),
    "mx_no_low_clamp": ("    if (e < -127)\n        e = -127;", "    if (e < -150)\n        e = -150;"),
    "subnormal_step": ("quantum = 0x1p-9;", "quantum = 0x1p-10;"),
    "dim1_group_start": ("int64_t c0 = g ? offsets[g - 1] : 0, c1 = offsets[g], c;",
                         "int64_t c0 = g ? offsets[g - 1] + 1 : 0, c1 = offsets[g], c;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: %s" % name
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / "mgs_oracle.c"
    c_path.write_text(mutated)
    (tmp_path / "mgs_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "mgs_oracle.h")).read())
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-w", "-o", str(so), str(c_path), "-lm"], check=True)
    env = dict(os.environ, MGS_ORACLE_LIB=str(so))
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_cast.py", "test_oracle_groups.py", "test_oracle_mx.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant %s passed every oracle pin:\n%s" % (name, r.stdout[-2000:])
