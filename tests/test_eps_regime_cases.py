"""The epsilon-regime seam cases of the GPU tests must be able to fail.

RMSNorm's epsilon (1e-6, inside the root, added to the mean square, in both
the layer-input norm and the gate norm) is invisible when a token's mean
square is near 1: a seam with the epsilon outside the root differs from the
oracle by at most one bf16 ulp there, inside every bar.  The GPU tests
therefore add tokens scaled by 2^-10, 2^-12 and zero (seam_harness.
eps_regime_case).  Here, on the CPU, a copy of the oracle with the epsilon
misplaced stands in for a wrong kernel: on those cases it must fail the GPU
tests' comparison (check_all), and on an ordinary unit-scale case it passes
it, which is why those cases are needed.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from seam_harness import check_all, eps_regime_case, host_case, run_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mhc_oracle.c")

MUTANTS = {
    "norm_eps_outside_root": (
        "float rstd_u = (float)(1.0 / sqrt(su / (double)H + (double)eps));",
        "float rstd_u = (float)(1.0 / (sqrt(su / (double)H) + (double)eps));"),
    "gate_eps_outside_root": (
        "double rstd_g = 1.0 / sqrt(ss / (double)K + (double)eps);",
        "double rstd_g = 1.0 / (sqrt(ss / (double)K) + (double)eps);"),
}

RUNNER = r"""
import sys
import numpy as np
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
from seam_harness import eps_regime_case, host_case, run_oracle
for kind in ("eps", "unit"):
    for form in ("post", "no_post"):
        c = (eps_regime_case if kind == "eps" else host_case)(40, 512, seed=31)
        np.savez(f"{sys.argv[2]}/{kind}_{form}.npz", **run_oracle(c, form))
"""


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_eps_regime_cases_fail_a_misplaced_epsilon(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found"
    (tmp_path / "mut.c").write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", str(tmp_path / "mut.c"), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    subprocess.run([sys.executable, "-c", RUNNER, ROOT, str(tmp_path)], env=env, check=True,
                   timeout=300)
    for form in ("post", "no_post"):
        bad = dict(np.load(tmp_path / f"eps_{form}.npz"))
        want = run_oracle(eps_regime_case(40, 512, seed=31), form)
        with pytest.raises(AssertionError):
            check_all(bad, want, form, "bf16")
        # unit-scale tokens alone do not show the mistake
        bad_unit = dict(np.load(tmp_path / f"unit_{form}.npz"))
        check_all(bad_unit, run_oracle(host_case(40, 512, seed=31), form), form, "bf16")
