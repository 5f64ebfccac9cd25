"""The FP8 activation quantiser forms x / s as a corrected reciprocal product instead of an
IEEE division per element; tests/quant_quotient_check.c checks, over every bf16 value and
every bf16 token maximum, that the codes cannot change (the IEEE quotient x / s of
oracle/proj.py's quantize_tokens is what the codes are defined on).  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_reciprocal_equals_ieee_quotient(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "quant_quotient_check")
    # No contraction: the products and sums are exactly the kernel's, each rounded once.
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "quant_quotient_check.c"),
                    "-o", exe, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    pairs, wrong, crossing = map(int, out.split())
    assert pairs > 700_000_000, pairs            # every (maximum, value) pair with s >= 2^-80
    assert wrong == 0, f"{wrong} quotients >= 2^-10 differ from the IEEE division"
    assert crossing == 0, f"{crossing} quotients below 2^-10 cross it or change sign"
