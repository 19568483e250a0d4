"""The decode kernels' query quotient, checked on the host (no GPU).

The in-wave query preparation replaces the per-element IEEE division x / s by a correctly rounded
reciprocal and one fma residual correction (tests/native/query_quotient.c states the form and the
claim).  The int8 query codes and the float-query residual codes are decisions taken in f32, so
this form must give the codes of the IEEE quotient bit for bit; the program checks that over every
binade of the row maximum and around every rounding boundary of the int8 code.  The GPU parity
tests check the kernels' codes through the score export and the outputs.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_fast_quotient_gives_ieee_codes(tmp_path):
    exe = tmp_path / "query_quotient"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "native", "query_quotient.c"),
                    "-lm"], check=True)
    r = subprocess.run([str(exe), "4000000", "12"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 quotient mismatches" in r.stdout and " 0 code mismatches" in r.stdout
