"""CPU check of the arithmetic the quantize kernels use for their rounding
decisions (not of the oracle). The kernels form x / D as RN(x r) plus one
fma-remainder correction, r = RN(1/D), and round that quotient with the hardware
f32 -> fp4 conversion (element codes) or bit arithmetic (E4M3 block scale). The
nearest-even decision on the computed quotient must equal the decision on the
exact real x / D. tests/native/quotient_decisions.c tries every binary32 x in
the binades where a decision can change, for every E4M3 mantissa (element
codes) and for the divisor 6 (block scale), and checks that a zero quotient
keeps the sign of x. The decision on the exact quotient is what the oracle
computes (nearest value, ties to the even code, on x / D and amax / (6 g)).

The hardware conversion's own rounding (nearest even, saturating at 6, sign
kept) is covered on the GPU by the bit-exact quantize parity tests, whose
inputs sit on every rounding edge."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "quotient_decisions.c")


def test_quotient_decisions_match_exact_division(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "quotient_decisions")
    flags = ["-O2", "-ffp-contract=off"]
    omp = subprocess.run([cc, *flags, "-fopenmp", "-o", exe, SRC, "-lm"], capture_output=True, text=True)
    if omp.returncode != 0:
        subprocess.run([cc, *flags, "-o", exe, SRC, "-lm"], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all decisions agree" in r.stdout
