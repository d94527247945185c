"""The division-free quotient of the FP8 page writer, checked on the host.

For scales in [2^-63, 2^63] and bf16 values of magnitude at most 2^63 the
prefill writer encodes x / s from the reciprocal and one Newton step, with
the exact fma remainder deciding round-to-odd, instead of dividing. The C
program beside this test states that arithmetic step for step and compares
its codes with the e4m3 code of the exact quotient over every bf16 pattern
under many scales and over the bf16 values nearest to every e4m3 midpoint
times a scale; two controls (the plain fp32 quotient, the reciprocal alone)
must be caught on the same inputs. The GPU parity tests of the writer then
compare the kernel itself with the oracle on the same kinds of inputs."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_recip_quotient_equals_exact_quotient_codes(tmp_path):
    exe = tmp_path / "recip_quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "native", "recip_quotient_check.c"), "-lm"], check=True)
    res = subprocess.run([str(exe), "120"], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout
