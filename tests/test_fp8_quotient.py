"""The FP8 encoders' quotient (a corrected product instead of a division)
gives the codes of true division. CPU only: compiles tests/fp8_quotient_check.c
with gcc and runs it over every fp32 value in the upper 20 binades of a block
(where codes are not zero) for scales across the fp32 range."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SCALES = ["0x1.cp+8", "0x1p+0", "0x1.8p+1", "0x1.43225p-43", "0x1.b394f4p+76", "0x1.fffffep+125"]


def test_corrected_quotient_codes_match_division():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        base = ["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "fp8_quotient_check.c"), "-o", exe, "-lm"]
        # OpenMP and the FMA unit when the host compiler has them; libm's fmaf otherwise (exact either way)
        for extra in (["-fopenmp", "-mfma"], ["-fopenmp"], []):
            if subprocess.run(base + extra, capture_output=True).returncode == 0:
                break
        else:
            pytest.fail("gcc could not build the checker")
        env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
        p = subprocess.run([exe, "20"] + SCALES, capture_output=True, text=True, env=env, timeout=900)
        print(p.stdout)
        assert p.returncode == 0, p.stdout + p.stderr
        assert p.stdout.count("0 code mismatches") == len(SCALES)
