"""The int8 activation quantizer's code rounding, checked exhaustively on the CPU.

The device quantizer forms a block's codes rne(x / d) as
rint(rint(x * 4096 * rcp(d)) / 4096) instead of a division.  That equals
rne(x / d) because a quotient of a bf16 by an fp16 value is a half-integer or
more than 2^-12 away from every half-integer, and the product's error is far
inside that gap.  ``native/q8_code_rounding.c`` runs the formula in fp32 over
every positive fp16 d and every bf16 x with |x| <= 128 d, with rcp(d) rounded
to nearest and one ulp either way, and compares with the exact rounding.  The
block format is [Sharp] "Item C2" (int8 activation blocks with an fp16 scale).
The GPU tests compare the device codes with the oracle's bit for bit; this one
covers every input the formula can meet.
"""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_code_rounding_exhaustive(tmp_path):
    exe = str(tmp_path / "q8_code_rounding")
    src = os.path.join(HERE, "native", "q8_code_rounding.c")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe, src, "-lm"]
    if subprocess.run(cmd, capture_output=True).returncode != 0:
        cmd.remove("-fopenmp")            # serial build where OpenMP is missing
        subprocess.run(cmd, check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout
    m = re.search(r"cases (\d+) mismatches (\d+)", out.stdout)
    assert m and int(m.group(1)) > 3_000_000_000 and int(m.group(2)) == 0, out.stdout
