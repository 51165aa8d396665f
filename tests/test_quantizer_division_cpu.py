"""The device quantizer's correctly rounded divisions, checked on the host.

The write kernels compute the scale fp32(range / L) and the reciprocal
fp32(1 / scale) of the format's quantizer without the general division
sequence: a residual-corrected multiply by RN(1/L), and the hardware
reciprocal refined by one Newton step.  The format asks for correctly
rounded results, so the same operation sequence is run on the host over
every non-negative finite binary32 range (L = 3 and 15) and every positive
fp16 scale (with every reciprocal start within two ulps), and must match the
host's IEEE division everywhere (tests/quantizer_division_check.c).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_sequences_are_correctly_rounded(tmp_path):
    exe = str(tmp_path / "quantizer_division_check")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quantizer_division_check.c"), "-lm"], check=True)
    n = max(1, min(8, len(os.sched_getaffinity(0))))
    procs = [subprocess.Popen([exe, str(i), str(n)], stdout=subprocess.PIPE, text=True) for i in range(n)]
    outs = [(p.communicate()[0], p.returncode) for p in procs]
    for out, rc in outs:
        print(out.strip())
        assert rc == 0, out
