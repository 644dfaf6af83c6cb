"""The identities behind the GPU quantizer's fast exact arithmetic, checked
on the host's IEEE fp32 (see tests/native/quant_identities.c): the rounding
by pred(1/2) (exhaustive), RN(m/7) by one correction step (exhaustive) and
Markstein's correction for the codes (sampled).  The GPU parity tests then
confirm that the kernels, built from these steps, agree with the oracle."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_quantizer_arithmetic_identities(tmp_path):
    exe = str(tmp_path / "quant_identities")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", "-std=c11", "-o", exe,
                    os.path.join(HERE, "native", "quant_identities.c"), "-lm"], check=True)
    r = subprocess.run([exe, "100000000"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    for line in r.stdout.splitlines():
        assert line.split(":")[1].strip().startswith("0 mismatches"), line
