"""The per-row int8 quantiser kernel computes x / s as r = RN(1/s),
q0 = RN(x r), q = fma(fma(-q0, s, x), r, q0) instead of a full IEEE
division.  This CPU test proves the two agree for every scale the quantiser
can produce and every finite fp16 x (2.0e9 pairs), so the kernel's codes equal
the oracle's, which divides.  The GPU parity tests then check that the kernel
implements this sequence."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_residual_quotient_is_exact(tmp_path):
    exe = str(tmp_path / "division_sequence")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                    os.path.join(HERE, "division_sequence.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    fields = dict(zip(out[0::2], map(int, out[1::2])))
    assert fields["pairs"] == 31743 * 2 * 31744      # both zeros included
    assert fields["quotient_mismatches"] == 0
    assert fields["code_mismatches"] == 0
