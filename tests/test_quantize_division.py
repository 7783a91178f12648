"""The quantising kernels form e4m3(f32(x) / s) with a reciprocal and one
FMA correction for scales in [2^-64, 2^64], after clamping x to +-RN(440 s);
the encoding is defined on the IEEE single-precision quotient.  This
compiles and runs an exhaustive and randomised comparison of that method
with IEEE division on the CPU (gcc, no fast-math, no contraction): the
quotient bit for bit where no clamp acts, the e4m3 code and |q| <= 448
everywhere.  The kernels themselves are compared with the oracle, which
divides, by the GPU tests."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_fma_quotient_equals_ieee_division(tmp_path):
    exe = tmp_path / "quantize_division_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "quantize_division_check.c"), "-lm"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    checked, bad = int(out[0]), int(out[1])
    assert checked > (1 << 30) and bad == 0, out
