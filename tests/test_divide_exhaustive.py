"""The quantiser's division shortcut, checked exhaustively on the host.

The row quantisers evaluate x / s (TeleFuser "Quantization", "Scaled FP8
checkpoints: W8A8" and "Core ideas") as one Markstein correction of x * RN(1/s)
with fused multiply-adds (remainder negated so that zeros keep their sign), and divide for real only when s is outside
[2^-90, 2^126].  ``divide_check.c`` replays that arithmetic in binary32 on the
host (FMA and division are correctly rounded there as on the GPU) for every
positive finite BF16 amax and every BF16 x of either sign with |x| <= amax,
with s = RN(amax / qmax), and requires:

* the same binary32 quotient as RN(x / s) wherever |x / s| >= 2^-12;
* below that, a result under 2^-10 in magnitude with the sign of x (zeros
  included), which encodes to the same signed zero as the true quotient
  (E4M3FN rounds anything at or below 2^-10 to zero; INT8 anything below 1/2);
* no quotient larger in magnitude than that of x = amax (so a row whose amax
  quotient is <= qmax needs no clamp);
* the same at the edges of the fast-path window (s = 2^-90 and s = 2^126).

The qmax values are the ones the workloads use: 448 (E4M3FN), the reduced
activation qmax 14, 12 and 7 of LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16
累加", and 127 (INT8).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "divide_check.c")


@pytest.fixture(scope="module")
def divide_check(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divchk") / "divide_check")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp", "-o", exe, SRC, "-lm"]
    # hardware FMA where the host has it (libm's fmaf is also correctly rounded)
    r = subprocess.run([gcc, "-mfma", *flags], capture_output=True, text=True)
    if r.returncode != 0:
        r = subprocess.run([gcc, *flags], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("qmax", ["448", "14", "12", "7", "127"])
def test_markstein_quotient_equals_true_division(divide_check, qmax):
    r = subprocess.run([divide_check, qmax], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    line = r.stdout.strip()
    assert " 0 mismatches" in line, line
    # every pair was visited: sum over amax of 2 (amax_bits + 1) for the
    # fast-path scales, plus the two edge sweeps
    tested = int(line.split(":")[1].split()[0])
    assert tested > 10 ** 9, line
