"""The C ABI from C: tests/c_client.c is compiled as C11 against
include/tfq.h, linked with libtfq.so and run (host validation only, no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "int8_w8a8_quantized_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_compiles_links_and_validates(tmp_path):
    lib = os.path.join(LIBDIR, "libtfq.so")
    if not os.path.exists(lib):
        pytest.skip("libtfq.so is not built")
    exe = str(tmp_path / "c_client")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_client.c"),
                    "-L", LIBDIR, "-ltfq", "-Wl,-rpath," + LIBDIR, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client ok" in r.stdout
