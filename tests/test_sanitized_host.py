"""Host code of the library under AddressSanitizer and UndefinedBehavior-
Sanitizer (no GPU): the host side of every source is compiled with the
sanitizers (the device code as usual; no kernel runs), linked with the C
client of include/tfq.h, and the client's validation checks must pass with
no sanitizer report (any report aborts the run)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_w8a8_quantized_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# sanitizer flags for the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs ROCm clang")
def test_host_validation_clean_under_asan_ubsan(tmp_path):
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    from int8_w8a8_quantized_amd.build import SOURCES

    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        jobs.append(([HIPCC] + common + SAN + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for r in ex.map(lambda j: subprocess.run(j[0], capture_output=True, text=True), jobs):
            assert r.returncode == 0, r.stderr[-2000:]
    client = str(tmp_path / "c_client.o")
    subprocess.run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "c_client.c"),
                    "-o", client], check=True)
    exe = str(tmp_path / "c_client_san")
    subprocess.run([CLANGXX, "-fsanitize=address,undefined", client] + [o for _, o in jobs] +
                   ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "c client ok" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
