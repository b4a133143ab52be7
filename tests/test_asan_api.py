"""api.cpp's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, CPU): api.cpp is compiled with
g++ -fsanitize=address,undefined and linked with the library's other
objects (built normally) and tests/asan/api_validation.cpp, which calls every
entry point with invalid arguments and with empty problems; none of them
reaches a launch."""
import glob
import os
import shutil
import subprocess

import pytest

from block_sparse_attention_bsattn_amd import _build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPLIB = "/opt/rocm/lib"


def _objects():
    return sorted(o for o in glob.glob(os.path.join(B.BUILD, "*.o"))
                  if os.path.basename(o) != "api.cpp.o")


@pytest.mark.timeout(600)
def test_api_validation_under_asan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(HIPLIB, "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    if len(_objects()) != len(B.SOURCES) - 1:
        B.build()
    objs = _objects()
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{B.CSRC}"]
    api_o = str(tmp_path / "api_asan.o")
    r = subprocess.run([gxx, "-std=c++17", *san, *inc, "-c",
                        os.path.join(B.CSRC, "api.cpp"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "api_validation")
    r = subprocess.run([gxx, "-std=c++17", *san, *inc,
                        os.path.join(ROOT, "tests", "asan", "api_validation.cpp"), api_o,
                        *objs, f"-L{HIPLIB}", "-lamdhip64", f"-Wl,-rpath,{HIPLIB}",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok: 0 failures" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr
