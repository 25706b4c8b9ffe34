"""The host C++ of libtq (tq_api.cpp, tq_codebook.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through its C ABI by tests/host_check.cpp: codebooks of
every family, width and head dimension, sign vectors, size queries and the argument validation
of every call.  The kernels' objects are linked unchanged (nothing is launched: the driver only
passes arguments that fail validation, or sizes of zero).  CPU only; about 30 s."""

import os
import shutil
import subprocess

import pytest

from packed_decode_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def test_host_code_under_sanitizers(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    device_objs = [os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
                   for src, kind, _ in B.SOURCES if kind == "device"]
    if not all(os.path.exists(o) for o in device_objs):
        pytest.skip("the library is not built")
    hip_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(B.HIPCC))), "lib")
    objs = []
    for src in (os.path.join(B.CSRC, "tq_api.cpp"), os.path.join(B.CSRC, "tq_codebook.cpp"),
                os.path.join(ROOT, "tests", "host_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", *SAN, "-c", src, "-o", obj],
                       check=True)
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    subprocess.run(["g++", *SAN, *objs, *device_objs, f"-L{hip_lib}", "-lamdhip64", f"-Wl,-rpath,{hip_lib}",
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "host checks: 0 failures" in r.stdout
