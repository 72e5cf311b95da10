"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

core.cpp and capi.cpp (ring state machine, pool layout, window layouts, argument validation,
the C ABI) are compiled with g++ -fsanitize=address,undefined and linked with the library's
device objects into a separate libsr; the host tests then drive it in a child Python with the
ASan runtime preloaded: test_host_abi.py (validation, ring against the oracle's model,
layouts, workspace sizes) and the exhaustive tiny append/evict enumeration, which runs the
host ring through every short order of operations.  No kernel is launched.  The child fails
on the first sanitizer report (UBSan made fatal; ASan aborts by itself).
"""
import glob
import os
import subprocess
import sys

import pytest

import harness

CSRC = os.path.join(harness.ROOT, "chunk_causal_attention_amd", "csrc")
BUILD = os.path.join(harness.ROOT, "chunk_causal_attention_amd", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    harness.lib_module()  # builds libsr (and its device objects) if needed
    asan = _runtime("libasan.so")
    if not asan or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++'s ASan runtime and the HIP runtime library")
    tmp = str(tmp_path_factory.mktemp("sanitized"))
    objs = []
    for src in ("core.cpp", "capi.cpp"):
        obj = os.path.join(tmp, src + ".o")
        subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                               "-I", os.path.join(harness.ROOT, "include"), "-I", CSRC] + SAN +
                              ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    device = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
    assert device, "device objects missing"
    lib = os.path.join(tmp, "libsr_sanitized.so")
    subprocess.check_call(["g++", "-shared", "-o", lib] + objs + device + SAN +
                          ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    return lib, asan


def test_host_code_under_sanitizers(sanitized_lib):
    lib, asan = sanitized_lib
    tests = ["tests/test_host_abi.py", "tests/test_oracle_native.py::test_exhaustive_tiny_orders"]
    code = ("import sys; sys.path[:0] = ['tests', '.']\n"
            "import chunk_causal_attention_amd as sr; sr.LIB_PATH = %r\n"
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider'] + %r))\n" % (lib, tests))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=harness.ROOT, env=env,
                         timeout=900)
    log = out.stdout + out.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert out.returncode == 0, log[-4000:]
    assert " passed" in out.stdout, log[-2000:]
