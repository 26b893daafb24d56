"""The oracle and the C ABI's host layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Each test builds the sanitized library into a temporary folder and runs the
tests that exercise it in a child process with the matching sanitizer
runtime preloaded (gcc's for the oracle, the HIP compiler's for libmoe); any
report ends that process with an error. The oracle run also shows that the
sanitizer is live: reading past the end of an input array is caught."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env, timeout=600):
    full = dict(os.environ, **SAN_ENV, **env)
    return subprocess.run(cmd, cwd=ROOT, env=full, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=timeout)


def _gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's libasan is not installed")
    return path


def test_oracle_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import oracle

    lib = oracle.build_sanitized(str(tmp_path / "liboracle_sanitized.so"))
    env = {"LD_PRELOAD": _gcc_asan(), "MOE_ORACLE_LIBRARY": lib}
    # live: an 8-token routing over a 2-token logits array reads past its end
    probe = ("import ctypes, numpy as np\n"
             "from oracle import oracle\n"
             "L = oracle.lib()\n"
             "assert L._name.endswith('liboracle_sanitized.so'), L._name\n"
             "lg = np.zeros((2, 8), np.float32)\n"
             "ids = np.zeros((8, 2), np.int32); w = np.zeros((8, 2), np.float64)\n"
             "L.oracle_route(lg.ctypes.data, 8, 8, 2, ids.ctypes.data, w.ctypes.data)\n")
    r = _run([sys.executable, "-c", probe], env)
    assert r.returncode != 0 and "AddressSanitizer" in r.stdout, r.stdout[-2000:]
    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle") and f.endswith(".py"))
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
              "not gpu", *tests], env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout


def test_abi_host_layer_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from grouped_gemm_softmax_amd import build

    lib = build.build_host_sanitized(str(tmp_path))
    env = {"LD_PRELOAD": build.asan_runtime(), "MOE_LIBRARY": lib}
    probe = ("from grouped_gemm_softmax_amd import binding as B\n"
             "B.lib()\n"
             "maps = open('/proc/self/maps').read()\n"
             "assert 'libmoe_sanitized.so' in maps and 'libclang_rt.asan' in maps\n")
    r = _run([sys.executable, "-c", probe], env)
    assert r.returncode == 0, r.stdout[-2000:]
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
              "not gpu", "tests/test_abi.py"], env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
