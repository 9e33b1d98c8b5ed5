"""Host sanitizers (CPU only): the oracle's C code and the C ABI's host code
(argument validation, workspace sizing and carving, error messages) run under
AddressSanitizer and UndefinedBehaviorSanitizer.

Each leg builds a sanitized copy of its library, then runs an existing CPU test
module against it in a child process that preloads the matching sanitizer
runtime: the oracle pins (gcc's runtimes) and the ABI boundary tests (clang's,
which the HIP compiler uses).  Any sanitizer report fails the child."""
import glob
import os
import subprocess
import sys

import pytest

from gguf_block_quantized_q8_amd import _build as ggq_build
from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "gguf_block_quantized_q8_amd", "_build", "sanitized")
REPORTS = ("AddressSanitizer", "runtime error:", "LeakSanitizer")


def _run_child(test_file, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    for word in REPORTS:
        assert word not in out, out[-3000:]
    assert " passed" in out


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc's {name} is not installed")
    return path


def test_oracle_pins_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = oracle_build.build_sanitized(os.path.join(OUT, "libggq_oracle_san.so"))
    pre = " ".join([_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")])
    _run_child(os.path.join("tests", "test_oracle_pins.py"), {"GGQO_LIB": lib, "LD_PRELOAD": pre})


def test_abi_validation_under_asan_ubsan():
    llvm = "/opt/rocm/llvm/lib/clang"
    rts = sorted(glob.glob(os.path.join(llvm, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    if any(not os.path.exists(os.path.join(ggq_build.BUILD, os.path.basename(s) + ".o"))
           for s in ggq_build.sources() if not s.endswith("api.hip")):
        ggq_build.build()
    os.makedirs(OUT, exist_ok=True)
    lib = ggq_build.build_host_sanitized(os.path.join(OUT, "libggq_san.so"))
    _run_child(os.path.join("tests", "test_boundary.py"), {"GGQ_LIB": lib, "LD_PRELOAD": rts[-1]})
