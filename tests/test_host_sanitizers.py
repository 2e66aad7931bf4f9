"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer builds (CPU only, no GPU).

* The C ABI's validation layer: every HIP source of the library is compiled with its host code
  instrumented (device code as usual, never run here) and linked into
  `tests/sanitize/abi_checks.cpp`, which drives every entry point through calls that must return
  before the library makes a HIP call: invalid arguments, overlapping or misaligned buffers, empty
  problems, undersized workspaces, and the workspace queries over every gate kind, order, width
  and size up to the documented limits (so that no byte count can overflow).
* The CPU oracle: `oracle/gdr_oracle.c` with `tests/sanitize/oracle_checks.c` (exactly sized heap
  buffers for every gate kind, both orders, ragged shapes and thread counts; its argument checks;
  two closed forms of the recurrence).

Each program exits non-zero on a failed expectation, and the sanitizers abort on the first memory
error or undefined behaviour."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_71_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# host-only instrumentation: each sanitizer flag applies to the host compilation of a HIP file
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError("%s failed (%d):\n%s\n%s" % (cmd[0], r.returncode, r.stdout[-4000:], r.stderr[-4000:]))
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_abi_validation_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = str(tmp_path / (f[:-4] + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", *HOST_SAN,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
              "-w", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_checks.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_checks")
    _run([CLANGXX, *SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV, timeout=120)
    assert "0 failure(s)" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), os.path.join(ROOT, "oracle", "gdr_oracle.c"),
          "-lm"])
    r = _run([exe], env=ENV, timeout=120)
    assert "0 failure(s)" in r.stdout, r.stdout
