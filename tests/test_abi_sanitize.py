"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled as usual for gfx950, with ASan and UBSan on
the host code only; no kernel is launched: tests/sanitize/abi_driver.cpp calls
every entry point with arguments the host validation must reject, and runs the
host-side computations (per-layer budgets, prefix matching, workspace sizes) on
random inputs.  Any sanitizer report fails the test.  The build is cached under
_build/ by the sources' hash."""
import glob
import hashlib
import os
import shutil
import subprocess
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_kv_quest_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"),
          "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_driver():
    h = hashlib.sha256()
    for f in sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [DRIVER, os.path.join(ROOT, "include",
                                                                                                  "se.h")]:
        h.update(open(f, "rb").read())
    out = os.path.join(ROOT, "_build", "asan", h.hexdigest()[:16])
    exe = os.path.join(out, "abi_driver")
    if os.path.exists(exe):
        return exe
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc is not available")
    os.makedirs(out, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        r = subprocess.run(["hipcc", *COMMON, *SAN, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{r.stderr[-3000:]}")
        return obj

    with cf.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, sources() + [DRIVER]))
    r = subprocess.run(["hipcc", *SAN, "-o", exe + ".tmp", *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking the driver failed:\n" + r.stderr[-3000:])
    os.replace(exe + ".tmp", exe)
    return exe


def test_abi_host_layer_under_asan_and_ubsan():
    exe = build_driver()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"driver failed (status {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
