"""The library's host code (argument checks, workspace sizing, status strings) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The C-ABI translation unit (moe_api.hip) is recompiled with the sanitizers on its host code only
(every `-fsanitize=` goes to the host pass through -Xarch_host; the GPU code is unchanged) and
linked, with the library's other objects, into tests/sanitize/abi_errors.cpp: a driver that calls
every entry point with arguments its host-side validation must refuse (fake pointers, never
dereferenced) and the sizing functions over normal, ragged, huge and degenerate shapes.  The run
must exit 0 with no sanitizer report.  No GPU is touched: every call returns before any launch.
"""

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_counting_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")


def _tool(name):
    for c in (os.path.join("/opt/rocm/bin", name), os.path.join("/opt/rocm/llvm/bin", name),
              shutil.which(name)):
        if c and os.path.exists(c):
            return c
    pytest.skip("%s not found" % name)


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def test_host_code_sanitizer_clean():
    from sparse_mixture_experts_counting_amd import build
    hipcc, clang = _tool("hipcc"), _tool("clang++")
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(build.BUILD_DIR, os.path.basename(s) + ".o")
            for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
            if os.path.basename(s) != "moe_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    api = os.path.join(OUT, "moe_api_san.o")
    flags = [f for f in build.HIPCC_FLAGS if not f.startswith("-O")]
    rc, out = _run([hipcc] + flags + [
        "-O1", "-g", "-fno-omit-frame-pointer",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined",
        "-c", os.path.join(CSRC, "moe_api.hip"), "-o", api])
    assert rc == 0, out
    drv = os.path.join(OUT, "abi_errors.o")
    rc, out = _run([clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I" + os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "tests", "sanitize", "abi_errors.cpp"), "-o", drv])
    assert rc == 0, out
    exe = os.path.join(OUT, "abi_errors")
    rc, out = _run([clang, "-fsanitize=address,undefined", drv, api] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ)
    # The HIP runtime's own start-up allocations are not this library's: leak checking is off,
    # every other report aborts the run.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert "abi_errors: 0 failures" in out, out
