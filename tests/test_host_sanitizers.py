"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every library source is compiled with its host side instrumented (device code as
usual), linked with tests/sanitize/abi_rejects.c, and run: each entry point is called
with invalid arguments (NULL, misaligned or fake pointers, zero, negative and extreme
sizes, bad windows, scales, group counts and prologue parameters) and must reject the
call before anything is enqueued; the workspace-size queries also run at extreme sizes.
Nothing here reaches a GPU: no call passes its argument checks.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from causal_sliding_window_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_sliding_window_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"
# host-only sanitizer flags: each -fsanitize= goes to the host compilation alone
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _tools():
    hip = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang, clangxx = os.path.join(LLVM, "clang"), os.path.join(LLVM, "clang++")
    for t in (hip, clang, clangxx):
        if not os.path.exists(t):
            pytest.skip(f"{t} not available")
    return hip, clang, clangxx


def test_c_abi_rejects_bad_arguments_under_sanitizers(tmp_path):
    hip, clang, clangxx = _tools()
    flags = [f for f in build.HIPCC_FLAGS if not f.startswith("-Rpass")]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [hip] + flags + build.EXTRA_FLAGS.get(src, []) + HOST_SAN + [
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
            "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}: {r.stderr[-2000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    drv = str(tmp_path / "abi_rejects.o")
    r = subprocess.run([clang, "-O1", "-g"] + SAN + ["-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_rejects.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_rejects")
    r = subprocess.run([clangxx] + SAN + [drv] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                       "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
