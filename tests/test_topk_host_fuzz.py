"""The workgroup top-(k-1) of the selection kernels, built for the host with
each GPU lane as a host thread (tests/cpusim), fuzzed under AddressSanitizer
+ UBSan and under ThreadSanitizer: random, tied, equal, two-level and
near-equal logits, k in {4, 16, 64, 256, 512}, 256- and 512-thread
workgroups.  The sanitizers check the kernel's LDS accesses and its barrier
placement (a removed barrier shows as a ThreadSanitizer data race); the
driver checks the kept set against the exact top-(k-1) of the kernel's own
importances, ties to the lower position."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = shutil.which("clang++", path="/opt/rocm/llvm/bin") or shutil.which("clang++")
SRC = os.path.join(ROOT, "tests", "cpusim", "topk_fuzz.cpp")
INC = ["-I" + os.path.join(ROOT, "tests", "cpusim", "shim"), "-I" + os.path.join(ROOT, "include"),
       "-I" + os.path.join(ROOT, "long_context_kv_amd", "csrc")]


def _build(tmp_path, name, flags):
    if CLANG is None:
        pytest.skip("no host clang++")
    exe = str(tmp_path / name)
    r = subprocess.run([CLANG, "-std=c++20", "-O1", "-g", *flags, *INC, SRC, "-o", exe, "-pthread"],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "cannot find" in r.stderr and "clang_rt" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("name,flags,env", [
    ("asan_ubsan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
     {"ASAN_OPTIONS": "detect_leaks=0"}),
    ("tsan", ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1 exitcode=66"}),
])
def test_topk_host_fuzz_under_sanitizers(tmp_path, name, flags, env):
    exe = _build(tmp_path, "topk_" + name, flags)
    r = subprocess.run([exe, "30"], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, **env))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 failed" in r.stdout
