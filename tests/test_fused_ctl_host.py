"""The fused decode's control protocol (recsa_fused_ctl.hpp: placement mark,
both barrier forms, the final arrival that elects the merging workgroup, its
status checks and the reset) built for the host, each emulated workgroup 64
host threads (tests/cpusim), and run under AddressSanitizer + UBSan and
under ThreadSanitizer through normal calls (two in a row on the same
control words, which must be left zero), members on two XCDs (one shared L2:
the placement check; two L2s: every wait runs out, no member merges), and a
straggler that arrives after the others' waits ran out, in both forms.  The
failure cases must end in NaN output and a nonzero error word, and a call
after the caller re-zeroes the control block must work."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = shutil.which("clang++", path="/opt/rocm/llvm/bin") or shutil.which("clang++")
SRC = os.path.join(ROOT, "tests", "cpusim", "fused_ctl_sim.cpp")
INC = ["-I" + os.path.join(ROOT, "tests", "cpusim", "shim"), "-I" + os.path.join(ROOT, "include"),
       "-I" + os.path.join(ROOT, "long_context_kv_amd", "csrc")]


@pytest.mark.parametrize("name,flags,env", [
    ("asan_ubsan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
     {"ASAN_OPTIONS": "detect_leaks=0"}),
    ("tsan", ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1 exitcode=66"}),
])
def test_fused_decode_control_protocol_on_host(tmp_path, name, flags, env):
    if CLANG is None:
        pytest.skip("no host clang++")
    exe = str(tmp_path / ("fused_ctl_" + name))
    r = subprocess.run([CLANG, "-std=c++20", "-O1", "-g", *flags, *INC, SRC, "-o", exe, "-pthread"],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "cannot find" in r.stderr and "clang_rt" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, **env))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 failed" in r.stdout
    assert r.stdout.count("\nok ") + r.stdout.startswith("ok ") >= 20, r.stdout
