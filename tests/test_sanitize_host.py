"""The C ABI library's host code (validation and the shard driver) built with
AddressSanitizer and UndefinedBehaviorSanitizer, host code only (no device code
is sanitized: the flags apply to the host pass only; the kernels are replaced by
stub launchers), and run over seeded random
problems by tests/sanitize/abi_host_check.cpp. No GPU is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_check"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "eagle_draft_amd", "csrc"),
           os.path.join(ROOT, "eagle_draft_amd", "csrc", "e3_abi.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe), "1500"], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
