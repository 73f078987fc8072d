"""The host code of the library (plan builder, C-ABI argument checks) built
with AddressSanitizer and UndefinedBehaviorSanitizer, host side only, and run
on 3000 random layouts and the error paths (tests/host/plan_driver.cpp). No
GPU is needed: the plans are host-only and the launch calls fail with
ZDO_EHIP before any kernel."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_distributed_optimizer_amd", "csrc")


def test_plan_and_abi_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs on a host without a GPU (the plans must stay host-only)")
    exe = str(tmp_path / "plan_driver")
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host", "plan_driver.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "abi.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "ok: 3000 plans" in r.stdout
