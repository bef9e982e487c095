"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Builds libmsa_kvouter's sources with the sanitizers on the host side only
(each -fsanitize flag after -Xarch_host, so the gfx950 device code is built
as usual) into a test executable with tests/abi_host_check.cpp, which drives
every entry point's validation and error paths, and runs it. On this
GPU-less host a well-formed call must also fail cleanly with MSA_ERR_HIP.
"""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_selection_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    from block_sparse_attention_selection_amd.build import FLAGS, SOURCES

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "abi_host_check.cpp")]
    exe = tmp_path / "abi_host_check"
    cmd = [HIPCC, *FLAGS, *SAN.split(), "-I", os.path.join(ROOT, "include"), *srcs, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    if torch.cuda.device_count() == 0:
        env["MSA_EXPECT_NO_DEVICE"] = "1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "abi host checks passed" in r.stdout
