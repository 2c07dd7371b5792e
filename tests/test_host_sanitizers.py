"""The C-ABI's host code (validation, argument marshalling, the RoPE rate table, keep_count and
the cache-reuse policy) built with AddressSanitizer and UndefinedBehaviorSanitizer and run on the
CPU against recording stubs of the kernel launchers (tests/host_abi_check.cpp). Host code only:
no device code is compiled with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_abi_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
           os.path.join(ROOT, "video_diffusion_transformer_qk_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host_abi_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert out.startswith("ok:"), out[-3000:]
