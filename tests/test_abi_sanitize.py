"""The C ABI's host code (argument checks, workspace and saved-state
carving, the VSA_VALIDATE path) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and run against launch stubs that touch exactly
the bytes each kernel would read or write (tests/host_abi/abi_sanitize.cpp).
CPU only: no GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "trainable_block_sparse_cube_amd", "csrc", "vsa_api.hip"),
       os.path.join(ROOT, "tests", "host_abi", "abi_sanitize.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    # the two macros that only the HIP compiler defines, for a host-only build
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(X)=X",
           "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "trainable_block_sparse_cube_amd", "csrc"),
           "-x", "c++", SRC[0], "-x", "c++", SRC[1], "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("VSA_VALIDATE", None)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300,
                       env=env)
    assert r.returncode == 0, r.stdout
    assert "host ABI checks passed" in r.stdout
