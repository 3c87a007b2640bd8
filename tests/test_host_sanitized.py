"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every HIP source is built with the sanitizers on its host side
(device code as usual), linked, and the plain-C ABI program
(tests/c/abi_check.c, argument checks and workspace sizes; nothing is
launched) runs against it with both sanitizers set to stop at the first
report."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def test_abi_program_clean_under_host_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    srcs = sorted(glob.glob(os.path.join(ROOT, "routed_expert_ffn_gate_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        subprocess.run([HIPCC, *flags, *HOST_SAN, "-c", src, "-o", obj], check=True, capture_output=True,
                       text=True, timeout=900)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libmoelb_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN[:4], *objs, "-o", lib],
                   check=True, capture_output=True, text=True, timeout=300)
    exe = str(tmp_path / "abi_check_san")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
                    "-L", str(tmp_path), "-lmoelb_san", f"-Wl,-rpath,{tmp_path}", "-o", exe],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
