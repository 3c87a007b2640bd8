"""The C ABI from a plain C program (tests/c/abi_check.c): compiled with gcc
against include/moelb.h, linked to the in-tree libmoelb.so, run on the CPU
(argument checks only, nothing is launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "routed_expert_ffn_gate_amd")


def test_plain_c_program_links_and_checks_arguments(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(PKG, "libmoelb.so")):
        pytest.fail("libmoelb.so is not built (run python -m routed_expert_ffn_gate_amd.build)")
    exe = str(tmp_path / "abi_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", PKG, "-lmoelb", f"-Wl,-rpath,{PKG}",
                    "-o", exe], check=True, capture_output=True, text=True, timeout=120)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
